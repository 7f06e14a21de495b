// fa_host.cpp -- the C ABI of libfa (declared in include/fa.h).
//
// Validates every argument on the host before touching HIP, picks the compiled
// kernel for (dtype, d, causal, tile shape) and enqueues it on the caller's
// stream.  Holds no state except a thread-local error message.
#include "fa.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <string>

#include "fa_kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg)
{
    g_last_error = msg;
    return code;
}

const fa::KernelEntry* find_kernel(int dtype, int d, int causal, int block_m, int block_n)
{
    const fa::KernelEntry* table = dtype == FA_DTYPE_BF16 ? fa::kBf16Kernels : fa::kF32Kernels;
    const int n = dtype == FA_DTYPE_BF16 ? fa::kNumBf16Kernels : fa::kNumF32Kernels;
    for (int i = 0; i < n; ++i) {
        const fa::KernelEntry& e = table[i];
        if (e.d != d || e.causal != causal) continue;
        if (block_m == 0 && block_n == 0) return &e;          // first listed is the default
        if (e.block_m == block_m && e.block_n == block_n) return &e;
    }
    return nullptr;
}

bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb)
{
    const uintptr_t x = reinterpret_cast<uintptr_t>(a);
    const uintptr_t y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

int run(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
        int N, int d, int causal, float scale, int dtype, void* stream, int block_m, int block_n)
{
    g_last_error.clear();
    if (dtype == FA_DTYPE_F16) return fail(FA_ERR_UNSUPPORTED, "fp16 inputs are not built");
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16)
        return fail(FA_ERR_INVALID_ARG, "unknown dtype " + std::to_string(dtype));
    if (B < 0 || N < 0) return fail(FA_ERR_INVALID_ARG, "B and N must be >= 0");
    if (Hq < 1 || Hkv < 1) return fail(FA_ERR_INVALID_ARG, "Hq and Hkv must be >= 1");
    if (Hq % Hkv != 0) return fail(FA_ERR_INVALID_ARG, "Hq must be a multiple of Hkv");
    if (d < 1) return fail(FA_ERR_INVALID_ARG, "d must be >= 1");
    if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite");
    const double folded = (double)scale * 1.4426950408889634;   // scale * log2(e)
    if (!std::isfinite((float)folded))
        return fail(FA_ERR_INVALID_ARG, "scale * log2(e) overflows float32");
    if ((block_m == 0) != (block_n == 0) || block_m < 0 || block_n < 0)
        return fail(FA_ERR_INVALID_ARG, "block_m and block_n must both be positive");
    if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "d must be 64 or 128");
    if (B == 0 || N == 0) return FA_OK;                         // empty output: nothing to do

    if (!q || !k || !v || !o || !lse) return fail(FA_ERR_INVALID_ARG, "null pointer");
    const void* ptrs[5] = {q, k, v, o, lse};
    for (const void* ptr : ptrs)
        if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0)
            return fail(FA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");

    const uint64_t esize = dtype == FA_DTYPE_F32 ? 4 : 2;
    const uint64_t qrows = (uint64_t)B * (uint64_t)Hq * (uint64_t)N;
    const uint64_t kvrows = (uint64_t)B * (uint64_t)Hkv * (uint64_t)N;
    const uint64_t qbytes = qrows * (uint64_t)d * esize;
    const uint64_t kvbytes = kvrows * (uint64_t)d * esize;
    const uint64_t lbytes = qrows * 4;
    if (qbytes >> 62 || kvbytes >> 62) return fail(FA_ERR_INVALID_ARG, "problem too large");
    if (overlaps(o, qbytes, q, qbytes) || overlaps(o, qbytes, k, kvbytes) ||
        overlaps(o, qbytes, v, kvbytes) || overlaps(lse, lbytes, q, qbytes) ||
        overlaps(lse, lbytes, k, kvbytes) || overlaps(lse, lbytes, v, kvbytes) ||
        overlaps(o, qbytes, lse, lbytes))
        return fail(FA_ERR_INVALID_ARG, "o and lse must not overlap the inputs or each other");

    const fa::KernelEntry* e = find_kernel(dtype, d, causal, block_m, block_n);
    if (!e) {
        char buf[96];
        std::snprintf(buf, sizeof buf, "tile %dx%d not built for this dtype and d", block_m, block_n);
        return fail(FA_ERR_UNSUPPORTED, buf);
    }
    const uint64_t ntiles = ((uint64_t)N + e->block_m - 1) / e->block_m;
    const uint64_t grid = (uint64_t)B * (uint64_t)Hq * ntiles;
    if (grid > 0x7fffffffULL) return fail(FA_ERR_UNSUPPORTED, "grid exceeds 2^31 - 1 workgroups");

    fa::FwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.N = N;
    p.group = Hq / Hkv;
    p.n_qtiles = (int)ntiles;
    p.scale_log2 = (float)folded;
    p.xcd_map = 0;
    const hipError_t err = e->launch(p, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(FA_ERR_HIP, std::string("launch failed: ") + hipGetErrorString(err));
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
           int N, int d, int causal, float scale, int dtype, void* stream)
{
    return run(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dtype, stream, 0, 0);
}

int fa_fwd_tiled(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                 int Hkv, int N, int d, int causal, float scale, int dtype, void* stream, int block_m,
                 int block_n)
{
    if (block_m <= 0 || block_n <= 0) {
        g_last_error = "block_m and block_n must both be positive";
        return FA_ERR_INVALID_ARG;
    }
    return run(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dtype, stream, block_m, block_n);
}

int fa_tile_shapes(int dtype, int d, int* block_m, int* block_n, int cap)
{
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return -1;
    if (d != 64 && d != 128) return -1;
    const fa::KernelEntry* table = dtype == FA_DTYPE_BF16 ? fa::kBf16Kernels : fa::kF32Kernels;
    const int n = dtype == FA_DTYPE_BF16 ? fa::kNumBf16Kernels : fa::kNumF32Kernels;
    int count = 0;
    for (int i = 0; i < n; ++i) {
        if (table[i].d != d || table[i].causal != 0) continue;
        if (count < cap && block_m && block_n) {
            block_m[count] = table[i].block_m;
            block_n[count] = table[i].block_n;
        }
        ++count;
    }
    return count;
}

const char* fa_error_string(int code)
{
    switch (code) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported request";
    case FA_ERR_HIP: return "HIP runtime error";
    default: return "unknown error code";
    }
}

const char* fa_last_error(void)
{
    return g_last_error.c_str();
}

int fa_abi_version(void)
{
    return 1;
}

}  // extern "C"
