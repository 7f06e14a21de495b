// fa_host.cpp -- the C ABI of libfa (declared in include/fa.h).
//
// Validates every argument on the host before touching HIP, picks the compiled
// kernel for (dtype, d, causal, tile shape) and enqueues it on the caller's
// stream.  Holds no state except a thread-local error message.
#include "fa.h"

#include <algorithm>
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <initializer_list>
#include <string>

#include "fa_kernels.h"

namespace {

thread_local std::string g_last_error;

constexpr int kMaxSplits = 1024;
constexpr int kMaxBwdSplits = 8;
constexpr uint64_t kTileSlack = 128;   // rows a kernel may address past N in its last tile
constexpr int kMaxSoftmaxCols = 0x7fffffff - 4095;   // 2^31 - 4096
// A launch's work-item count (workgroups x threads) is a 32-bit quantity, and every kernel here
// runs at most 256 threads per workgroup: at most this many workgroups per launch.
constexpr uint64_t kMaxWorkgroups = 0xffffffffULL / 256;   // 2^24 - 1
// The row softmax runs one workgroup per row and launches longer lists in pieces of this many rows.
constexpr long long kSoftmaxRowsPerLaunch = 1LL << 23;
// The merge runs four rows per workgroup in a single launch.
constexpr uint64_t kMaxMergeRows = 4 * kMaxWorkgroups;

int fail(int code, const std::string& msg)
{
    g_last_error = msg;
    return code;
}

bool known_dtype(int dtype)
{
    return dtype == FA_DTYPE_F32 || dtype == FA_DTYPE_BF16 || dtype == FA_DTYPE_F16;
}

// The square-forward kernels compiled for a dtype (n = 0 for an unknown one).
const fa::KernelEntry* table_for(int dtype, int* n)
{
    switch (dtype) {
    case FA_DTYPE_F32: *n = fa::kNumF32Kernels; return fa::kF32Kernels;
    case FA_DTYPE_BF16: *n = fa::kNumBf16Kernels; return fa::kBf16Kernels;
    case FA_DTYPE_F16: *n = fa::kNumF16Kernels; return fa::kF16Kernels;
    default: *n = 0; return nullptr;
    }
}

}  // namespace

namespace fa {
int device_cus()
{
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cache[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev] = n;
    }
    return cache[dev];
}
}  // namespace fa

namespace {

// units: B * Hq (query heads of the batch), N: query rows per head; they size the grid when the
// default tile depends on it.
const fa::KernelEntry* find_kernel(int dtype, int d, int causal, int block_m, int block_n, long long units = 0,
                                   long long N = 0)
{
    // 16-bit inputs: the 64-rows-per-wave kernels serve the 256 x 64 and 128 x 64 tiles
    bool w64 = dtype == FA_DTYPE_BF16 || dtype == FA_DTYPE_F16;
    if (w64 && block_m == 0 && block_n == 0) {
        // by default, only when its 64-row waves cover every SIMD (one wave per SIMD each);
        // fewer rows go to the 32-rows-per-wave kernel of the table below, which runs twice the
        // waves, two per SIMD
        const int cus = fa::device_cus();
        const uint64_t simds = 4 * (uint64_t)(cus > 0 ? cus : 256);
        if ((uint64_t)units * (((uint64_t)N + 63) / 64) < simds) {
            w64 = false;
        } else {
            // 256-row workgroups when the grid gives every CU at least two of them, else
            // 128-row ones (twice the workgroups)
            const uint64_t wg256 = (uint64_t)units * (((uint64_t)N + 255) / 256);
            block_m = wg256 >= 2 * 256 ? 256 : 128;
            block_n = 64;
        }
    }
    if (w64) {
        const fa::KernelEntry* w = dtype == FA_DTYPE_BF16 ? fa::kBf16W64Kernels : fa::kF16W64Kernels;
        for (int i = 0; i < fa::kNumW64Kernels; ++i)
            if (w[i].d == d && w[i].causal == causal && w[i].block_m == block_m && w[i].block_n == block_n)
                return &w[i];
    }
    int n = 0;
    const fa::KernelEntry* table = table_for(dtype, &n);
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

// Checks shared by the attention entry points: head counts, head dimension, mask flag
// and scale (which must stay finite once folded with log2(e)).  FA_OK or the error.
int check_attention_args(int Hq, int Hkv, int d, int causal, float scale)
{
    if (Hq < 1 || Hkv < 1) return fail(FA_ERR_INVALID_ARG, "Hq and Hkv must be >= 1");
    if (Hq % Hkv != 0) return fail(FA_ERR_INVALID_ARG, "Hq must be a multiple of Hkv");
    if (d < 1) return fail(FA_ERR_INVALID_ARG, "d must be >= 1");
    if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite");
    if (!std::isfinite((float)((double)scale * 1.4426950408889634)))
        return fail(FA_ERR_INVALID_ARG, "scale * log2(e) overflows float32");
    return FA_OK;
}

// Every pointer non-null and 16-byte aligned.  FA_OK or the error.
int check_pointers(std::initializer_list<const void*> ptrs)
{
    for (const void* ptr : ptrs)
        if (!ptr) return fail(FA_ERR_INVALID_ARG, "null pointer");
    for (const void* ptr : ptrs)
        if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0)
            return fail(FA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
    return FA_OK;
}

int run(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
        int N, int d, int causal, float scale, int dtype, void* stream, int block_m, int block_n,
        unsigned long long* stamps = nullptr, long long stamp_slots = 0)
{
    g_last_error.clear();
    if (!known_dtype(dtype)) return fail(FA_ERR_INVALID_ARG, "unknown dtype " + std::to_string(dtype));
    if (B < 0 || N < 0) return fail(FA_ERR_INVALID_ARG, "B and N must be >= 0");
    if (const int rc = check_attention_args(Hq, Hkv, d, causal, scale)) return rc;
    if ((block_m == 0) != (block_n == 0) || block_m < 0 || block_n < 0)
        return fail(FA_ERR_INVALID_ARG, "block_m and block_n must both be positive");
    if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "d must be 64 or 128");
    if (B == 0 || N == 0) return FA_OK;                         // empty output: nothing to do
    if (const int rc = check_pointers({q, k, v, o, lse})) return rc;

    const uint64_t esize = dtype == FA_DTYPE_F32 ? 4 : 2;
    const uint64_t qrows = (uint64_t)B * (uint64_t)Hq * (uint64_t)N;
    const uint64_t kvrows = (uint64_t)B * (uint64_t)Hkv * (uint64_t)N;
    const uint64_t qbytes = qrows * (uint64_t)d * esize;
    const uint64_t kvbytes = kvrows * (uint64_t)d * esize;
    const uint64_t lbytes = qrows * 4;
    if (qbytes >> 62 || kvbytes >> 62) return fail(FA_ERR_INVALID_ARG, "problem too large");
    // K/V tiles are read through buffer descriptors whose range and offsets are 32-bit;
    // the offsets of the last tile's rows past N must stay below 2^31 as well
    if (((uint64_t)N + kTileSlack) * (uint64_t)d * esize > 0x7fffffffULL)
        return fail(FA_ERR_UNSUPPORTED, "one head of K or V exceeds 2 GiB");
    if (overlaps(o, qbytes, q, qbytes) || overlaps(o, qbytes, k, kvbytes) ||
        overlaps(o, qbytes, v, kvbytes) || overlaps(lse, lbytes, q, qbytes) ||
        overlaps(lse, lbytes, k, kvbytes) || overlaps(lse, lbytes, v, kvbytes) ||
        overlaps(o, qbytes, lse, lbytes))
        return fail(FA_ERR_INVALID_ARG, "o and lse must not overlap the inputs or each other");

    const fa::KernelEntry* e = find_kernel(dtype, d, causal, block_m, block_n, (long long)B * Hq, N);
    if (!e) {
        char buf[96];
        std::snprintf(buf, sizeof buf, "tile %dx%d not built for this dtype and d", block_m, block_n);
        return fail(FA_ERR_UNSUPPORTED, buf);
    }
    const uint64_t ntiles = ((uint64_t)N + e->block_m - 1) / e->block_m;
    uint64_t grid = (uint64_t)B * (uint64_t)Hq * ntiles;
    if (grid > kMaxWorkgroups) return fail(FA_ERR_UNSUPPORTED, "grid exceeds 2^24 - 1 workgroups");
    if (e->blocks) {
        const long long walk = e->blocks((long long)B * Hq, (long long)ntiles, causal);
        if (walk > 0) grid = (uint64_t)walk;
    }
    if (stamps) {
        const uint64_t slots = grid * (uint64_t)(e->waves ? e->waves : e->block_m / 32);   // one per wave
        if (stamp_slots < 0 || (uint64_t)stamp_slots < slots)
            return fail(FA_ERR_INVALID_ARG, "stamps holds fewer slots than the launch has waves");
        if (overlaps(stamps, slots * 32, q, qbytes) || overlaps(stamps, slots * 32, k, kvbytes) ||
            overlaps(stamps, slots * 32, v, kvbytes) || overlaps(stamps, slots * 32, o, qbytes) ||
            overlaps(stamps, slots * 32, lse, lbytes))
            return fail(FA_ERR_INVALID_ARG, "stamps must not overlap the inputs or outputs");
    }

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
    p.Nk = N;
    p.q_off = 0;
    p.chunk = N;
    p.splits = 1;
    p.group = Hq / Hkv;
    p.n_qtiles = (int)ntiles;
    p.scale_log2 = (float)((double)scale * 1.4426950408889634);   // scale * log2(e)
    p.xcd_map = 0;
    p.walk = 0;
    p.stamps = stamps;
    const hipError_t err = e->launch(p, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(FA_ERR_HIP, std::string("launch failed: ") + hipGetErrorString(err));
    return FA_OK;
}

// Keys per split: ceil(Nk / splits) rounded up to the 64-key tile.
int split_chunk(int Nk, int splits)
{
    const int64_t per = ((int64_t)Nk + splits - 1) / splits;
    return (int)((per + 63) / 64 * 64);
}

int run_splitkv(const void* q, const void* k, const void* v, float* o_part, float* lse_part, int B,
                int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale, int dtype,
                int num_splits, void* stream)
{
    g_last_error.clear();
    if (!known_dtype(dtype)) return fail(FA_ERR_INVALID_ARG, "unknown dtype " + std::to_string(dtype));
    if (dtype == FA_DTYPE_F32) return fail(FA_ERR_UNSUPPORTED, "split-KV is built for 16-bit inputs only");
    if (B < 0 || Nq < 0 || Nk < 0) return fail(FA_ERR_INVALID_ARG, "B, Nq and Nk must be >= 0");
    if (const int rc = check_attention_args(Hq, Hkv, d, causal, scale)) return rc;
    if (num_splits < 1 || num_splits > kMaxSplits)
        return fail(FA_ERR_INVALID_ARG, "num_splits must be in 1.." + std::to_string(kMaxSplits));
    if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "d must be 64 or 128");
    if (B == 0 || Nq == 0) return FA_OK;                        // no query row: nothing to do
    if (Nk == 0) return fail(FA_ERR_INVALID_ARG, "Nk must be >= 1 when there are query rows");
    if (causal && Nq > Nk)
        return fail(FA_ERR_INVALID_ARG, "causal needs Nq <= Nk (the queries are the last Nq positions)");

    if (const int rc = check_pointers({q, k, v, o_part, lse_part})) return rc;
    const uint64_t qrows = (uint64_t)B * (uint64_t)Hq * (uint64_t)Nq;
    const uint64_t qbytes = qrows * (uint64_t)d * 2;
    const uint64_t kvbytes = (uint64_t)B * (uint64_t)Hkv * (uint64_t)Nk * (uint64_t)d * 2;
    const uint64_t obytes = (uint64_t)num_splits * qrows * (uint64_t)d * 4;
    const uint64_t lbytes = (uint64_t)num_splits * qrows * 4;
    if (qbytes >> 62 || kvbytes >> 62 || obytes >> 62) return fail(FA_ERR_INVALID_ARG, "problem too large");
    if (((uint64_t)Nk + kTileSlack) * (uint64_t)d * 2 > 0x7fffffffULL)
        return fail(FA_ERR_UNSUPPORTED, "one head of K or V exceeds 2 GiB");
    if (overlaps(o_part, obytes, q, qbytes) || overlaps(o_part, obytes, k, kvbytes) ||
        overlaps(o_part, obytes, v, kvbytes) || overlaps(lse_part, lbytes, q, qbytes) ||
        overlaps(lse_part, lbytes, k, kvbytes) || overlaps(lse_part, lbytes, v, kvbytes) ||
        overlaps(o_part, obytes, lse_part, lbytes))
        return fail(FA_ERR_INVALID_ARG, "o_part and lse_part must not overlap the inputs or each other");

    const fa::KernelEntry* split_table = dtype == FA_DTYPE_BF16 ? fa::kBf16SplitKernels : fa::kF16SplitKernels;
    const int split_n = dtype == FA_DTYPE_BF16 ? fa::kNumBf16SplitKernels : fa::kNumF16SplitKernels;
    const fa::KernelEntry* e = nullptr;
    for (int i = 0; i < split_n && !e; ++i)
        if (split_table[i].d == d && split_table[i].causal == causal) e = &split_table[i];
    if (!e) return fail(FA_ERR_UNSUPPORTED, "no split-KV kernel for this d");
    // the G query heads of a K/V head share its workgroups: G*Nq packed rows per K/V head,
    // indexed in 32 bits by the kernel (its last tile may reach block_m rows past them)
    const uint64_t packed = (uint64_t)(Hq / Hkv) * (uint64_t)Nq;
    if (packed + (uint64_t)e->block_m > 0x7fffffffULL)
        return fail(FA_ERR_UNSUPPORTED, "more than 2^31 - 129 query rows per K/V head (G * Nq)");
    const uint64_t ntiles = (packed + e->block_m - 1) / e->block_m;
    const uint64_t grid = (uint64_t)num_splits * (uint64_t)B * (uint64_t)Hkv * ntiles;
    if (grid > kMaxWorkgroups) return fail(FA_ERR_UNSUPPORTED, "grid exceeds 2^24 - 1 workgroups");

    fa::FwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o_part;
    p.lse = lse_part;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.N = Nq;
    p.Nk = Nk;
    p.q_off = Nk - Nq;
    p.chunk = split_chunk(Nk, num_splits);
    p.splits = num_splits;
    p.group = Hq / Hkv;
    p.n_qtiles = (int)ntiles;
    p.scale_log2 = (float)((double)scale * 1.4426950408889634);   // scale * log2(e)
    p.xcd_map = 0;
    p.walk = 0;
    p.stamps = nullptr;
    const hipError_t err = e->launch(p, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(FA_ERR_HIP, std::string("launch failed: ") + hipGetErrorString(err));
    return FA_OK;
}

int run_merge(const float* o_part, const float* lse_part, void* o, float* lse, int num_splits, int B,
              int H, int N, int d, int dtype, void* stream)
{
    g_last_error.clear();
    if (!known_dtype(dtype)) return fail(FA_ERR_INVALID_ARG, "unknown dtype " + std::to_string(dtype));
    if (B < 0 || N < 0) return fail(FA_ERR_INVALID_ARG, "B and N must be >= 0");
    if (H < 1) return fail(FA_ERR_INVALID_ARG, "H must be >= 1");
    if (d < 1) return fail(FA_ERR_INVALID_ARG, "d must be >= 1");
    if (num_splits < 1 || num_splits > kMaxSplits)
        return fail(FA_ERR_INVALID_ARG, "num_splits must be in 1.." + std::to_string(kMaxSplits));
    if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "d must be 64 or 128");
    if (B == 0 || N == 0) return FA_OK;
    if (const int rc = check_pointers({o_part, lse_part, o, lse})) return rc;
    const uint64_t rows = (uint64_t)B * (uint64_t)H * (uint64_t)N;
    const uint64_t pbytes = (uint64_t)num_splits * rows * (uint64_t)d * 4;
    const uint64_t plbytes = (uint64_t)num_splits * rows * 4;
    const uint64_t obytes = rows * (uint64_t)d * (dtype == FA_DTYPE_F32 ? 4 : 2);
    const uint64_t lbytes = rows * 4;
    if (pbytes >> 62) return fail(FA_ERR_INVALID_ARG, "problem too large");
    if (overlaps(o, obytes, o_part, pbytes) || overlaps(o, obytes, lse_part, plbytes) ||
        overlaps(lse, lbytes, o_part, pbytes) || overlaps(lse, lbytes, lse_part, plbytes) ||
        overlaps(o, obytes, lse, lbytes))
        return fail(FA_ERR_INVALID_ARG, "o and lse must not overlap the partial states or each other");
    if (rows > kMaxMergeRows)
        return fail(FA_ERR_UNSUPPORTED, "more than " + std::to_string(kMaxMergeRows) + " rows (B * H * N) in one merge");

    fa::MergeParams p;
    p.o_part = o_part;
    p.lse_part = lse_part;
    p.o = o;
    p.lse = lse;
    p.rows = (long long)rows;
    p.splits = num_splits;
    const hipError_t err = fa::launch_merge(p, d, dtype, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(FA_ERR_HIP, std::string("launch failed: ") + hipGetErrorString(err));
    return FA_OK;
}

int run_softmax(const void* x, void* y, float* lse, long long rows, int cols, int dtype, int algo, void* stream)
{
    g_last_error.clear();
    if (!known_dtype(dtype)) return fail(FA_ERR_INVALID_ARG, "unknown dtype " + std::to_string(dtype));
    if (algo != FA_SOFTMAX_ONLINE && algo != FA_SOFTMAX_SAFE)
        return fail(FA_ERR_INVALID_ARG, "algo must be FA_SOFTMAX_ONLINE or FA_SOFTMAX_SAFE");
    if (rows < 0 || cols < 0) return fail(FA_ERR_INVALID_ARG, "rows and cols must be >= 0");
    if (rows == 0) return FA_OK;
    if (cols == 0) return fail(FA_ERR_INVALID_ARG, "a row needs at least one entry (cols >= 1)");
    if (rows > 0x7fffffffLL) return fail(FA_ERR_UNSUPPORTED, "more than 2^31 - 1 rows");
    // the kernels step 32-bit column indices 1024 vectors at a time; this keeps every step below 2^31
    if (cols > kMaxSoftmaxCols) return fail(FA_ERR_UNSUPPORTED, "more than 2^31 - 4096 columns");
    if (!x || !y) return fail(FA_ERR_INVALID_ARG, "null pointer");
    if (reinterpret_cast<uintptr_t>(x) % 16 != 0 || reinterpret_cast<uintptr_t>(y) % 16 != 0 ||
        (lse && reinterpret_cast<uintptr_t>(lse) % 16 != 0))
        return fail(FA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
    const uint64_t bytes = (uint64_t)rows * (uint64_t)cols * (dtype == FA_DTYPE_F32 ? 4 : 2);
    if (bytes >> 62) return fail(FA_ERR_INVALID_ARG, "problem too large");
    if (x != y && overlaps(x, bytes, y, bytes))
        return fail(FA_ERR_INVALID_ARG, "y must be x itself or not overlap it");
    if (lse && (overlaps(lse, (uint64_t)rows * 4, x, bytes) || overlaps(lse, (uint64_t)rows * 4, y, bytes)))
        return fail(FA_ERR_INVALID_ARG, "lse must not overlap x or y");
    // One workgroup per row, so a long list of rows goes out in launches of at most
    // kSoftmaxRowsPerLaunch rows (2^23: each piece starts 16-byte aligned like x itself).
    const uint64_t row_bytes = (uint64_t)cols * (dtype == FA_DTYPE_F32 ? 4 : 2);
    fa::SoftmaxParams p;
    p.cols = cols;
    p.dtype = dtype;
    p.online = algo == FA_SOFTMAX_ONLINE;
    for (long long r0 = 0; r0 < rows; r0 += kSoftmaxRowsPerLaunch) {
        p.x = static_cast<const char*>(x) + (uint64_t)r0 * row_bytes;
        p.y = static_cast<char*>(y) + (uint64_t)r0 * row_bytes;
        p.lse = lse ? lse + r0 : nullptr;
        p.rows = std::min(rows - r0, kSoftmaxRowsPerLaunch);
        const hipError_t err = fa::launch_softmax(p, static_cast<hipStream_t>(stream));
        if (err != hipSuccess) return fail(FA_ERR_HIP, std::string("launch failed: ") + hipGetErrorString(err));
    }
    return FA_OK;
}

// static_scratch: the dK/dV partials go to the library's static workspace (fa::bwd_scratch)
// instead of dkv_part, which must then be null.
int run_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
            void* dq, void* dk, void* dv, float* delta, float* dkv_part, int num_splits, int B, int Hq, int Hkv,
            int N, int d, int causal, float scale, int dtype, void* stream, bool static_scratch = false)
{
    g_last_error.clear();
    if (!known_dtype(dtype)) return fail(FA_ERR_INVALID_ARG, "unknown dtype " + std::to_string(dtype));
    if (dtype == FA_DTYPE_F32) return fail(FA_ERR_UNSUPPORTED, "the backward is built for 16-bit inputs only");
    if (B < 0 || N < 0) return fail(FA_ERR_INVALID_ARG, "B and N must be >= 0");
    if (const int rc = check_attention_args(Hq, Hkv, d, causal, scale)) return rc;
    if (num_splits < 1 || num_splits > kMaxBwdSplits)
        return fail(FA_ERR_INVALID_ARG, "num_splits must be in 1.." + std::to_string(kMaxBwdSplits));
    if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "d must be 64 or 128");
    if (B == 0 || N == 0) return FA_OK;
    if (num_splits > 1 && !dkv_part && !static_scratch)
        return fail(FA_ERR_INVALID_ARG, "dkv_part is required when num_splits > 1");
    if (num_splits > 1 && reinterpret_cast<uintptr_t>(dkv_part) % 16 != 0)
        return fail(FA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");

    if (const int rc = check_pointers({q, k, v, o, lse, dout, dq, dk, dv, delta})) return rc;
    const uint64_t qrows = (uint64_t)B * (uint64_t)Hq * (uint64_t)N;
    const uint64_t qbytes = qrows * (uint64_t)d * 2;
    const uint64_t kvbytes = (uint64_t)B * (uint64_t)Hkv * (uint64_t)N * (uint64_t)d * 2;
    const uint64_t lbytes = qrows * 4;
    if (qbytes >> 62 || kvbytes >> 62) return fail(FA_ERR_INVALID_ARG, "problem too large");
    if (((uint64_t)N + kTileSlack) * (uint64_t)d * 2 > 0x7fffffffULL)
        return fail(FA_ERR_UNSUPPORTED, "one head of a tensor exceeds 2 GiB");
    const uint64_t kvelems = kvbytes / 2;
    const uint64_t pbytes = num_splits > 1 ? 2ULL * num_splits * kvelems * 4 : 0;   // fp32 partials
    if (pbytes >> 62) return fail(FA_ERR_INVALID_ARG, "problem too large");
    const void* in[6] = {q, k, v, o, lse, dout};
    const uint64_t in_n[6] = {qbytes, kvbytes, kvbytes, qbytes, lbytes, qbytes};
    void* out[5] = {dq, dk, dv, delta, dkv_part};
    const uint64_t out_n[5] = {qbytes, kvbytes, kvbytes, lbytes, pbytes};
    const int nout = num_splits > 1 && !static_scratch ? 5 : 4;
    for (int a = 0; a < nout; ++a) {
        for (int i = 0; i < 6; ++i)
            if (overlaps(out[a], out_n[a], in[i], in_n[i]))
                return fail(FA_ERR_INVALID_ARG, "dq, dk, dv, delta and dkv_part must not overlap the inputs or each other");
        for (int b = a + 1; b < nout; ++b)
            if (overlaps(out[a], out_n[a], out[b], out_n[b]))
                return fail(FA_ERR_INVALID_ARG, "dq, dk, dv, delta and dkv_part must not overlap the inputs or each other");
    }
    // one workgroup per 128 query rows (dq), per 128 keys and split (dk, dv), per 8 elements (reduce)
    const uint64_t tiles = ((uint64_t)N + 127) / 128;
    if ((uint64_t)B * (uint64_t)Hq * tiles > kMaxWorkgroups ||
        (uint64_t)B * (uint64_t)Hkv * tiles * (uint64_t)num_splits > kMaxWorkgroups ||
        (2 * kvelems / 8 + 255) / 256 > kMaxWorkgroups)
        return fail(FA_ERR_UNSUPPORTED, "grid exceeds 2^24 - 1 workgroups");

    fa::BwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.dout = dout;
    p.lse = lse;
    p.delta = delta;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.N = N;
    p.group = Hq / Hkv;
    p.scale = scale;
    p.xcd_map = 0;
    p.splits = num_splits;
    p.dkv_part = num_splits > 1 ? dkv_part : nullptr;
    if (static_scratch && num_splits > 1) {
        if (pbytes > fa::kBwdScratchBytes)
            return fail(FA_ERR_UNSUPPORTED, "the dK/dV partials (" + std::to_string(pbytes) +
                                                " bytes) exceed the static workspace of " +
                                                std::to_string(fa::kBwdScratchBytes) + " bytes");
        const hipError_t serr = fa::bwd_scratch(static_cast<hipStream_t>(stream), &p.dkv_part);
        if (serr != hipSuccess)
            return fail(FA_ERR_HIP, std::string("static workspace: ") + hipGetErrorString(serr));
    }
    const hipError_t err = fa::launch_bwd(p, d, dtype, causal, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(FA_ERR_HIP, std::string("launch failed: ") + hipGetErrorString(err));
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_softmax(const void* x, void* y, float* lse, long long rows, int cols, int dtype, int algo, void* stream)
{
    return run_softmax(x, y, lse, rows, cols, dtype, algo, stream);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
           void* dq, void* dk, void* dv, float* delta, int B, int Hq, int Hkv, int N, int d, int causal,
           float scale, int dtype, void* stream)
{
    return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, nullptr, 1, B, Hq, Hkv, N, d, causal, scale, dtype,
                   stream);
}

int fa_bwd_split(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                 void* dq, void* dk, void* dv, float* delta, float* dkv_part, int num_splits, int B, int Hq,
                 int Hkv, int N, int d, int causal, float scale, int dtype, void* stream)
{
    return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, dkv_part, num_splits, B, Hq, Hkv, N, d, causal, scale,
                   dtype, stream);
}

int fa_bwd_split_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, float* delta, int num_splits, int B,
                         int Hq, int Hkv, int N, int d, int causal, float scale, int dtype, void* stream)
{
    return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, nullptr, num_splits, B, Hq, Hkv, N, d, causal, scale,
                   dtype, stream, true);
}

long long fa_bwd_noalloc_max_bytes(void)
{
    return (long long)fa::kBwdScratchBytes;
}

int fa_bwd_num_splits(int B, int Hq, int Hkv, int N)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || N < 1) return -1;
    // About 1024 dK/dV workgroups (two rounds of the chip's 512 slots) let the longest
    // key tiles of a causal problem start first and the short ones fill in behind them.
    const int64_t base = (int64_t)B * Hkv * (((int64_t)N + 127) / 128);
    int64_t s = (1024 + base - 1) / base;
    if (s > kMaxBwdSplits) s = kMaxBwdSplits;
    return (int)s;
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
           int N, int d, int causal, float scale, int dtype, void* stream)
{
    return run(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dtype, stream, 0, 0);
}

int fa_fwd_stamped(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                   int N, int d, int causal, float scale, int dtype, void* stream, unsigned long long* stamps,
                   long long stamp_slots)
{
    g_last_error.clear();
    if (dtype == FA_DTYPE_F32) {
        g_last_error = "clock stamps are built into the 16-bit kernels only";
        return FA_ERR_UNSUPPORTED;
    }
    if (!stamps || reinterpret_cast<uintptr_t>(stamps) % 32 != 0) {
        g_last_error = "stamps must be a non-null, 32-byte aligned device pointer";
        return FA_ERR_INVALID_ARG;
    }
    return run(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dtype, stream, 0, 0, stamps, stamp_slots);
}

long long fa_fwd_stamp_slots(int B, int Hq, int N, int d, int dtype)
{
    if (B < 0 || Hq < 1 || N < 0 || (d != 64 && d != 128)) return -1;
    if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return -1;
    const fa::KernelEntry* e = find_kernel(dtype, d, 0, 0, 0, (long long)B * Hq, N);
    if (!e) return -1;
    const long long ntiles = ((long long)N + e->block_m - 1) / e->block_m;
    long long grid = (long long)B * Hq * ntiles;
    if (e->blocks) {
        // the walk may differ with the mask: room for the larger launch
        long long most = 0;
        for (int causal = 0; causal < 2; ++causal) {
            const long long walk = e->blocks((long long)B * Hq, ntiles, causal);
            most = std::max(most, walk > 0 ? walk : grid);
        }
        grid = most;
    }
    return grid * (e->waves ? e->waves : e->block_m / 32);
}

int fa_wall_clock_khz(int device)
{
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, device) != hipSuccess) return -1;
    return khz;
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

int fa_fwd_splitkv(const void* q, const void* k, const void* v, float* o_part, float* lse_part, int B,
                   int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale, int dtype,
                   int num_splits, void* stream)
{
    return run_splitkv(q, k, v, o_part, lse_part, B, Hq, Hkv, Nq, Nk, d, causal, scale, dtype, num_splits,
                       stream);
}

int fa_merge(const float* o_part, const float* lse_part, void* o, float* lse, int num_splits, int B, int H,
             int N, int d, int dtype, void* stream)
{
    return run_merge(o_part, lse_part, o, lse, num_splits, B, H, N, d, dtype, stream);
}

int fa_split_chunk(int Nk, int num_splits)
{
    if (Nk < 0 || num_splits < 1 || num_splits > kMaxSplits) return -1;
    return split_chunk(Nk, num_splits);
}

int fa_splitkv_num_splits(int B, int Hq, int Hkv, int Nq, int Nk)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Nq < 1 || Nk < 1) return -1;
    // Enough workgroups to fill the chip twice over (256 CUs, two workgroups each),
    // but at least four 64-key tiles per split.  A workgroup holds 128 rows of the
    // G = Hq/Hkv query heads that share one K/V head.
    const int64_t base = (int64_t)B * Hkv * (((int64_t)(Hq / Hkv) * Nq + 127) / 128);
    int64_t s = (1024 + base - 1) / base;
    const int64_t cap = ((int64_t)Nk + 255) / 256;
    if (s > cap) s = cap;
    if (s > kMaxSplits) s = kMaxSplits;
    return s < 1 ? 1 : (int)s;
}

int fa_tile_shapes(int dtype, int d, int* block_m, int* block_n, int cap)
{
    if (!known_dtype(dtype)) return -1;
    if (d != 64 && d != 128) return -1;
    // every distinct (block_m, block_n) that find_kernel can reach, in the order it prefers them
    int pairs[16][2];
    int count = 0;
    auto add = [&](const fa::KernelEntry* t, int n) {
        for (int i = 0; i < n; ++i) {
            if (t[i].d != d || t[i].causal != 0) continue;
            bool seen = false;
            for (int j = 0; j < count; ++j) seen = seen || (pairs[j][0] == t[i].block_m && pairs[j][1] == t[i].block_n);
            if (seen || count == 16) continue;
            pairs[count][0] = t[i].block_m;
            pairs[count][1] = t[i].block_n;
            ++count;
        }
    };
    if (dtype == FA_DTYPE_BF16 || dtype == FA_DTYPE_F16)
        add(dtype == FA_DTYPE_BF16 ? fa::kBf16W64Kernels : fa::kF16W64Kernels, fa::kNumW64Kernels);
    int n = 0;
    const fa::KernelEntry* table = table_for(dtype, &n);
    add(table, n);
    for (int j = 0; j < count && j < cap && block_m && block_n; ++j) {
        block_m[j] = pairs[j][0];
        block_n[j] = pairs[j][1];
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
    return 7;
}

}  // extern "C"
