// Host-side checks of the C ABI (include/fa.h), built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_asan.py and run on the CPU.
//
// Every call below is one the library must refuse, or finish as empty, before it makes any
// HIP call: the pointers are never dereferenced (they stand for device memory), so a
// sanitizer report here means the host validation itself read, wrote or computed something
// it should not.  The cases mirror tests/test_abi.py.  Exit status: 0 when every call
// returned what it should, 1 otherwise (each failure printed).
#include "fa.h"

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <limits>

namespace {

int failures = 0;

// Entry points that return FA_OK or an error code: a refusal must also leave a message.
void expect(int got, int want, const char* what, int line, bool code)
{
    if (got != want) {
        std::printf("line %d: %s returned %d, expected %d (%s)\n", line, what, got, want, fa_last_error());
        ++failures;
    } else if (code && want != FA_OK && (!fa_last_error() || !*fa_last_error())) {
        std::printf("line %d: %s refused without a message\n", line, what);
        ++failures;
    }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__, true)
#define EXPECT_VALUE(call, want) expect((call), (want), #call, __LINE__, false)

const uintptr_t P = 0x10000;   // 16-byte aligned, non-null, never dereferenced
void* at(uintptr_t off) { return reinterpret_cast<void*>(P + off); }
float* fat(uintptr_t off) { return reinterpret_cast<float*>(P + off); }
const float nan_ = std::numeric_limits<float>::quiet_NaN();
const float inf_ = std::numeric_limits<float>::infinity();

struct Fwd {
    void *q = at(0), *k = at(0x100000), *v = at(0x200000), *o = at(0x300000);
    float* lse = fat(0x400000);
    int B = 1, Hq = 2, Hkv = 1, N = 16, d = 64, causal = 0;
    float scale = 0.125f;
    int dtype = FA_DTYPE_BF16;
    int run() const { return fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, scale, dtype, nullptr); }
};

struct Split {
    void *q = at(0), *k = at(0x100000), *v = at(0x200000);
    float *op = fat(0x300000), *lp = fat(0x500000);
    int B = 1, Hq = 2, Hkv = 1, Nq = 4, Nk = 300, d = 64, causal = 1;
    float scale = 0.125f;
    int dtype = FA_DTYPE_BF16, splits = 3;
    int run() const
    {
        return fa_fwd_splitkv(q, k, v, op, lp, B, Hq, Hkv, Nq, Nk, d, causal, scale, dtype, splits, nullptr);
    }
};

struct Bwd {
    void *q = at(0), *k = at(0x100000), *v = at(0x200000), *o = at(0x300000);
    float* lse = fat(0x400000);
    void *dO = at(0x500000), *dq = at(0x600000), *dk = at(0x700000), *dv = at(0x800000);
    float* delta = fat(0x900000);
    float* part = fat(0xa00000);
    int B = 1, Hq = 2, Hkv = 1, N = 300, d = 64, causal = 1;
    float scale = 0.125f;
    int dtype = FA_DTYPE_BF16, splits = 2;
    int run() const { return fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, delta, B, Hq, Hkv, N, d, causal, scale, dtype, nullptr); }
    int split() const
    {
        return fa_bwd_split(q, k, v, o, lse, dO, dq, dk, dv, delta, part, splits, B, Hq, Hkv, N, d, causal, scale, dtype,
                            nullptr);
    }
    int noalloc() const
    {
        return fa_bwd_split_noalloc(q, k, v, o, lse, dO, dq, dk, dv, delta, splits, B, Hq, Hkv, N, d, causal, scale,
                                    dtype, nullptr);
    }
};

template <typename T, typename F>
int with(F change)
{
    T t;
    change(t);
    return t.run();
}

}  // namespace

int main()
{
    // ---- version, error strings, tile shapes, sizes
    EXPECT_VALUE(fa_abi_version() > 0, 1);
    for (int code = -2; code < 8; ++code)
        if (!fa_error_string(code) || !*fa_error_string(code)) {
            std::printf("empty error string for %d\n", code);
            ++failures;
        }
    int bm[16], bn[16];
    for (int dtype = 0; dtype < 3; ++dtype)
        for (int d : {64, 128}) {
            const int n = fa_tile_shapes(dtype, d, bm, bn, 16);
            if (n < 2 || n > 16) {
                std::printf("fa_tile_shapes(%d, %d) = %d\n", dtype, d, n);
                ++failures;
            }
            if (fa_tile_shapes(dtype, d, nullptr, nullptr, 0) != n) ++failures;
            if (fa_tile_shapes(dtype, d, bm, bn, 1) != n) ++failures;   // capacity smaller than the list
        }
    EXPECT_VALUE(fa_tile_shapes(1, 96, nullptr, nullptr, 0), -1);
    EXPECT_VALUE(fa_tile_shapes(7, 64, nullptr, nullptr, 0), -1);
    EXPECT_VALUE(fa_fwd_stamp_slots(1, 1, 64, 64, 0) == -1, 1);
    EXPECT_VALUE(fa_fwd_stamp_slots(1, 0, 64, 64, 1) == -1, 1);
    EXPECT_VALUE(fa_fwd_stamp_slots(0, 3, 100, 64, 1), 0);
    EXPECT_VALUE(fa_split_chunk(4096, 3), 1408);
    EXPECT_VALUE(fa_split_chunk(-1, 2), -1);
    EXPECT_VALUE(fa_split_chunk(10, 0), -1);
    EXPECT_VALUE(fa_splitkv_num_splits(8, 32, 8, 1, 32768), 16);
    EXPECT_VALUE(fa_splitkv_num_splits(1, 3, 2, 1, 1), -1);
    EXPECT_VALUE(fa_bwd_num_splits(1, 32, 8, 8192), 2);
    EXPECT_VALUE(fa_bwd_num_splits(0, 1, 1, 1), -1);
    EXPECT_VALUE(fa_bwd_noalloc_max_bytes() == (128ll << 20), 1);

    // ---- forward
    EXPECT(with<Fwd>([](Fwd& a) { a.q = nullptr; }), FA_ERR_INVALID_ARG);
    EXPECT(with<Fwd>([](Fwd& a) { a.lse = nullptr; }), FA_ERR_INVALID_ARG);
    EXPECT(with<Fwd>([](Fwd& a) { a.q = at(8); }), FA_ERR_INVALID_ARG);               // misaligned
    EXPECT(with<Fwd>([](Fwd& a) { a.B = -1; }), FA_ERR_INVALID_ARG);
    EXPECT(with<Fwd>([](Fwd& a) { a.N = -5; }), FA_ERR_INVALID_ARG);
    EXPECT(with<Fwd>([](Fwd& a) { a.Hq = 3; a.Hkv = 2; }), FA_ERR_INVALID_ARG);
    EXPECT(with<Fwd>([](Fwd& a) { a.causal = 2; }), FA_ERR_INVALID_ARG);
    EXPECT(with<Fwd>([](Fwd& a) { a.scale = inf_; }), FA_ERR_INVALID_ARG);
    EXPECT(with<Fwd>([](Fwd& a) { a.scale = nan_; }), FA_ERR_INVALID_ARG);
    EXPECT(with<Fwd>([](Fwd& a) { a.scale = 3e38f; }), FA_ERR_INVALID_ARG);
    EXPECT(with<Fwd>([](Fwd& a) { a.dtype = 5; }), FA_ERR_INVALID_ARG);
    EXPECT(with<Fwd>([](Fwd& a) { a.d = 96; }), FA_ERR_UNSUPPORTED);
    EXPECT(with<Fwd>([](Fwd& a) { a.o = a.q; }), FA_ERR_INVALID_ARG);                 // o overlaps q
    EXPECT(with<Fwd>([](Fwd& a) { a.lse = fat(0x300010); }), FA_ERR_INVALID_ARG);     // lse overlaps o
    EXPECT(with<Fwd>([](Fwd& a) { a.N = (0x7FFFFFFF / 256) - 127; a.d = 128; a.Hq = 1; }), FA_ERR_UNSUPPORTED);
    EXPECT(with<Fwd>([](Fwd& a) { a.q = a.k = a.v = a.o = nullptr; a.lse = nullptr; a.B = 0; }), FA_OK);
    EXPECT(with<Fwd>([](Fwd& a) { a.q = a.k = a.v = a.o = nullptr; a.lse = nullptr; a.N = 0; }), FA_OK);
    {
        Fwd a;
        EXPECT(fa_fwd_tiled(a.q, a.k, a.v, a.o, a.lse, 1, 2, 1, 16, 64, 0, 0.125f, 1, nullptr, 96, 64),
               FA_ERR_UNSUPPORTED);
        unsigned long long* st = reinterpret_cast<unsigned long long*>(P + 0x600000);
        EXPECT(fa_fwd_stamped(a.q, a.k, a.v, a.o, a.lse, 1, 2, 1, 16, 64, 0, 0.125f, 1, nullptr, nullptr, 1 << 20),
               FA_ERR_INVALID_ARG);
        EXPECT(fa_fwd_stamped(a.q, a.k, a.v, a.o, a.lse, 1, 2, 1, 16, 64, 0, 0.125f, 1, nullptr, st, 3),
               FA_ERR_INVALID_ARG);
        EXPECT(fa_fwd_stamped(a.q, a.k, a.v, a.o, a.lse, 1, 2, 1, 16, 64, 0, 0.125f, 1, nullptr,
                              reinterpret_cast<unsigned long long*>(P + 0x300000), 1 << 20),
               FA_ERR_INVALID_ARG);
        EXPECT(fa_fwd_stamped(a.q, a.k, a.v, a.o, a.lse, 1, 2, 1, 16, 64, 0, 0.125f, 0, nullptr, st, 1 << 20),
               FA_ERR_UNSUPPORTED);
    }

    // ---- split-KV partial states and their merge
    EXPECT(with<Split>([](Split& a) { a.q = nullptr; }), FA_ERR_INVALID_ARG);
    EXPECT(with<Split>([](Split& a) { a.lp = fat(0x500004); }), FA_ERR_INVALID_ARG);
    EXPECT(with<Split>([](Split& a) { a.Nk = 0; }), FA_ERR_INVALID_ARG);
    EXPECT(with<Split>([](Split& a) { a.splits = 0; }), FA_ERR_INVALID_ARG);
    EXPECT(with<Split>([](Split& a) { a.splits = 1025; }), FA_ERR_INVALID_ARG);
    EXPECT(with<Split>([](Split& a) { a.Nq = 301; }), FA_ERR_INVALID_ARG);
    EXPECT(with<Split>([](Split& a) { a.dtype = 0; }), FA_ERR_UNSUPPORTED);
    EXPECT(with<Split>([](Split& a) { a.op = fat(0x100000); }), FA_ERR_INVALID_ARG);
    EXPECT(with<Split>([](Split& a) {
               a.Hq = 64; a.Hkv = 1; a.Nq = 1 << 25; a.causal = 0;
               a.k = at(1ull << 40); a.v = at(2ull << 40); a.op = fat(4ull << 40); a.lp = fat(8ull << 40);
           }),
           FA_ERR_UNSUPPORTED);
    EXPECT(with<Split>([](Split& a) { a.q = a.k = a.v = nullptr; a.op = a.lp = nullptr; a.B = 0; }), FA_OK);
    EXPECT(fa_merge(nullptr, fat(0x100000), at(0x200000), fat(0x300000), 4, 1, 2, 8, 64, 1, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_merge(fat(0), fat(0x100000), at(0x200000), fat(0x300000), 0, 1, 2, 8, 64, 1, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_merge(fat(0), fat(0x100000), at(0x200000), fat(0x300000), 4, 1, 2, 8, 96, 1, nullptr), FA_ERR_UNSUPPORTED);
    EXPECT(fa_merge(fat(0), fat(0x100000), at(8), fat(0x300000), 4, 1, 2, 8, 64, 1, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_merge(nullptr, nullptr, nullptr, nullptr, 4, 0, 2, 8, 64, 1, nullptr), FA_OK);

    // ---- row softmax
    EXPECT(fa_softmax(nullptr, at(0x100000), nullptr, 4, 64, 0, 0, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_softmax(at(0), at(0x100000), nullptr, 4, 64, 5, 0, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_softmax(at(0), at(0x100000), nullptr, 4, 64, 0, 2, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_softmax(at(0), at(0x100000), nullptr, -1, 64, 0, 0, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_softmax(at(0), at(4), nullptr, 4, 64, 0, 0, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_softmax(at(0), at(0x40), nullptr, 4, 64, 0, 0, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_softmax(at(0), at(0x100000), fat(0x20), 4, 64, 0, 0, nullptr), FA_ERR_INVALID_ARG);
    EXPECT(fa_softmax(at(0), at(0x100000), nullptr, 1ll << 31, 64, 0, 0, nullptr), FA_ERR_UNSUPPORTED);
    EXPECT(fa_softmax(at(0), at(0), nullptr, 1, 0x7FFFFFFF, 0, 0, nullptr), FA_ERR_UNSUPPORTED);
    EXPECT(fa_softmax(nullptr, nullptr, nullptr, 0, 64, 0, 0, nullptr), FA_OK);

    // ---- backward
    EXPECT(with<Bwd>([](Bwd& a) { a.q = nullptr; }), FA_ERR_INVALID_ARG);
    EXPECT(with<Bwd>([](Bwd& a) { a.delta = nullptr; }), FA_ERR_INVALID_ARG);
    EXPECT(with<Bwd>([](Bwd& a) { a.dv = at(0x800008); }), FA_ERR_INVALID_ARG);
    EXPECT(with<Bwd>([](Bwd& a) { a.Hkv = 0; }), FA_ERR_INVALID_ARG);
    EXPECT(with<Bwd>([](Bwd& a) { a.scale = 3e38f; }), FA_ERR_INVALID_ARG);
    EXPECT(with<Bwd>([](Bwd& a) { a.dtype = 0; }), FA_ERR_UNSUPPORTED);
    EXPECT(with<Bwd>([](Bwd& a) { a.d = 80; }), FA_ERR_UNSUPPORTED);
    EXPECT(with<Bwd>([](Bwd& a) { a.dk = at(0x600100); }), FA_ERR_INVALID_ARG);
    EXPECT(with<Bwd>([](Bwd& a) { a.dv = at(0x400000); }), FA_ERR_INVALID_ARG);
    {
        Bwd a;
        a.q = a.k = a.v = a.o = a.dO = a.dq = a.dk = a.dv = nullptr;
        a.lse = a.delta = nullptr;
        a.B = 0;
        EXPECT(a.run(), FA_OK);
        a.part = nullptr;
        a.splits = 4;
        EXPECT(a.split(), FA_OK);
        a.splits = 8;
        EXPECT(a.noalloc(), FA_OK);
    }
    {
        Bwd a;
        a.splits = 0;
        EXPECT(a.split(), FA_ERR_INVALID_ARG);
        a.splits = 9;
        EXPECT(a.split(), FA_ERR_INVALID_ARG);
        a.splits = 2;
        a.part = fat(0x700000);                            // workspace overlaps dk
        EXPECT(a.split(), FA_ERR_INVALID_ARG);
        a.part = nullptr;
        a.splits = 1;
        a.q = nullptr;                                     // one split needs no workspace: the q check speaks
        EXPECT(a.split(), FA_ERR_INVALID_ARG);
    }
    {
        Bwd a;
        a.splits = 9;
        EXPECT(a.noalloc(), FA_ERR_INVALID_ARG);
        a.splits = 8;
        a.Hq = a.Hkv = 8;
        a.N = 4096;
        a.d = 128;
        void** ptrs[] = {&a.q, &a.k, &a.v, &a.o, &a.dO, &a.dq, &a.dk, &a.dv};
        for (int i = 0; i < 8; ++i) *ptrs[i] = at((uintptr_t)(i + 1) << 32);
        a.lse = fat(9ull << 32);
        a.delta = fat(10ull << 32);
        EXPECT(a.noalloc(), FA_ERR_UNSUPPORTED);          // partials beyond the static workspace
    }

    if (failures) std::printf("%d host checks failed\n", failures);
    else std::printf("host checks passed\n");
    return failures ? 1 : 0;
}
