// fa_fwd_bf16.hip -- bf16 FlashAttention forward for gfx950 (CDNA4, MI355X).
//
// One workgroup owns BM query rows of one (batch, query head) and walks the key
// tiles of its K/V head in order (query blocks outer, key blocks inner: kbwen.com
// FlashAttention feed, "More than two blocks").  Each wave owns 32 query rows.
//
// Per key tile of BN keys, for each wave:
//   S^T = K_tile Q_w^T        v_mfma_f32_32x32x16_bf16, fp32 accumulate
//   t   = S^T * scale*log2(e), -inf where masked (causal j > i, or j >= N)
//   m'  = max(m, rowmax t)     in-lane max over 32 keys, then one lane swap
//   a   = exp2(m - m'),  P = exp2(t - m')      (a row with no finite score yet
//                                               uses 0 as its reference: the guard)
//   l   = a*l + rowsum P,  O^T = a*O^T + V_tile^T P^T     (P rounded to bf16)
// and after the last tile O = O^T / l, LSE = (m + log2 l) * ln 2.
// The update is the one the pages derive (mbrenndoerfer.com "Online Softmax
// Computation", its five steps; spicyshark.co online-softmax lesson, "From
// softmax to attention" and "The implementation"), in base 2: exp(x) =
// exp2(x*log2 e), so the scale and log2(e) fold into one multiplier.
//
// Why the scores are computed transposed: the 32x32 MFMA leaves lane L holding
// one column of its output.  With K as the A operand and Q as the B operand
// that column is one query row, so the row max and row sum are in-lane except
// for one exchange between lane halves, and the bf16-rounded probabilities are
// already where the PV MFMA wants its B operand: no LDS round trip for P.
//
// LDS, double-buffered: K tile [BN][D+8] (row-major, 16-byte pad) and V^T tile
// [D][BN+8].  V is transposed in registers while it is staged (4 keys x 8 dims per
// thread, v_perm_b32), and the keys of each group of 16 are stored in the order
// that makes each lane's 8 PV operands one contiguous 16-byte read.
#include "fa_kernels.h"

#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

constexpr float kLn2 = 0.693147180559945309f;

// Position of key `key4` (a multiple of 4) inside the V^T row: within each group
// of 16 keys, key 16g + 8a + 4b + c is stored at 16g + 8b + 4a + c.  The lane
// half `hi` of a PV MFMA then reads keys {4hi..4hi+3, 8+4hi..8+4hi+3} of the
// group -- exactly the keys its score registers hold -- as one 16-byte vector.
__device__ __forceinline__ int vt_pos(int key4)
{
    return (key4 & ~15) | ((key4 & 4) << 1) | ((key4 & 8) >> 1);
}

template <int D, int BM, int BN, bool CAUSAL>
__global__ void __launch_bounds__(BM * 2)
fwd_bf16_kernel(const FwdParams p)
{
    constexpr int NW = BM / 32;            // waves, 32 query rows each
    constexpr int NT = NW * 64;            // threads
    constexpr int KS = D + 8;              // K tile row stride (elements)
    constexpr int VS = BN + 8;             // V^T tile row stride (elements)
    constexpr int DK = D / 16;             // MFMA k-steps over the head dimension
    constexpr int ST = BN / 32;            // 32-key score tiles per K/V tile
    constexpr int DT = D / 32;             // 32-dim output tiles
    constexpr int KCH = BN * D / 8 / NT;   // 16-byte K chunks per thread per tile
    constexpr int VUNITS = (BN / 4) * (D / 8);   // V staging units: 4 keys x 8 dims
    constexpr int VPT = (VUNITS + NT - 1) / NT;
    static_assert(BM % 32 == 0 && BN % 32 == 0 && D % 32 == 0, "tile shape");
    static_assert((BN * D / 8) % NT == 0, "K tile must split evenly over the threads");

    __shared__ __attribute__((aligned(16))) bf16 sk[2][BN * KS];
    __shared__ __attribute__((aligned(16))) bf16 sv[2][D * VS];

    const int N = p.N;
    const int bhc = p.B * p.Hq;
    const int bid = blockIdx.x;
    // Causal: the longest rows first, so the tail of the grid is short work.
    const int qt = CAUSAL ? (p.n_qtiles - 1 - bid / bhc) : (bid / bhc);
    const int bh = bid % bhc;
    const int b = bh / p.Hq;
    const int hq = bh - b * p.Hq;
    const int hk = hq / p.group;
    const bf16* __restrict__ Qh = (const bf16*)p.q + (size_t)bh * N * D;
    const bf16* __restrict__ Kh = (const bf16*)p.k + (size_t)(b * p.Hkv + hk) * N * D;
    const bf16* __restrict__ Vh = (const bf16*)p.v + (size_t)(b * p.Hkv + hk) * N * D;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const int q0 = qt * BM;
    const int qw0 = q0 + wave * 32;
    const int my_q = qw0 + l32;            // the query row this lane's columns belong to

    const u32x4 zero4 = {0u, 0u, 0u, 0u};

    // Q as the B operand: lane holds dims 16kk + 8hi .. +7 of its query row.
    bf16x8 qf[DK];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
        qf[kk] = (my_q < N) ? *(const bf16x8*)(Qh + (size_t)my_q * D + 16 * kk + 8 * hi)
                            : __builtin_bit_cast(bf16x8, zero4);

    f32x16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
    float m_run = -INFINITY;   // running max, log2 domain of the scaled score
    float l_run = 0.f;         // running sum over this lane half's keys

    const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
    const int ntiles = (kv_end + BN - 1) / BN;

    u32x4 kr[KCH];
    u32x4 vr[VPT][4];

    auto gload = [&](int j) {
        const int kv0 = j * BN;
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int c = tid + i * NT;
            const int key = c / (D / 8);
            const int col = (c % (D / 8)) * 8;
            const int gk = kv0 + key;
            kr[i] = (gk < N) ? *(const u32x4*)(Kh + (size_t)gk * D + col) : zero4;
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int u = tid + i * NT;
            if ((VUNITS % NT) == 0 || u < VUNITS) {
                const int quad = u % (BN / 4);
                const int ch = u / (BN / 4);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int gk = kv0 + 4 * quad + r;
                    vr[i][r] = (gk < N) ? *(const u32x4*)(Vh + (size_t)gk * D + 8 * ch) : zero4;
                }
            }
        }
    };

    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int c = tid + i * NT;
            const int key = c / (D / 8);
            const int col = (c % (D / 8)) * 8;
            *(u32x4*)&sk[buf][key * KS + col] = kr[i];
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int u = tid + i * NT;
            if ((VUNITS % NT) == 0 || u < VUNITS) {
                const int quad = u % (BN / 4);
                const int ch = u / (BN / 4);
                const int pos = vt_pos(4 * quad);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // dims 8ch+2e (low halves) and 8ch+2e+1 (high halves) of keys 0..3
                    u32x2 ev, od;
                    ev[0] = __builtin_amdgcn_perm(vr[i][1][e], vr[i][0][e], 0x05040100u);
                    ev[1] = __builtin_amdgcn_perm(vr[i][3][e], vr[i][2][e], 0x05040100u);
                    od[0] = __builtin_amdgcn_perm(vr[i][1][e], vr[i][0][e], 0x07060302u);
                    od[1] = __builtin_amdgcn_perm(vr[i][3][e], vr[i][2][e], 0x07060302u);
                    *(u32x2*)&sv[buf][(8 * ch + 2 * e) * VS + pos] = ev;
                    *(u32x2*)&sv[buf][(8 * ch + 2 * e + 1) * VS + pos] = od;
                }
            }
        }
    };

    auto compute = [&](int j, int buf) {
        const int kv0 = j * BN;
        if (CAUSAL && kv0 > qw0 + 31) return;     // every key of the tile is masked for this wave

        f32x16 s[ST];
#pragma unroll
        for (int t = 0; t < ST; ++t) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[t][r] = 0.f;
#pragma unroll
            for (int kk = 0; kk < DK; ++kk) {
                const bf16x8 a = *(const bf16x8*)&sk[buf][(32 * t + l32) * KS + 16 * kk + 8 * hi];
                s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[t], 0, 0, 0);
            }
        }

        // lane holds keys kv0 + 32t + 8(r/4) + 4hi + r%4 of query my_q
        const bool need_mask = (CAUSAL && kv0 + BN - 1 > qw0) || (kv0 + BN > N);
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < ST; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = s[t][r] * p.scale_log2;
                if (need_mask) {
                    const int key = kv0 + 32 * t + 8 * (r >> 2) + 4 * hi + (r & 3);
                    if (key >= N || (CAUSAL && key > my_q)) x = -INFINITY;
                }
                s[t][r] = x;
                mx = fmaxf(mx, x);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;   // no finite score yet
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;

        float rs = 0.f;
        bf16x8 pb[ST][2];
#pragma unroll
        for (int t = 0; t < ST; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = __builtin_amdgcn_exp2f(s[t][r] - m_use);
                rs += e;
                pb[t][r >> 3][r & 7] = (bf16)e;
            }
        l_run = l_run * alpha + rs;

#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;

#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int t = 0; t < ST; ++t)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const bf16x8 a =
                        *(const bf16x8*)&sv[buf][(32 * dt + l32) * VS + 32 * t + 16 * u + 8 * hi];
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[t][u], o[dt], 0, 0, 0);
                }
    };

    gload(0);
    lstore(0);
    __syncthreads();
    for (int j = 0; j < ntiles; ++j) {
        const bool more = j + 1 < ntiles;
        if (more) gload(j + 1);
        compute(j, j & 1);
        if (more) lstore((j + 1) & 1);
        __syncthreads();
    }

    // epilogue: O = u / l, LSE = m + ln l
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (my_q < N) {
        const float inv = 1.f / l_tot;
        bf16* Orow = (bf16*)p.o + (size_t)bh * N * D + (size_t)my_q * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 w;
#pragma unroll
                for (int c = 0; c < 4; ++c) w[c] = (bf16)(o[dt][4 * g + c] * inv);
                *(bf16x4*)(Orow + 32 * dt + 8 * g + 4 * hi) = w;
            }
        if (hi == 0)
            p.lse[(size_t)bh * N + my_q] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
}

// Explicit instantiations: both the host and the device pass must see every
// kernel the dispatch table names.
#define FA_BF16_INSTANTIATE(D, BM, BN)                                              \
    template __global__ void fwd_bf16_kernel<D, BM, BN, false>(const FwdParams);  \
    template __global__ void fwd_bf16_kernel<D, BM, BN, true>(const FwdParams);
FA_BF16_INSTANTIATE(128, 128, 64)
FA_BF16_INSTANTIATE(128, 128, 128)
FA_BF16_INSTANTIATE(128, 64, 64)
FA_BF16_INSTANTIATE(64, 128, 64)
FA_BF16_INSTANTIATE(64, 128, 128)
FA_BF16_INSTANTIATE(64, 64, 64)

namespace {

template <int D, int BM, int BN, bool CAUSAL>
hipError_t launch_bf16(const FwdParams& p, hipStream_t stream)
{
    const unsigned grid = (unsigned)((long long)p.B * p.Hq * p.n_qtiles);
    FwdParams args = p;
    void* kargs[] = {&args};
    return hipLaunchKernel((const void*)&fwd_bf16_kernel<D, BM, BN, CAUSAL>, dim3(grid),
                           dim3(BM * 2), kargs, 0, stream);
}

}  // namespace

// The dispatch table is host data: it is not emitted in the device pass.
#if !defined(__HIP_DEVICE_COMPILE__)
#define FA_BF16_ENTRY(D, BM, BN)                                   \
    {1, D, BM, BN, 0, &launch_bf16<D, BM, BN, false>},            \
    {1, D, BM, BN, 1, &launch_bf16<D, BM, BN, true>}

// The first shape listed for each head dimension is the default.
const KernelEntry kBf16Kernels[] = {
    FA_BF16_ENTRY(128, 128, 64),
    FA_BF16_ENTRY(128, 128, 128),
    FA_BF16_ENTRY(128, 64, 64),
    FA_BF16_ENTRY(64, 128, 64),
    FA_BF16_ENTRY(64, 128, 128),
    FA_BF16_ENTRY(64, 64, 64),
};
const int kNumBf16Kernels = sizeof(kBf16Kernels) / sizeof(kBf16Kernels[0]);

#endif

}  // namespace fa
