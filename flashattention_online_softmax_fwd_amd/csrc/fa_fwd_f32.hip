// fa_fwd_f32.hip -- float32 FlashAttention forward for gfx950 (CDNA4, MI355X).
//
// Same recurrence as the bf16 path (kbwen.com FlashAttention feed, "Two blocks"
// and "More than two blocks"; spicyshark.co online-softmax lesson, "From
// softmax to attention" and "The implementation"), with float32 everywhere:
// both products run on v_mfma_f32_16x16x4_f32, and P stays float32.
//
// A workgroup of 4 waves owns 64 query rows; each wave owns 16.  Scores are
// computed transposed (S^T = K Q^T) so that lane L of the 16x16 output holds
// one query row, four keys per 16-key tile; the row max and row sum then need
// one in-lane pass and two lane exchanges, and P is already the B operand of
// the PV product.  K and V tiles are staged row-major in LDS with a 4-float
// pad; the PV A operand (V^T) is one float per lane, read down a column.
#include "fa_kernels.h"

#include <stdint.h>

namespace fa {

typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr float kLn2 = 0.693147180559945309f;

template <int D, int BN, bool CAUSAL>
__global__ void __launch_bounds__(256)
fwd_f32_kernel(const FwdParams p)
{
    constexpr int BM = 64;
    constexpr int NT = 256;
    constexpr int KS = D + 4;          // row stride of the K and V tiles (floats)
    constexpr int DK = D / 4;          // MFMA k-steps over the head dimension
    constexpr int ST = BN / 16;        // 16-key score tiles per K/V tile
    constexpr int DT = D / 16;         // 16-dim output tiles
    constexpr int CH = BN * D / 4 / NT;  // 16-byte chunks per thread per tile (each of K, V)
    static_assert((BN * D / 4) % NT == 0, "tile must split evenly over the threads");

    __shared__ __attribute__((aligned(16))) float sk[BN * KS];
    __shared__ __attribute__((aligned(16))) float sv[BN * KS];

    const int N = p.N;
    const int bhc = p.B * p.Hq;
    const int bid = blockIdx.x;
    const int qt = CAUSAL ? (p.n_qtiles - 1 - bid / bhc) : (bid / bhc);
    const int bh = bid % bhc;
    const int b = bh / p.Hq;
    const int hq = bh - b * p.Hq;
    const int hk = hq / p.group;
    const float* __restrict__ Qh = (const float*)p.q + (size_t)bh * N * D;
    const float* __restrict__ Kh = (const float*)p.k + (size_t)(b * p.Hkv + hk) * N * D;
    const float* __restrict__ Vh = (const float*)p.v + (size_t)(b * p.Hkv + hk) * N * D;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int g = lane >> 4;               // k-slot group of the MFMA operands
    const int q0 = qt * BM;
    const int qw0 = q0 + wave * 16;
    const int my_q = qw0 + l16;

    // Q as the B operand: lane holds dim 4kk + g of its query row.
    float qf[DK];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
        qf[kk] = (my_q < N) ? Qh[(size_t)my_q * D + 4 * kk + g] : 0.f;

    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;
    float l_run = 0.f;

    const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
    const int ntiles = (kv_end + BN - 1) / BN;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    for (int j = 0; j < ntiles; ++j) {
        const int kv0 = j * BN;
        __syncthreads();                   // the previous tile is no longer read
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + i * NT;
            const int key = c / (D / 4);
            const int col = (c % (D / 4)) * 4;
            const int gk = kv0 + key;
            const bool in = gk < N;
            *(f32x4*)&sk[key * KS + col] = in ? *(const f32x4*)(Kh + (size_t)gk * D + col) : zero4;
            *(f32x4*)&sv[key * KS + col] = in ? *(const f32x4*)(Vh + (size_t)gk * D + col) : zero4;
        }
        __syncthreads();
        if (CAUSAL && kv0 > qw0 + 15) continue;   // fully masked for this wave

        f32x4 s[ST];
#pragma unroll
        for (int t = 0; t < ST; ++t) {
            s[t] = zero4;
#pragma unroll
            for (int kk = 0; kk < DK; ++kk)
                s[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(sk[(16 * t + l16) * KS + 4 * kk + g], qf[kk],
                                                           s[t], 0, 0, 0);
        }
        // lane holds keys kv0 + 16t + 4g + i of query my_q
        const bool need_mask = (CAUSAL && kv0 + BN - 1 > qw0) || (kv0 + BN > N);
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < ST; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float x = s[t][i] * p.scale_log2;
                if (need_mask) {
                    const int key = kv0 + 16 * t + 4 * g + i;
                    if (key >= N || (CAUSAL && key > my_q)) x = -INFINITY;
                }
                s[t][i] = x;
                mx = fmaxf(mx, x);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;
        float rs = 0.f;
#pragma unroll
        for (int t = 0; t < ST; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = __builtin_amdgcn_exp2f(s[t][i] - m_use);
                s[t][i] = e;
                rs += e;
            }
        l_run = l_run * alpha + rs;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int t = 0; t < ST; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        sv[(16 * t + 4 * g + i) * KS + 16 * dt + l16], s[t][i], o[dt], 0, 0, 0);
    }

    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (my_q < N) {
        const float inv = 1.f / l_tot;
        float* Orow = (float*)p.o + (size_t)bh * N * D + (size_t)my_q * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) *(f32x4*)(Orow + 16 * dt + 4 * g) = o[dt] * inv;
        if (g == 0)
            p.lse[(size_t)bh * N + my_q] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
}

// Explicit instantiations, seen by both the host and the device pass.
#define FA_F32_INSTANTIATE(D, BN)                                              \
    template __global__ void fwd_f32_kernel<D, BN, false>(const FwdParams);  \
    template __global__ void fwd_f32_kernel<D, BN, true>(const FwdParams);
FA_F32_INSTANTIATE(64, 32)
FA_F32_INSTANTIATE(64, 64)
FA_F32_INSTANTIATE(128, 32)
FA_F32_INSTANTIATE(128, 64)

namespace {

template <int D, int BN, bool CAUSAL>
hipError_t launch_f32(const FwdParams& p, hipStream_t stream)
{
    const unsigned grid = (unsigned)((long long)p.B * p.Hq * p.n_qtiles);
    FwdParams args = p;
    void* kargs[] = {&args};
    return hipLaunchKernel((const void*)&fwd_f32_kernel<D, BN, CAUSAL>, dim3(grid), dim3(256),
                           kargs, 0, stream);
}

}  // namespace

// The dispatch table is host data: it is not emitted in the device pass.
#if !defined(__HIP_DEVICE_COMPILE__)
#define FA_F32_ENTRY(D, BN)                                  \
    {0, D, 64, BN, 0, &launch_f32<D, BN, false>},           \
    {0, D, 64, BN, 1, &launch_f32<D, BN, true>}

const KernelEntry kF32Kernels[] = {
    FA_F32_ENTRY(64, 32),
    FA_F32_ENTRY(64, 64),
    FA_F32_ENTRY(128, 32),
    FA_F32_ENTRY(128, 64),
};
const int kNumF32Kernels = sizeof(kF32Kernels) / sizeof(kF32Kernels[0]);

#endif

}  // namespace fa
