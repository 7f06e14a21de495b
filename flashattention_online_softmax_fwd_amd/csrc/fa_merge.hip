// fa_merge.hip -- merge of partial attention states (split-KV) for gfx950.
//
// Each of S partial states of a row is held normalised, o_s = acc_s / l_s and
// lse_s = m_s + ln l_s, which is the pages' state (m, l, acc) measured against
// m_s + ln l_s: (lse_s, 1, o_s).  Their merge is the pages' merge of states built
// from disjoint key sets (spicyshark.co lesson, "From softmax to attention", two
// workers; kbwen.com feed, "More than two blocks"): take the largest max, weight
// each state by exp(its max - that max), add, and divide once at the end:
//     m = max_s lse_s,  w_s = exp(lse_s - m),  lse = m + ln sum_s w_s,
//     o = sum_s w_s o_s / sum_s w_s.
// An empty state (lse_s = -inf) has weight 0; a row whose states are all empty
// gets o = 0 and lse = -inf.
//
// HBM-bound: every partial value is read once and the result written once.  One
// wave per row, each lane holding D/64 consecutive floats of it, so every wave
// reads 4*D contiguous bytes per state.  The states are folded in chunks of eight
// whose loads are all in flight together: a chunk's largest max becomes the
// running reference, the running sum and weighted sum are rescaled to it once,
// and the chunk's states are added (the pages' block update, with states for
// blocks).
#include "fa_kernels.h"

#include <math.h>

namespace fa {

template <int D, typename OutT>
__global__ void __launch_bounds__(256) merge_kernel(const MergeParams p)
{
    constexpr int PER = D / 64;            // floats per lane
    constexpr int CH = 8;                  // states per chunk
    static_assert(PER == 1 || PER == 2, "head dimension 64 or 128");
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= p.rows) return;
    const long long R = p.rows;
    const int S = p.splits;

    float m = -INFINITY;                   // running reference (largest lse so far)
    float l = 0.f;                         // sum of weights against m
    float acc[PER];                        // weighted sum of the o_s against m
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    for (int s0 = 0; s0 < S; s0 += CH) {
        float ls[CH], x[CH][PER];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int s = s0 + c;
            ls[c] = -INFINITY;
#pragma unroll
            for (int e = 0; e < PER; ++e) x[c][e] = 0.f;
            if (s < S) {
                ls[c] = p.lse_part[s * R + row];
                const float* src = p.o_part + (s * R + row) * D + PER * lane;
                if constexpr (PER == 2) {
                    const float2 v = *(const float2*)src;
                    x[c][0] = v.x;
                    x[c][1] = v.y;
                } else {
                    x[c][0] = src[0];
                }
            }
        }
        float cm = m;
#pragma unroll
        for (int c = 0; c < CH; ++c) cm = fmaxf(cm, ls[c]);
        if (cm == -INFINITY) continue;     // nothing but empty states so far
        const float a = expf(m - cm);      // 0 while m is still -inf
        l *= a;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] *= a;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const bool live = ls[c] > -INFINITY;   // an empty state adds nothing, whatever its o
            const float w = live ? expf(ls[c] - cm) : 0.f;
            l += w;
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, live ? x[c][e] : 0.f, acc[e]);
        }
        m = cm;
    }
    const bool empty = !(l > 0.f);
    const float inv = empty ? 0.f : 1.f / l;
    OutT* dst = (OutT*)p.o + row * D + PER * lane;
#pragma unroll
    for (int e = 0; e < PER; ++e) dst[e] = (OutT)(acc[e] * inv);   // round to nearest even
    if (lane == 0) p.lse[row] = empty ? -INFINITY : m + logf(l);
}

template __global__ void merge_kernel<128, float>(const MergeParams);
template __global__ void merge_kernel<128, __bf16>(const MergeParams);
template __global__ void merge_kernel<128, _Float16>(const MergeParams);
template __global__ void merge_kernel<64, float>(const MergeParams);
template __global__ void merge_kernel<64, __bf16>(const MergeParams);
template __global__ void merge_kernel<64, _Float16>(const MergeParams);

#if !defined(__HIP_DEVICE_COMPILE__)
namespace {
template <int D>
const void* merge_fn(int out_dtype)
{
    // out_dtype: 0 float32, 1 bfloat16, 2 float16 (validated by the caller)
    if (out_dtype == 1) return (const void*)&merge_kernel<D, __bf16>;
    if (out_dtype == 2) return (const void*)&merge_kernel<D, _Float16>;
    return (const void*)&merge_kernel<D, float>;
}
}  // namespace

hipError_t launch_merge(const MergeParams& p, int d, int out_dtype, hipStream_t stream)
{
    const long long grid = (p.rows + 3) / 4;
    MergeParams args = p;
    void* kargs[] = {&args};
    const void* fn = d == 128 ? merge_fn<128>(out_dtype) : merge_fn<64>(out_dtype);
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), kargs, 0, stream);
}
#endif

}  // namespace fa
