// fa_softmax.hip -- softmax of every row of a matrix, for gfx950, two ways.
//
// Both compute y_j = exp(x_j - m) / l with m the row's max and l the sum of
// exp(x_j - m) (spicyshark.co online-softmax lesson, "The fix: subtract the
// maximum"), and the row's log normaliser m + ln l.  They differ in how often the
// row is read (the lesson's "Why reading once matters"):
//   SAFE    three passes: the max, then the sum, then the output ("The cost: three
//           passes"): 3 reads and 1 write per element;
//   ONLINE  the running max and the running sum in one pass, the sum rescaled by
//           exp(m_old - m_new) whenever the max grows ("The idea"; the update of
//           Milakov and Gimelshein the pages cite), then the output: 2 reads and
//           1 write per element.
// The kernel is HBM-bound: the arithmetic per element is a few VALU operations and
// one exponential.
//
// One workgroup of 256 threads per row.  Thread t takes the 16-byte vectors
// t, t + 256, ... of its row, so each wave reads 1 KiB contiguous per step, four
// vectors in flight per thread.  A thread's partial states (m, l) are merged over
// the wave with lane exchanges and over the four waves through LDS, by the merge
// of two states (take the larger max, rescale each sum to it, add).  Exponentials
// are exp2 of x*log2(e) - m*log2(e), one FMA and one v_exp_f32 per element.
// A row whose entries are all -inf has no softmax: y is nan and lse is -inf, as
// the definition gives.  y may be x itself (in place): a row is written only after
// its statistics are complete, each element by the thread that read it.
#include "fa_kernels.h"

#include <math.h>

namespace fa {
namespace sm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.693147180559945309f;
constexpr int kThreads = 256;
constexpr int kUnroll = 4;

template <typename T>
__device__ __forceinline__ float to_f(T v) { return (float)v; }

// Merge two partial states (m, l): l measured against m, in base 2 (m in units of log2).
__device__ __forceinline__ void merge(float& m, float& l, float mo, float lo)
{
    const float mn = fmaxf(m, mo);
    if (mn == -INFINITY) return;   // both empty
    l = l * __builtin_amdgcn_exp2f(m - mn) + lo * __builtin_amdgcn_exp2f(mo - mn);
    m = mn;
}

// Over the 256 threads of the workgroup; every thread gets the result.
__device__ __forceinline__ void block_merge(float& m, float& l, float* sh)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float mo = __shfl_xor(m, off, 64);
        const float lo = __shfl_xor(l, off, 64);
        merge(m, l, mo, lo);
    }
    const int wave = threadIdx.x >> 6;
    __syncthreads();                       // sh may still be read by a previous reduction
    if ((threadIdx.x & 63) == 0) {
        sh[2 * wave] = m;
        sh[2 * wave + 1] = l;
    }
    __syncthreads();
    m = sh[0];
    l = sh[1];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) merge(m, l, sh[2 * w], sh[2 * w + 1]);
}

__device__ __forceinline__ float block_max(float v, float* sh)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[wave] = v;
    __syncthreads();
    v = sh[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) v = fmaxf(v, sh[w]);
    return v;
}

__device__ __forceinline__ float block_sum(float v, float* sh)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[wave] = v;
    __syncthreads();
    v = sh[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) v += sh[w];
    return v;
}

// VEC elements of T in one load (16 bytes, or one element for rows that are not
// 16-byte aligned).
template <typename T, int VEC>
struct __attribute__((aligned(sizeof(T) * VEC))) Vec {
    T e[VEC];
};

}  // namespace sm

template <typename T, bool ONLINE, int VEC>
__global__ void __launch_bounds__(256) softmax_kernel(const T* x, T* y, float* lse, int cols)
{
    using namespace sm;
    typedef Vec<T, VEC> V;
    __shared__ float sh[2 * kThreads / 64];
    const long long r = blockIdx.x;
    const V* xr = (const V*)(x + r * cols);
    V* yr = (V*)(y + r * cols);
    const int tid = threadIdx.x;
    const int nv = cols / VEC;            // VEC divides cols (the host picks VEC = 1 otherwise)

    // Statistics, in base 2: m2 = max * log2(e), l = sum of exp2(x log2(e) - m2).
    float m2 = -INFINITY, l = 0.f;
    if constexpr (ONLINE) {
        for (int i0 = tid; i0 < nv; i0 += kThreads * kUnroll) {
            V v[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int i = i0 + u * kThreads;
                if (i < nv) v[u] = xr[i];
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int i = i0 + u * kThreads;
                if (i >= nv) break;
                float cm = -INFINITY;
#pragma unroll
                for (int e = 0; e < VEC; ++e) cm = fmaxf(cm, to_f(v[u].e[e]));
                cm *= kLog2e;
                if (cm > m2) {                 // the max grew: rescale the sum to it
                    l *= __builtin_amdgcn_exp2f(m2 - cm);
                    m2 = cm;
                }
                if (m2 > -INFINITY) {          // nothing finite yet: nothing to add
#pragma unroll
                    for (int e = 0; e < VEC; ++e) l += __builtin_amdgcn_exp2f(__builtin_fmaf(to_f(v[u].e[e]), kLog2e, -m2));
                }
            }
        }
        block_merge(m2, l, sh);
    } else {
        float mx = -INFINITY;
        for (int i0 = tid; i0 < nv; i0 += kThreads * kUnroll) {
            V v[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int i = i0 + u * kThreads;
                if (i < nv) v[u] = xr[i];
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                if (i0 + u * kThreads >= nv) break;
#pragma unroll
                for (int e = 0; e < VEC; ++e) mx = fmaxf(mx, to_f(v[u].e[e]));
            }
        }
        m2 = block_max(mx, sh) * kLog2e;
        if (m2 > -INFINITY) {
            for (int i0 = tid; i0 < nv; i0 += kThreads * kUnroll) {
                V v[kUnroll];
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const int i = i0 + u * kThreads;
                    if (i < nv) v[u] = xr[i];
                }
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    if (i0 + u * kThreads >= nv) break;
#pragma unroll
                    for (int e = 0; e < VEC; ++e) l += __builtin_amdgcn_exp2f(__builtin_fmaf(to_f(v[u].e[e]), kLog2e, -m2));
                }
            }
        }
        l = block_sum(l, sh);
    }

    // Output: y = exp2(x log2(e) - m2) / l.  An all -inf row has m2 = -inf: x log2(e) - m2
    // is then nan for every entry, and so is y.
    const float inv = 1.f / l;
    for (int i0 = tid; i0 < nv; i0 += kThreads * kUnroll) {
        V v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int i = i0 + u * kThreads;
            if (i < nv) v[u] = xr[i];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int i = i0 + u * kThreads;
            if (i >= nv) break;
            V w;
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                w.e[e] = (T)(__builtin_amdgcn_exp2f(__builtin_fmaf(to_f(v[u].e[e]), kLog2e, -m2)) * inv);
            yr[i] = w;
        }
    }
    if (lse && tid == 0) lse[r] = m2 == -INFINITY ? -INFINITY : (m2 + __builtin_amdgcn_logf(l)) * kLn2;
}

#define FA_SOFTMAX_INSTANTIATE(T, VEC)                                                   \
    template __global__ void softmax_kernel<T, true, VEC>(const T*, T*, float*, int);  \
    template __global__ void softmax_kernel<T, false, VEC>(const T*, T*, float*, int);
FA_SOFTMAX_INSTANTIATE(float, 4)
FA_SOFTMAX_INSTANTIATE(float, 1)
FA_SOFTMAX_INSTANTIATE(__bf16, 8)
FA_SOFTMAX_INSTANTIATE(__bf16, 1)
FA_SOFTMAX_INSTANTIATE(_Float16, 8)
FA_SOFTMAX_INSTANTIATE(_Float16, 1)

#if !defined(__HIP_DEVICE_COMPILE__)
namespace {
template <typename T>
const void* softmax_fn(bool online, bool vec)
{
    constexpr int VW = 16 / sizeof(T);
    if (online) return vec ? (const void*)&softmax_kernel<T, true, VW> : (const void*)&softmax_kernel<T, true, 1>;
    return vec ? (const void*)&softmax_kernel<T, false, VW> : (const void*)&softmax_kernel<T, false, 1>;
}
}  // namespace

hipError_t launch_softmax(const SoftmaxParams& p, hipStream_t stream)
{
    const int esize = p.dtype == 0 ? 4 : 2;
    const bool vec = ((long long)p.cols * esize) % 16 == 0;   // every row starts 16-byte aligned
    const void* fn = p.dtype == 0 ? softmax_fn<float>(p.online, vec)
                   : p.dtype == 1 ? softmax_fn<__bf16>(p.online, vec)
                                  : softmax_fn<_Float16>(p.online, vec);
    const void* x = p.x;
    void* y = p.y;
    float* lse = p.lse;
    int cols = p.cols;
    void* kargs[] = {(void*)&x, (void*)&y, (void*)&lse, (void*)&cols};
    return hipLaunchKernel(fn, dim3((unsigned)p.rows), dim3(256), kargs, 0, stream);
}
#endif

}  // namespace fa
