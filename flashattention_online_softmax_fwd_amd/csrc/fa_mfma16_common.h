// fa_mfma16_common.h -- device helpers shared by the 16-bit (bf16 / fp16) forward and
// backward kernels for gfx950: element-type traits, the LDS tile layout, lane-half
// reductions and the tile barrier.  Internal; not installed.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

// The element type's MFMA, pair dot product and vector types.  fp16's largest value,
// 65504, is never approached: P stays below 2^8 in the forward (its lazy rescale) and
// at most 1 in the backward, and scores and accumulators are fp32 until the final
// rounding.
template <typename E>
struct Elem;
template <>
struct Elem<__bf16> {
    typedef __attribute__((ext_vector_type(8))) __bf16 x8;
    typedef __attribute__((ext_vector_type(4))) __bf16 x4;
    typedef __attribute__((ext_vector_type(2))) __bf16 x2;
    static __device__ __forceinline__ __attribute__((ext_vector_type(16))) float
    mfma(x8 a, x8 b, __attribute__((ext_vector_type(16))) float c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float dot2(x2 a, x2 b, float c)
    {
        return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
    }
};
template <>
struct Elem<_Float16> {
    typedef __attribute__((ext_vector_type(8))) _Float16 x8;
    typedef __attribute__((ext_vector_type(4))) _Float16 x4;
    typedef __attribute__((ext_vector_type(2))) _Float16 x2;
    static __device__ __forceinline__ __attribute__((ext_vector_type(16))) float
    mfma(x8 a, x8 b, __attribute__((ext_vector_type(16))) float c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float dot2(x2 a, x2 b, float c)
    {
        return __builtin_amdgcn_fdot2(a, b, c, false);
    }
};
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kRescaleSlack = 8.0f;   // log2 units: P may grow to 2^8 before m moves

// XOR mask for the 16-byte chunks of K/V tile row r.  Chosen so that both LDS read
// patterns are free of bank conflicts: 16 consecutive rows at one logical chunk
// (the K operand) and 4 consecutive rows x 4 consecutive chunks (the V operand).
template <int D>
__device__ __forceinline__ int swz(int r)
{
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);   // D == 64: 8 chunks, 2 rows per bank row
}

// Reductions over the two lane halves, which hold the same query row.
__device__ __forceinline__ float lane_half_max(float x)
{
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

__device__ __forceinline__ float lane_half_sum(float x)
{
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// The tile barrier.  Loads that write LDS directly (buffer_load ... lds) count in
// vmcnt, and a workgroup barrier does not by itself wait for them, so each wave
// first waits for its own tile loads to land; after the barrier every wave's loads
// have, and the whole tile is visible.
__device__ __forceinline__ void tile_barrier()
{
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), expcnt and lgkmcnt unconstrained
    __syncthreads();
}

// Workgroup order over the 8 XCDs, which receive blocks round-robin (block b runs on
// XCD b % 8).  Each XCD gets a contiguous run of the units (heads) so that its L2 holds
// few of them at a time, and walks them two at a time, the tiles of the pair
// interleaved: (u0, t0), (u1, t0), (u0, t1), (u1, t1), ...  Under causal masking the
// callers map t = 0 to the longest tile, so all long tiles of a pair start before its
// short ones and the short tiles of the last pair fill the tail of the grid.  Units
// per XCD (units / 8, units a multiple of 8) odd: one unit at a time.
__device__ __forceinline__ void xcd_order(int bid, int units, int ntiles, int& u, int& t)
{
    const int xcd = bid & 7;
    const int k = bid >> 3;
    const int per = units >> 3;
    if ((per & 1) == 0) {
        const int pair = k / (2 * ntiles);
        const int r = k - pair * 2 * ntiles;
        u = xcd * per + 2 * pair + (r & 1);
        t = r >> 1;
    } else {
        const int q = k / ntiles;
        u = xcd * per + q;
        t = k - q * ntiles;
    }
}

template <bool V>
struct Flag {
    static constexpr bool value = V;
};

template <int V>
struct Int {
    static constexpr int value = V;
};

}  // namespace fa
