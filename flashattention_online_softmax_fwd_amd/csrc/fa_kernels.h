// fa_kernels.h -- internal interface between the C ABI (fa_host.cpp) and the
// gfx950 kernels.  Not installed; the public interface is include/fa.h.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

// Arguments shared by every forward kernel.  Sizes were validated on the host.
struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;           // [B][Hq][N][d] in the input dtype; split kernels: float [splits][B][Hq][N][d]
    float* lse;        // [B][Hq][N]; split kernels: [splits][B][Hq][N]
    int B, Hq, Hkv, N; // N: query rows per head
    int Nk;            // keys per head (== N for the square forward)
    int q_off;         // Nk - N: query i sits at key position i + q_off (causal offset)
    int chunk;         // keys per split, a multiple of 64 (split kernels)
    int splits;        // number of key splits (1 for the square forward)
    int group;       // Hq / Hkv: query heads per K/V head
    int n_qtiles;    // ceil(N / block_m)
    float scale_log2;  // scale * log2(e): scores go straight to the exp2 domain
    int xcd_map;       // 1: block order spreads whole heads over the 8 XCDs (set by the launcher)
    int walk;          // 1: each workgroup walks pairs of query tiles (set by the launcher)
    // Square 16-bit forward only, else null: per wave {real-time start, real-time end,
    // shader-cycle start, shader-cycle end}, at [(block * waves + wave) * 4].
    unsigned long long* stamps;
};

using Launcher = hipError_t (*)(const FwdParams&, hipStream_t);
// Compute units of the current device (cached per device), 0 when there is none.
int device_cus();
// Workgroups of a launch that walks several query tiles per workgroup, or 0 for one
// workgroup per query tile (units = B * Hq, ntiles = query tiles per head).
using Blocks = long long (*)(long long units, long long ntiles, int causal);

// One compiled instantiation.
struct KernelEntry {
    int dtype;      // FA_DTYPE_*
    int d;
    int block_m;
    int block_n;
    int causal;
    Launcher launch;
    int waves;      // waves per workgroup; 0: block_m / 32 (one 32-row block per wave)
    Blocks blocks;  // null: one workgroup per query tile
};

// Tables defined by the kernel translation units.
extern const KernelEntry kBf16Kernels[];
extern const int kNumBf16Kernels;
extern const KernelEntry kF16Kernels[];
extern const int kNumF16Kernels;
extern const KernelEntry kF32Kernels[];
extern const int kNumF32Kernels;
// The 64-rows-per-wave forward (fa_fwd_w64.hip): d = 128, 128 x 64 tiles (2 waves) and
// 256 x 64 tiles (4 waves); the default for 16-bit inputs at d = 128 comes first.
extern const KernelEntry kBf16W64Kernels[];
extern const KernelEntry kF16W64Kernels[];
constexpr int kNumW64Kernels = 8;
// Split-KV partial-state kernels (16-bit inputs, float partial outputs).
extern const KernelEntry kBf16SplitKernels[];
extern const int kNumBf16SplitKernels;
extern const KernelEntry kF16SplitKernels[];
extern const int kNumF16SplitKernels;

// Merge of partial states: o_part [splits][rows][d], lse_part [splits][rows] (float).
struct MergeParams {
    const float* o_part;
    const float* lse_part;
    void* o;           // [rows][d], float, bf16 or fp16
    float* lse;        // [rows]
    long long rows;
    int splits;
};
hipError_t launch_merge(const MergeParams& p, int d, int out_dtype, hipStream_t stream);   // FA_DTYPE_*

// Backward pass (16-bit inputs): dq, dk, dv from q, k, v, o, do and the forward's lse.
struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;   // dO [B][Hq][N][d]
    const float* lse;   // [B][Hq][N], natural log
    float* delta;       // [B][Hq][N]: rowsum(dO * O), written by the dq kernel
    void* dq;           // [B][Hq][N][d]
    void* dk;           // [B][Hkv][N][d]
    void* dv;           // [B][Hkv][N][d]
    int B, Hq, Hkv, N;
    int group;          // Hq / Hkv
    float scale;        // multiplies q.k
    int xcd_map;        // set by the launchers
    int splits;         // workgroups sharing each key tile's query tiles (1: dk, dv written directly)
    float* dkv_part;    // splits > 1: [2][splits][B][Hkv][N][d] fp32 partial dK, then dV
};
// Enqueues the kernels (dq with D, then dk/dv, then the reduce when splits > 1) on the
// stream; d is 64 or 128,
// dtype FA_DTYPE_BF16 or FA_DTYPE_F16.
hipError_t launch_bwd(const BwdParams& p, int d, int dtype, int causal, hipStream_t stream);

// The library's own dK/dV partial workspace for fa_bwd_split_noalloc: a static device
// array of kBwdScratchBytes on each GPU.  *ptr receives its device address on the
// stream's device (looked up once per device).
constexpr unsigned long long kBwdScratchBytes = 128ULL << 20;
hipError_t bwd_scratch(hipStream_t stream, float** ptr);

// Row softmax: y [rows][cols] = softmax of each row of x, lse [rows] (optional).
struct SoftmaxParams {
    const void* x;
    void* y;
    float* lse;        // may be null
    long long rows;    // rows of this launch, <= 2^23 (one workgroup per row)
    int cols;
    int dtype;         // FA_DTYPE_*: x and y
    bool online;       // true: running max and sum in one pass; false: three passes
};
hipError_t launch_softmax(const SoftmaxParams& p, hipStream_t stream);

}  // namespace fa
