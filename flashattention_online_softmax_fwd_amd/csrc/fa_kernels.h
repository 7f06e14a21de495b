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
    void* o;
    float* lse;
    int B, Hq, Hkv, N;
    int group;       // Hq / Hkv: query heads per K/V head
    int n_qtiles;    // ceil(N / block_m)
    float scale_log2;  // scale * log2(e): scores go straight to the exp2 domain
    int xcd_map;       // 1: block order spreads whole heads over the 8 XCDs (set by the launcher)
};

using Launcher = hipError_t (*)(const FwdParams&, hipStream_t);

// One compiled instantiation.
struct KernelEntry {
    int dtype;      // FA_DTYPE_*
    int d;
    int block_m;
    int block_n;
    int causal;
    Launcher launch;
};

// Tables defined by the kernel translation units.
extern const KernelEntry kBf16Kernels[];
extern const int kNumBf16Kernels;
extern const KernelEntry kF32Kernels[];
extern const int kNumF32Kernels;

}  // namespace fa
