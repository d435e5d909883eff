// Stand-in for <hip/hip_runtime.h> used ONLY by the CPU emulation of the
// kernels (tests/emu/emu.cpp).  It lets the unmodified kernel headers compile
// as host C++: every lane becomes a std::thread, __shared__ memory becomes a
// static array shared by the workgroup's threads, and __syncthreads() is a
// real barrier.  Built with AddressSanitizer and UBSan, an out-of-bounds or
// misaligned access in the kernel logic becomes a CPU error report.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <cmath>
using std::fmax;
using std::fmin;
using std::rint;
using std::sqrt;

#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(...)
#define __shared__ static
#define __builtin_amdgcn_readfirstlane(x) (x)

struct EmuDim3 {
    unsigned x, y, z;
};
extern thread_local EmuDim3 threadIdx;
extern thread_local EmuDim3 blockIdx;
extern EmuDim3 blockDim;
extern EmuDim3 gridDim;
void __syncthreads();
// Wavefront vote: every lane of the 64-lane wavefront must call it together
// (the emulator meets them at a per-wavefront barrier).
unsigned long long __ballot(int pred);
// Wavefront shuffle: lane `src` of the caller's 64-lane wavefront (same
// meeting rule as __ballot).
double __shfl(double var, int src);
// Butterfly shuffle: var of lane (lane ^ mask) of the caller's wavefront.
int __shfl_xor(int var, int mask);
// DPP move (row_mask and bank_mask all set; the controls the kernels use:
// quad_perm, row_ror, row_mirror, row_half_mirror) and ds_swizzle in bit
// mode, as the GCN/CDNA ISA defines them, over the caller's wavefront.
int __builtin_amdgcn_update_dpp(int old, int src, int ctrl, int row_mask, int bank_mask,
                                bool bound_ctrl);
int __builtin_amdgcn_mov_dpp(int src, int ctrl, int row_mask, int bank_mask, bool bound_ctrl);
int __builtin_amdgcn_ds_swizzle(int src, int pattern);
inline int __popcll(unsigned long long x) { return __builtin_popcountll(x); }
template <typename T>
inline T min(T a, T b) { return b < a ? b : a; }
template <typename T>
inline T max(T a, T b) { return a < b ? b : a; }
