// Optional per-workgroup timeline of the main matmul kernel, for
// measurement builds only. With W8A8_TIMELINE defined (build.py compiles
// scaled_mm.hip once more that way and links libw8a8_timeline.so beside the
// library), thread 0 of every workgroup records two clocks at the kernel's
// phase boundaries; without it W8A8_STAMP expands to nothing and the
// library's code is unchanged.
//
// Record of workgroup b (kSlots 64-bit words at b * kSlots):
//   [0, 8)   s_memrealtime at stamp i (the 100 MHz constant clock),
//   [8, 15)  s_memtime at stamp i (shader clock cycles),
//   15       XCC id << 32 | HW_ID register (which die and CU ran it).
// Stamps: 0 kernel entry; 1 own rows quantized (fused form); 2 rows
// published; 3 producers' rows seen; 4 prologue done (first stages in LDS
// and registers); 5 K loop done; 6 epilogue's stores issued.
// Each launch overwrites the records of its workgroups; only workgroups
// below kMaxBlocks record. One array per translation unit: the int8
// kernels' (scaled_mm.hip) is the one w8a8_timeline_read copies out.
#pragma once

#ifdef W8A8_TIMELINE
#include <hip/hip_runtime.h>

namespace w8a8 {
namespace timeline {

constexpr int kSlots = 16;
constexpr int kMaxBlocks = 16384;
static __device__ unsigned long long g_stamp[kMaxBlocks * kSlots];

// hwreg(HW_REG_XCC_ID, 0, 16) and hwreg(HW_REG_HW_ID, 0, 32) in s_getreg's
// encoding: id | offset << 6 | (size - 1) << 11.
constexpr int kXccIdReg = 20 | (15 << 11);
constexpr int kHwIdReg = 4 | (31 << 11);

__device__ __forceinline__ void stamp(int i)
{
    __builtin_amdgcn_sched_barrier(0);
    if (threadIdx.x == 0 && blockIdx.x < (unsigned)kMaxBlocks) {
        unsigned long long *rec = g_stamp + (size_t)blockIdx.x * kSlots;
        rec[i] = __builtin_amdgcn_s_memrealtime();
        rec[8 + i] = __builtin_amdgcn_s_memtime();
        if (i == 0)
            rec[15] = (unsigned long long)(unsigned)__builtin_amdgcn_s_getreg(kXccIdReg) << 32 |
                      (unsigned)__builtin_amdgcn_s_getreg(kHwIdReg);
    }
    __builtin_amdgcn_sched_barrier(0);
}

}  // namespace timeline
}  // namespace w8a8

#define W8A8_STAMP(i) ::w8a8::timeline::stamp(i)
#else
#define W8A8_STAMP(i) ((void)0)
#endif
