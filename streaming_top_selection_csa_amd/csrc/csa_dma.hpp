// csa_dma.hpp -- direct global -> LDS loads issued as inline assembly.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace csa {

// Direct global -> LDS load of 16 (or 4) bytes per lane: lane l's bytes land
// at LDS byte lds + 16*l (4*l).  Issued as inline assembly: with the builtin
// in the function the compiler waits for every outstanding LDS read
// (lgkmcnt(0)) before each use of one, which serialises the MFMA operand
// reads that are meant to run ahead.  No register is written; the kernel
// waits for these loads itself (vmcnt, then a workgroup barrier) before
// reading the LDS they fill.  M0 holds the LDS address; an SALU write of M0
// needs one wait state before the load.  The scoring kernel uses them for fp8
// only: in the bf16 kernels (256 VGPRs) the 64-bit per-lane addresses they
// take cost more than the pipelined operand reads gain (same-device A/B at
// S=262,144: +2.3%; fp8 at S=1,048,576: -1.1%).  The sparse attention
// kernel uses them for its key and value rows.
__device__ __forceinline__ void dma16(const void *src, void *lds)
{
    const uint32_t m = uint32_t(uintptr_t((__attribute__((address_space(3))) void *)lds));
    __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                     :
                     : "v"(src), "s"(m)
                     : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void *src, void *lds)
{
    const uint32_t m = uint32_t(uintptr_t((__attribute__((address_space(3))) void *)lds));
    __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                     :
                     : "v"(src), "s"(m)
                     : "memory", "m0");
}

}  // namespace csa
