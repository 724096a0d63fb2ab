// Device helpers of the gfx950 GEMM tile engine shared by the bf16 and e4m3
// kernels: LDS swizzles, direct-to-LDS loads, explicit waits and barriers.
#pragma once

#include "common.hpp"

namespace tpmlp {
namespace engine {

// Keeps the interleaved order of one k-step slot (MFMA, its fragment read,
// its DMA instruction) from being rearranged by the scheduler.
#ifndef SCHED_PIN
#define SCHED_PIN() __builtin_amdgcn_sched_barrier(0)
#endif

// Position of 16-byte chunk c in P row r (CH chunks per row). 8 chunks
// (128-byte rows): c ^ ((r & 7) ^ ((r >> 3) & 1)). 4 chunks (64-byte rows):
// c ^ (((r >> 1) ^ (r >> 3)) & 3). Either way a ds_read_b128 of 32
// consecutive rows at one chunk spreads each 8 (or 16) consecutive lanes over
// distinct 16-byte bank groups of a 32-bank (or 64-bank) LDS.
template <int CH>
__device__ __forceinline__ int swz_p(int r, int c) {
  if constexpr (CH == 8) return c ^ ((r & 7) ^ ((r >> 3) & 1));
  else return c ^ (((r >> 1) ^ (r >> 3)) & 3);
}

// LDS byte address of a __shared__ pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) void*)p);
}

// 16 bytes from base + off (per lane) into LDS at lds + 16·lane, where `lds`
// and `base` are wave-uniform. Issued through asm so that the only waits on
// it are the explicit s_waitcnt below (the compiler cannot tell which LDS
// stage a DMA writes and would otherwise wait for it before every ds_read).
// M0 is used by nothing else in these kernels. GFX9 needs one wait state
// between an SALU write of M0 and an LDS DMA instruction that reads it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(off), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(VM) expcnt(7) lgkmcnt(LGKM), gfx9 encoding (vmcnt in bits 3:0 and 15:14).
template <int VM, int LGKM>
__device__ __forceinline__ void waitcnt() {
  static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "waitcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4) | (LGKM << 8));
}

// Wait until at most `slices` DMA slices of R instructions each are in flight
// (and every LDS read has returned).
template <int R, int MAXS>
__device__ __forceinline__ void wait_dma(int slices) {
  static_assert(MAXS <= 3, "extend wait_dma");
  if (MAXS >= 3 && slices >= 3) waitcnt<(MAXS >= 3 ? 3 * R : 0), 0>();
  else if (MAXS >= 2 && slices == 2) waitcnt<(MAXS >= 2 ? 2 * R : 0), 0>();
  else if (MAXS >= 1 && slices == 1) waitcnt<R, 0>();
  else waitcnt<0, 0>();
}

// Workgroup barrier that the compiler may not move memory operations across;
// the hardware waits are issued explicitly by the caller.
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Clock stamps of one workgroup, taken only when a measurement call passes a
// stamps array (else the kernel is unchanged but for one uniform branch at
// each end): the shader-clock counter (s_memtime) and the constant 100 MHz
// counter (s_memrealtime) when the workgroup starts, and again once every
// wave's stores have completed. Workgroup w writes
// stamps[4w .. 4w+3] = {shader start, constant start, shader end, constant end},
// so Δshader / Δconstant · 100 MHz is the shader clock the workgroup ran at.
struct ClockStamp {
  uint64_t shader0 = 0, wall0 = 0;
  __device__ __forceinline__ explicit ClockStamp(const uint64_t* stamps) {
    if (stamps != nullptr) {
      shader0 = __builtin_amdgcn_s_memtime();
      wall0 = __builtin_amdgcn_s_memrealtime();
    }
  }
  __device__ __forceinline__ void finish(uint64_t* stamps) const {
    if (stamps == nullptr) return;
    waitcnt<0, 0>();
    barrier();
    if (threadIdx.x == 0) {
      const uint64_t shader1 = __builtin_amdgcn_s_memtime();
      const uint64_t wall1 = __builtin_amdgcn_s_memrealtime();
      typedef __attribute__((ext_vector_type(4))) unsigned long long u64x4;
      const u64x4 v = {shader0, wall0, shader1, wall1};
      *reinterpret_cast<u64x4*>(stamps + 4 * (uint64_t)blockIdx.x) = v;
    }
  }
};

}  // namespace engine
}  // namespace tpmlp
