// gfx950 bf16 MFMA operand helpers shared by the forward and weight-gradient group GEMMs (internal).
//
// Lane layouts of v_mfma_f32_32x32x16_bf16 (checked on the device with a
// known-value run): lane l supplies A[m = l%32][k = 8*(l/32) + i] and
// B[k = 8*(l/32) + i][n = l%32] for i = 0..7; accumulator element v of lane l is
// C[m = 8*(v/4) + 4*(l/32) + v%4][n = l%32].
//
// ds_read_b64_tr_b16 (checked the same way): inside each group of 16 lanes,
// lane i receives, as element j (0..3), element i%4 of the 8-byte chunk whose
// address lane 4*j + i/4 supplied.  So if lane c of a group points at
// T[row0 + c/4][col0 + 4*(c%4)] of a row-major LDS tile T, lane i gets
// T[row0 + j][col0 + i], j = 0..3: a column of T, i.e. an MFMA operand whose
// reduction index runs along T's rows.
#pragma once

#include "moonep_common.h"

namespace moonep {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ bf16x4 lds_tr4(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_32x32x2_f32: lane l supplies A[m = l%32][k = l/32] and B[k = l/32][n = l%32]; the
// accumulator layout is that of the bf16 32x32 instruction (acc_row below).
__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// 64 lanes x 16 bytes: lane l copies 16 bytes from its global address g to LDS byte address
// lds_byte + 16*l (global_load_lds_dwordx4; lds_byte must be wave-uniform).  Issued from asm so
// the compiler does not wait for every outstanding load before each LDS read: the kernels wait on
// vmcnt themselves (wait_vmcnt) before a barrier.  The destination is an LDS byte address the
// caller computes as base + offset (lds_addr once per kernel), not a pointer: converting a pointer
// back to the LDS address space costs a null check per instruction, which measured 4-8% on the
// GEMMs' memory phases.
typedef __attribute__((address_space(3))) uint16_t lds_u16;
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_byte) : "memory", "m0");
}

// LDS byte address of (an element of) a shared array, wave-uniform.
__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_u16*)p);
}

// Waits until at most N of this wave's vector-memory operations are outstanding (they retire in order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that does not drain outstanding global loads (unlike __syncthreads, whose fence
// waits for every memory operation); LDS visibility of the DMA'd stage is ensured by wait_vmcnt
// first.  It does drain this wave's LDS reads, so no ring slot is refilled under a pending read.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Barrier that leaves this wave's LDS reads in flight: for the one after a ping-pong memory phase
// whose slot no wave refills before the next barrier.
__device__ __forceinline__ void plain_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Row of accumulator element v for lane l inside a 32x32 tile.
__device__ __forceinline__ int acc_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

}  // namespace moonep
