// LDS stage ring fed by direct global->LDS loads (gfx950), shared by the
// grouped GEMM kernels.
//
// A stage holds rows of 128 bytes (64 bf16 or 128 fp8 reduction elements):
// full cache lines, which matters -- streaming weight rows from HBM 64 bytes
// at a time (half lines) runs at ~3.6 TB/s on MI355X, whole 128-byte lines
// at ~6.3 TB/s.  Each wave instruction moves 8 rows x 128 bytes = 1 KB: lane
// i fetches 16 bytes and the hardware writes them to LDS at m0 + 16 i.  The
// eight 16-byte chunks of row r are stored at slot ring_slot(r, q), so 16
// lanes reading one chunk of 16 consecutive rows touch 16 distinct 16-byte
// slots of a 256-byte window (no bank conflicts).
#pragma once

#include "common.h"

namespace moe {

typedef __attribute__((address_space(3))) void lds_ptr_t;

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(lds_ptr_t *)p;
}

__device__ __forceinline__ int ring_slot(int r, int q) { return q ^ ((r >> 1) & 7); }

// Direct global->LDS load of 16 bytes per lane to LDS byte address
// lds_byte_addr + 16 * lane.  Written as inline assembly so the compiler's
// wait-count insertion does not track it (a tracked load into one ring slot
// makes the compiler drain every outstanding load before reads of another
// slot); completion is awaited explicitly with wait_vm().  m0 is written
// here and used by nothing else in these kernels; the s_nop covers the
// m0-write -> LDS-DMA hazard.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_byte_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_byte_addr)
               : "memory");
}

// The same load with the non-temporal hint, for weight rows read once.  On
// MI355X it raised the gate/up kernel over 401 tokens (about nine rows per
// expert) from ~5.75 to ~6.35 TB/s of weights.
__device__ __forceinline__ void dma16_nt(const void *src, uint32_t lds_byte_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(src), "s"(lds_byte_addr)
               : "memory");
}

// Workgroup barrier without a memory fence.  __syncthreads() would make the
// compiler drain every outstanding vector-memory operation first (the
// direct loads count as LDS writes), emptying the ring at every stage.  Each
// wave instead waits for its own loads of the stage about to be read
// (wait_vm) and then meets the others here; the "memory" clobber keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vm_imm() {
  // s_waitcnt: vmcnt in bits 3:0 and 15:14, expcnt (7) and lgkmcnt (15) left open
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Wait until at most n of this wave's vector-memory operations are
// outstanding (n > 32 waits for all of them).  n is wave-uniform.
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
#define MOE_WAIT_CASE(N) \
  case N:                \
    wait_vm_imm<N>();    \
    break;
    MOE_WAIT_CASE(1) MOE_WAIT_CASE(2) MOE_WAIT_CASE(3) MOE_WAIT_CASE(4) MOE_WAIT_CASE(5)
    MOE_WAIT_CASE(6) MOE_WAIT_CASE(7) MOE_WAIT_CASE(8) MOE_WAIT_CASE(9) MOE_WAIT_CASE(10)
    MOE_WAIT_CASE(11) MOE_WAIT_CASE(12) MOE_WAIT_CASE(13) MOE_WAIT_CASE(14) MOE_WAIT_CASE(15)
    MOE_WAIT_CASE(16) MOE_WAIT_CASE(17) MOE_WAIT_CASE(18) MOE_WAIT_CASE(19) MOE_WAIT_CASE(20)
    MOE_WAIT_CASE(21) MOE_WAIT_CASE(22) MOE_WAIT_CASE(23) MOE_WAIT_CASE(24) MOE_WAIT_CASE(25)
    MOE_WAIT_CASE(26) MOE_WAIT_CASE(27) MOE_WAIT_CASE(28) MOE_WAIT_CASE(29) MOE_WAIT_CASE(30)
    MOE_WAIT_CASE(31) MOE_WAIT_CASE(32)
#undef MOE_WAIT_CASE
    default:
      wait_vm_imm<0>();
      break;
  }
}

}  // namespace moe
