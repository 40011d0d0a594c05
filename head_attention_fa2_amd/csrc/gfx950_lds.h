// LDS tile-pipeline primitives shared by the gfx950 kernels of this library: the
// HBM -> LDS copy (global_load_lds_dwordx4) with explicit m0, the vmcnt wait that
// completes those copies, and a workgroup barrier without the all-loads fence of
// __syncthreads().
#ifndef GFX950_LDS_H_
#define GFX950_LDS_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gfx950 {

// 32-bit LDS address of a pointer into __shared__ memory.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One 16-byte-per-lane copy HBM -> LDS (global_load_lds_dwordx4): lane l reads
// sbase + voff and the data lands at LDS address lds + 16*l.  Issued as inline asm so
// that the compiler does not track it: the only waits on these copies are the explicit
// vmcnt waits of the tile pipeline, which order them against the LDS reads.
// A load with LDS=1 reads m0 and needs one wait state after an SALU write of m0 (CDNA
// ISA, manually inserted wait states); the compiler cannot see inside the asm block, so
// the s_nop is written here.
__device__ __forceinline__ void copy_to_lds(const void* sbase, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}

// As copy_to_lds, with a full 64-bit source address per lane (gathers from a block pool).
__device__ __forceinline__ void copy_to_lds_addr(const void* src, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds)
               : "memory", "m0");
}

// A wavefront-uniform pointer the compiler cannot prove uniform, moved to SGPRs (the
// scalar base of copy_to_lds must be in SGPRs).
__device__ __forceinline__ const char* uniform_ptr(const char* ptr) {
  const uint64_t a = (uint64_t)(uintptr_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Wait until at most N vector-memory operations of this wavefront are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Workgroup barrier for the LDS tile pipeline.  __syncthreads() would also wait for
// every outstanding global load, including the prefetch of the next tile; here each
// wavefront has already waited (vmcnt) for the loads of the tile about to be read, and
// its LDS reads of the previous tile were consumed before it arrives, so only the
// execution barrier is needed.  The empty asm statements keep the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void tile_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

}  // namespace gfx950

#endif  // GFX950_LDS_H_
