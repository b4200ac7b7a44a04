// dma.h -- operands copied from global memory straight into shared memory
// (gfx950 global_load_lds_dwordx4) and the waits and barrier that go with
// them: a step waits for its own requests while the next steps' stay in
// flight.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace moe {

typedef __attribute__((address_space(3))) void lds_t;

// 16 bytes per lane from global memory into shared memory at base + 16 lane.
__device__ __forceinline__ void dma16(const void *g, int8_t *base) {
  __builtin_amdgcn_global_load_lds(g, (lds_t *)base, 16, 0, 0);
}

// Wait until at most N of this wave's vector-memory operations are in
// flight.  s_waitcnt fields: vmcnt bits 3:0, expcnt 6:4 and lgkmcnt 11:8
// (expcnt at its maximum; lgkmcnt at its maximum, or 0 with LDS0: every
// shared-memory read of the wave has returned).
template <int N, bool LDS0 = false>
__device__ __forceinline__ void wait_vm_at_most() {
  static_assert(N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((LDS0 ? 0x0070 : 0x0F70) | N);
}

// The workgroup barrier of a step: this wave's pieces of the step are in
// (the next step's may stay in flight) and its shared-memory reads of the
// previous step have returned; then every wave's are.  The compiler may
// move no memory access across it (the empty asm) and the scheduler no
// instruction (sched_barrier); no fence, which would wait for the requests
// in flight as well.
template <int PIECES>
__device__ __forceinline__ void dma_step_barrier() {
  asm volatile("" ::: "memory");
  wait_vm_at_most<PIECES, true>();
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// A workgroup barrier after this wave's shared-memory accesses have
// completed, leaving its global-to-shared requests in flight (vmcnt at its
// maximum: bits 3:0 and 15:14 all set).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

}  // namespace moe
