// Device-side helpers shared by the kernels of libeagle_verify: words that
// one workgroup writes for another on a different XCD.
//
// The L2 caches of the XCDs are not coherent with each other, and
// agent-scope release/acquire would write back / invalidate a whole L2 per
// operation.  Instead every word exchanged between workgroups goes through
// system-scope relaxed atomics, which bypass the non-coherent caches, and
// ordering comes from waiting for the stores to complete before signalling.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ev {

__device__ __forceinline__ uint64_t ld_u64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ double ld_f64(const double* p) {
  return __builtin_bit_cast(double, ld_u64(reinterpret_cast<const uint64_t*>(p)));
}
__device__ __forceinline__ void st_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void st_f64(double* p, double v) { st_u64(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, v)); }

// this thread's earlier stores have completed (been acknowledged by the
// coherent memory side) before anything that follows is issued
__device__ __forceinline__ void stores_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// later loads are not moved above the poll that allowed them
__device__ __forceinline__ void loads_after() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ uint64_t poll(const uint64_t* w) {
  return __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Diagnostic timeline: thread 0 of the workgroup records the constant-rate
// real-time counter (100 MHz) in word k of the workgroup's slots (32 words
// per workgroup), or a value; nothing when no timeline buffer was given.
__device__ __forceinline__ void stamp(uint64_t* stamps, int k) {
  if (stamps && threadIdx.x == 0) stamps[static_cast<int64_t>(blockIdx.x) * 32 + k] = __builtin_amdgcn_s_memrealtime();
}
__device__ __forceinline__ void stamp_value(uint64_t* stamps, int k, uint64_t v) {
  if (stamps && threadIdx.x == 0) stamps[static_cast<int64_t>(blockIdx.x) * 32 + k] = v;
}

// where the workgroup runs: the hardware-id register (shader engine, CU,
// SIMD, wave slot) in the low word, the XCD's index in the high word
__device__ __forceinline__ uint64_t placement() {
  const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);     // HW_ID, all 32 bits
  const uint32_t xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);   // XCC_ID, all 32 bits
  return (static_cast<uint64_t>(xcc) << 32) | hw;
}

__device__ __forceinline__ void publish(uint64_t* w, uint64_t v) {
  stores_done();
  __hip_atomic_store(w, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

}  // namespace ev
