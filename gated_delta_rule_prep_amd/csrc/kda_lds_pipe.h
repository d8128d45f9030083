// kda_lds_pipe.h -- gfx950 helpers for streaming operands from HBM straight
// into LDS (buffer_load_dwordx4 ... lds), shared by the kernels that keep a
// ring of chunk slots in LDS.  Waits are explicit: the loads are inline
// assembly, so the compiler neither counts them nor waits for them itself.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBufWord3 = 0x00020000;   // raw buffer descriptor, dword 3 (gfx9 family)

// Raw buffer descriptor over `bytes` bytes at `base` (stride 0, no swizzle),
// made wave-uniform so that it can live in scalar registers.
__device__ __forceinline__ i32x4 buf_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a),
               __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(a >> 32) & 0xffff),
               __builtin_amdgcn_readfirstlane(bytes), kBufWord3};
}

// buffer_load_dwordx4 ... lds: lane i's 16 bytes at rsrc + voff land at LDS
// byte address lds + 16 i (lds wave-uniform).  Written as inline assembly so
// that the compiler does not treat it as an LDS store of unknown extent (it
// would then wait for every outstanding load before each LDS read); the waits
// are explicit in the kernels.  M0 carries the LDS address (one wait state
// between setting it and the load); it is declared clobbered, so the compiler
// sets it again wherever it needs it itself.
__device__ __forceinline__ void load_lds16(const i32x4& rsrc, uint32_t lds, int voff) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %2, 0 offen lds"
      :
      : "v"(voff), "s"(__builtin_amdgcn_readfirstlane((int)lds)), "s"(rsrc)
      : "memory", "m0");
}

// LDS byte address of a __shared__ object, as the 32-bit value M0 takes.
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)p);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Waits between the waves of a workgroup through flags in LDS instead of
// workgroup barriers.  A wait polls until its condition holds, sleeping
// 64 * SLEEP cycles between polls, and gives up after `limit` polls (2^21
// polls: about 0.06 s at SLEEP = 1 and 0.9 s at SLEEP = 16, at 2.4 GHz; it
// never happens unless a wave stops being scheduled for that long), so that
// every wave always finishes.  The kernels stop waiting after one wait gave up
// and report it in the status word; the limit comes with the launch.
template <int SLEEP = 1, typename Pred>
__device__ __forceinline__ bool spin_until(int limit, Pred pred) {
#pragma nounroll
  for (int k = 0; k < limit; ++k) {
    if (pred()) return true;
    __builtin_amdgcn_s_sleep(SLEEP);
  }
  return false;
}

// A flag in LDS (every lane reads the same word: the value is wave-uniform).
typedef __attribute__((address_space(3))) volatile int lds_vint;
__device__ __forceinline__ int lds_get(const int* p) {
  return __builtin_amdgcn_readfirstlane(*(const lds_vint*)(p));
}
__device__ __forceinline__ void lds_put(int* p, int v) { *(lds_vint*)(p) = v; }
// The smallest of four flags at a 16-byte aligned address, in one LDS read.
typedef int lds_i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) volatile lds_i32x4 lds_vi32x4;
__device__ __forceinline__ int lds_min4(const int* p) {
  const lds_i32x4 v = *(const lds_vi32x4*)(p);
  return __builtin_amdgcn_readfirstlane(min(min(v[0], v[1]), min(v[2], v[3])));
}

}  // namespace kda
