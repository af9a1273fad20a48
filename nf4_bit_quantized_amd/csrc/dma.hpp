// Copies of global memory straight into LDS (buffer_load_dwordx4 ... lds) and
// the waits that go with them, shared by the streaming kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {
namespace dma {

typedef __attribute__((address_space(3))) void lds_void_t;

// A buffer offset no range here reaches (ranges are capped below 2^31):
// loads, and copies into LDS, read zero.
constexpr uint32_t kOob = 0x80000000u;

// Buffer resource (base, stride 0, byte range capped below 2^31) as four
// dwords, for the copies below.
typedef int v4i_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4i_t rsrc(const void* p, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const int32_t n = bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0 : (int32_t)bytes;
  return v4i_t{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xFFFFu), n, 0x00020000};
}

// Wait until at most N of this wave's vector-memory operations are in flight
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// 16-byte copy of global memory (buffer offset voff) to LDS: lane l lands at
// LDS byte address dst + 16 l.  Written as inline asm so that the compiler does
// not track the copy as an LDS store: its own bookkeeping would wait for every
// copy in flight before each LDS read it cannot prove disjoint (draining the
// prefetch); the kernels wait for exactly the copies they read instead, and
// issue no compiler-visible vector-memory operation while copies are in
// flight, so that the counts they wait on are exact.  The kernels that
// include this file use M0 for nothing else (checked in the generated code).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16(v4i_t r, uint32_t voff, uint32_t dst) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(dst);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(l), "v"(voff), "s"(r)
               : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace dma
}  // namespace qlora

// LDS byte address of a __shared__ array (apply to the array itself).
#define LDS_ADDR(arr) ((uint32_t)reinterpret_cast<uintptr_t>((qlora::dma::lds_void_t*)(arr)))
