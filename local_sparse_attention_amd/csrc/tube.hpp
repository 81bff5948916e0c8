// Building blocks of the pipelined (frame-sweeping) kernels on gfx950: direct
// global->LDS loads that the compiler does not track, counted vmcnt waits, a
// barrier that leaves those loads in flight, the swizzled 128-byte-row tile
// layout and the XCD-aware workgroup order.
#pragma once

#include "common.hpp"

namespace dsa3d {

typedef short shortx4_t __attribute__((ext_vector_type(4)));
// Read-only tables (query order, start-cell boundaries) read at wave-uniform
// addresses: through the constant address space they become scalar loads, which
// keeps the vector memory counter free for the direct tile loads.
typedef const __attribute__((address_space(4))) int* cint_ptr;
typedef __attribute__((address_space(3))) shortx4_t lds_shortx4_t;

// byte offset of (row, byte-in-row) in a swizzled 128-byte-row tile
__device__ __forceinline__ int sw(int row, int byte) {
  return row * 128 + ((((byte >> 4) ^ row) & 7) << 4) + (byte & 15);
}

// One 16-byte direct global->LDS load per lane (global_load_lds_dwordx4): lane l's
// 16 bytes land at lds_base + 16 l, lds_base wave-uniform (it goes to M0).  Issued
// from inline asm so the compiler does not track it: left to itself it waits for
// every such load to finish before any LDS read that might alias, which would drain
// the prefetch ring.  Completion is awaited with explicit vmcnt waits (wait_vmcnt)
// before the barrier that publishes the data.
__device__ __forceinline__ void dma16(const void* gptr, const void* lds_base) {
  const unsigned m0 = (unsigned)(size_t)(const __attribute__((address_space(3))) char*)lds_base;
  __asm__ __volatile__("global_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(m0) : "memory");
}

// The same load with a wave-uniform 64-bit base (SGPRs) and a per-lane 32-bit byte
// offset: the address needs no vector arithmetic (the base of a frame goes in
// scalar registers, the lane's offset inside the frame is computed once).
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, const void* lds_base) {
  const unsigned m0 = (unsigned)(size_t)(const __attribute__((address_space(3))) char*)lds_base;
  __asm__ __volatile__("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
}

// Workgroup barrier for the pipelined loop: the LDS reads and writes of this wave
// are complete, the direct loads are covered by the preceding vmcnt wait.
// (__syncthreads() would also wait for every outstanding global access.)
__device__ __forceinline__ void lds_barrier() { __asm__ __volatile__("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// s_waitcnt vmcnt(n) for a run-time n (the immediate must be a constant).
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
#define DSA3D_VMCNT_CASE(k) \
  case k:                   \
    __asm__ __volatile__("s_waitcnt vmcnt(" #k ")" ::: "memory"); \
    break;
    DSA3D_VMCNT_CASE(0) DSA3D_VMCNT_CASE(1) DSA3D_VMCNT_CASE(2) DSA3D_VMCNT_CASE(3) DSA3D_VMCNT_CASE(4)
    DSA3D_VMCNT_CASE(5) DSA3D_VMCNT_CASE(6) DSA3D_VMCNT_CASE(7) DSA3D_VMCNT_CASE(8) DSA3D_VMCNT_CASE(9)
    DSA3D_VMCNT_CASE(10) DSA3D_VMCNT_CASE(11) DSA3D_VMCNT_CASE(12) DSA3D_VMCNT_CASE(13) DSA3D_VMCNT_CASE(14)
    DSA3D_VMCNT_CASE(15) DSA3D_VMCNT_CASE(16) DSA3D_VMCNT_CASE(17) DSA3D_VMCNT_CASE(18) DSA3D_VMCNT_CASE(19)
    DSA3D_VMCNT_CASE(20) DSA3D_VMCNT_CASE(21) DSA3D_VMCNT_CASE(22) DSA3D_VMCNT_CASE(23) DSA3D_VMCNT_CASE(24)
    DSA3D_VMCNT_CASE(25) DSA3D_VMCNT_CASE(26) DSA3D_VMCNT_CASE(27) DSA3D_VMCNT_CASE(28) DSA3D_VMCNT_CASE(29)
    DSA3D_VMCNT_CASE(30) DSA3D_VMCNT_CASE(31) DSA3D_VMCNT_CASE(32) DSA3D_VMCNT_CASE(33) DSA3D_VMCNT_CASE(34)
    DSA3D_VMCNT_CASE(35) DSA3D_VMCNT_CASE(36) DSA3D_VMCNT_CASE(37) DSA3D_VMCNT_CASE(38) DSA3D_VMCNT_CASE(39)
    DSA3D_VMCNT_CASE(40) DSA3D_VMCNT_CASE(41) DSA3D_VMCNT_CASE(42)
#undef DSA3D_VMCNT_CASE
    default:
      __asm__ __volatile__("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

// s_waitcnt vmcnt(N) for a compile-time N >= 0.  The field holds 6 bits; a larger
// N is clamped to 63, which only makes the wait stricter.
template <int N>
__device__ __forceinline__ void wait_vmcnt_c() {
  static_assert(N >= 0, "vmcnt counts are non-negative");
  __asm__ __volatile__("s_waitcnt vmcnt(%0)" ::"n"(N > 63 ? 63 : N) : "memory");
}

// Logical workgroup index from the hardware one: consecutive workgroups go round
// robin to the 8 XCDs, so hand each XCD a contiguous range of logical indices
// (neighbouring tubes then share that XCD's L2).
__device__ __forceinline__ int xcd_remap(int L, int total) {
  const int per = total >> 3, rem = total & 7, xcd = L & 7, slot = L >> 3;
  return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

// One 4-byte direct load per active lane (global_load_lds_dword): lane l's word
// lands at lds_base + 4 l.
__device__ __forceinline__ void dma4(const void* gptr, const void* lds_base) {
  const unsigned m0 = (unsigned)(size_t)(const __attribute__((address_space(3))) char*)lds_base;
  __asm__ __volatile__("global_load_lds_dword %0, off" ::"v"(gptr), "{m0}"(m0) : "memory");
}

}  // namespace dsa3d
