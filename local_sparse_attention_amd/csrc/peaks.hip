// Measured-peak microbenchmarks for the roofline report (include/dsa3d_peaks.h): an
// all-CU bf16 matrix-core loop and streaming HBM read / copy kernels.  They are timed
// by the caller with events on the stream it passes.
#include "dsa3d_peaks.h"
#include "common.hpp"

namespace dsa3d {

// Eight independent accumulator chains per wave keep the matrix core busy without
// waiting on a result; the operands stay in registers.  Each MFMA is written as
// one inline instruction with its accumulator tied to the result registers: left
// to the register allocator, this loop rotated the accumulators through shared
// registers with about six moves per MFMA, which halved the rate it measured.
// The compiler does not see the asm's latency, so the waits are explicit: before
// the first MFMAs (which start from a zero accumulator and read only a and b) and
// after the last, in a statement that takes the accumulators as operands so the
// reads below cannot move above it.
__global__ __launch_bounds__(256) void k_peak_mfma_bf16(float* __restrict__ out, int iters, float seed) {
  bf16x8_t a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = static_cast<__bf16>(seed + 0.001f * (threadIdx.x & 7) + 0.01f * j);
    b[j] = static_cast<__bf16>(seed - 0.002f * j);
  }
  f32x4_t c[8];
  __asm__ __volatile__("s_nop 7\n\ts_nop 7" ::"v"(a), "v"(b));
#pragma unroll
  for (int u = 0; u < 8; ++u) __asm__ __volatile__("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=v"(c[u]) : "v"(a), "v"(b));
  for (int i = 1; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      __asm__ __volatile__("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c[u]) : "v"(a), "v"(b));
  }
  __asm__ __volatile__("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                       : "+v"(c[0]), "+v"(c[1]), "+v"(c[2]), "+v"(c[3]), "+v"(c[4]), "+v"(c[5]), "+v"(c[6]), "+v"(c[7]));
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) s += c[u][0] + c[u][1] + c[u][2] + c[u][3];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// The same with the 32 x 32 x 16 shape (four chains of 16 accumulators).
typedef float f32x16_t __attribute__((ext_vector_type(16)));
__global__ __launch_bounds__(256) void k_peak_mfma32_bf16(float* __restrict__ out, int iters, float seed) {
  bf16x8_t a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = static_cast<__bf16>(seed + 0.001f * (threadIdx.x & 7) + 0.01f * j);
    b[j] = static_cast<__bf16>(seed - 0.002f * j);
  }
  f32x16_t c[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) c[u][i] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 4; ++u) c[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[u], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[u][i];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Grid-stride 16-byte loads; the xor of everything read is written once per thread.
__global__ __launch_bounds__(256) void k_peak_read(const uint4* __restrict__ src, size_t n16,
                                                   uint32_t* __restrict__ out) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const uint4 u = src[i];
    acc ^= u.x ^ u.y ^ u.z ^ u.w;
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

__global__ __launch_bounds__(256) void k_peak_copy(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                   size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace dsa3d

using namespace dsa3d;

extern "C" {

double dsa3d_peak_mfma_bf16(float* out, int blocks, int iters, hipStream_t stream) {
  if (!out || blocks < 1 || iters < 1) return -1.0;
  k_peak_mfma_bf16<<<blocks, 256, 0, stream>>>(out, iters, 0.5f);
  if (hipGetLastError() != hipSuccess) return -1.0;
  // 4 waves a block, 8 MFMAs of 16 x 16 x 32 (2 * 16 * 16 * 32 flops) per iteration
  return (double)blocks * 4 * iters * 8 * (2.0 * 16 * 16 * 32);
}

double dsa3d_peak_mfma32_bf16(float* out, int blocks, int iters, hipStream_t stream) {
  if (!out || blocks < 1 || iters < 1) return -1.0;
  k_peak_mfma32_bf16<<<blocks, 256, 0, stream>>>(out, iters, 0.5f);
  if (hipGetLastError() != hipSuccess) return -1.0;
  // 4 waves a block, 4 MFMAs of 32 x 32 x 16 per iteration
  return (double)blocks * 4 * iters * 4 * (2.0 * 32 * 32 * 16);
}

int dsa3d_peak_read(const void* src, size_t bytes, uint32_t* out, int blocks, hipStream_t stream) {
  if (!src || !out || blocks < 1 || (bytes & 15) || ((uintptr_t)src & 15)) return -1;
  k_peak_read<<<blocks, 256, 0, stream>>>((const uint4*)src, bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int dsa3d_peak_copy(const void* src, void* dst, size_t bytes, int blocks, hipStream_t stream) {
  if (!src || !dst || blocks < 1 || (bytes & 15) || (((uintptr_t)src | (uintptr_t)dst) & 15)) return -1;
  k_peak_copy<<<blocks, 256, 0, stream>>>((const uint4*)src, (uint4*)dst, bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
