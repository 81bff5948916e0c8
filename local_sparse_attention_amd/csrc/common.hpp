// Shared device helpers: geometry, MFMA fragments, wave reductions (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace dsa3d {

typedef uint16_t u16;  // bf16 bits
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Queries are bucketed by window start; a bucket ("start blob") is 1 x 4 x 4
// start cells.  Key blobs for the dK/dV pass are 1 x 4 x 4 key positions.
constexpr int BLOB_Y = 4, BLOB_X = 4, BLOB_CELLS = BLOB_Y * BLOB_X;
constexpr int GROUP_Q = 16;   // queries per group (rows of a 16x16 MFMA tile)
constexpr int CHUNK = 32;     // keys (or queries) per streamed chunk
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

struct Geom {
  int F, Hp, Wp;     // token grid
  int kt, ky, kx;    // window
  int Lt, Ly, Lx;    // start lattice: G - k + 1 per axis
  int nby, nbx;      // start blobs per lattice row / column (Lt blobs along t)
  int H;             // heads (the row stride of [N][H][D] tensors)
  int h0, nh;        // heads an attention launch covers: h0 .. h0 + nh - 1
  int ph;            // heads the bucketing covers: 1 (offsets shared by every head) or nh
                     // (per-head offsets: the bucketing arrays hold one block per head,
                     // head-major, block hl for head h0 + hl)
  int N;             // tokens
  int nblobs;        // Lt * nby * nbx
  int keyspace;      // nblobs * BLOB_CELLS
};

// Sort key of a start cell: blob-major, then the cell inside its blob, so the
// queries of one blob are contiguous after sorting.
__device__ __forceinline__ int cell_key(const Geom& g, int st, int sy, int sx) {
  const int blob = (st * g.nby + (sy >> 2)) * g.nbx + (sx >> 2);
  return blob * BLOB_CELLS + ((sy & 3) << 2) + (sx & 3);
}

// ---- MFMA fragments -------------------------------------------------------
// A 16 x 16 tile with a 32-deep contraction.  Lane l owns row/column (l & 15) of
// its operand and the 8 contraction slots 8 * (l >> 4) + j, j = 0..7.  The
// result lane l holds C[4 * (l >> 4) + i][l & 15], i = 0..3.
// bf16: one v_mfma_f32_16x16x32_bf16.  fp32: eight v_mfma_f32_16x16x4_f32, the
// s-th taking slot j = s of every lane (slot order is free as long as both
// operands agree).
template <typename T> struct Frag;
template <> struct Frag<u16> { bf16x8_t v; };
template <> struct Frag<float> { float v[8]; };

__device__ __forceinline__ f32x4_t mma(const Frag<u16>& a, const Frag<u16>& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma(const Frag<float>& a, const Frag<float>& b, f32x4_t c) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], c, 0, 0, 0);
  return c;
}

// 8 contiguous elements (global or LDS), 16-byte aligned for bf16, 32 for fp32.
__device__ __forceinline__ void load_frag(Frag<u16>& f, const u16* p) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  __builtin_memcpy(&f.v, &u, 16);
}
__device__ __forceinline__ void load_frag(Frag<float>& f, const float* p) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
__device__ __forceinline__ void zero_frag(Frag<u16>& f) {
  const uint4 z = {0u, 0u, 0u, 0u};
  __builtin_memcpy(&f.v, &z, 16);
}
__device__ __forceinline__ void zero_frag(Frag<float>& f) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = 0.f;
}

// Fragment from 8 fp32 values (bf16: round to nearest even).
__device__ __forceinline__ void set_frag(Frag<u16>& f, const float* x) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = static_cast<__bf16>(x[j]);
}
__device__ __forceinline__ void set_frag(Frag<float>& f, const float* x) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = x[j];
}

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_f32(u16 b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float frag_elem(const Frag<u16>& f, int j) { return static_cast<float>(f.v[j]); }
__device__ __forceinline__ float frag_elem(const Frag<float>& f, int j) { return f.v[j]; }

// Gather one fragment column-wise from a row-major LDS tile: slot j takes row
// rows_j at column `col`.  Used where the contraction runs along tile rows.
template <typename T>
__device__ __forceinline__ void gather_frag(Frag<T>& f, const T* lds, int stride, const int* rows, int col);
template <>
__device__ __forceinline__ void gather_frag<u16>(Frag<u16>& f, const u16* lds, int stride, const int* rows, int col) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const u16 b = lds[rows[j] * stride + col];
    f.v[j] = __builtin_bit_cast(__bf16, b);
  }
}
template <>
__device__ __forceinline__ void gather_frag<float>(Frag<float>& f, const float* lds, int stride, const int* rows,
                                                   int col) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = lds[rows[j] * stride + col];
}

// Store 4 consecutive output elements from fp32.
__device__ __forceinline__ void store4(u16* p, float a, float b, float c, float d) {
  // round to nearest even, two values per conversion instruction
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  *reinterpret_cast<bf16x4*>(p) = __builtin_convertvector((f32x4_t{a, b, c, d}), bf16x4);
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// Calls f(std::integral_constant<int, I>{}) for I = B .. E-1: loop bodies whose index
// must be a compile-time constant (register-array subscripts) whatever the unroller
// decides.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// ---- wave helpers ---------------------------------------------------------
__device__ __forceinline__ float xor_max(float v, int m) { return fmaxf(v, __shfl_xor(v, m, 64)); }
__device__ __forceinline__ float xor_sum(float v, int m) { return v + __shfl_xor(v, m, 64); }

// Reductions over the 4 lanes that share (lane & 15).
__device__ __forceinline__ float quad_max(float v) { return xor_max(xor_max(v, 16), 32); }
__device__ __forceinline__ float quad_sum(float v) { return xor_sum(xor_sum(v, 16), 32); }

// The same reductions by row swaps (v_permlane16_swap / v_permlane32_swap: VALU
// instructions, no LDS round trip).  Every lane of the wave must be active.
__device__ __forceinline__ float2 swap_rows16(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return float2{__uint_as_float(a[0]), __uint_as_float(a[1])};  // rows (2r, 2r + 1), both lanes
}
__device__ __forceinline__ float2 swap_rows32(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return float2{__uint_as_float(a[0]), __uint_as_float(a[1])};  // halves (0, 1), both lanes
}
__device__ __forceinline__ float quad_max_rs(float v) {
  float2 a = swap_rows16(v);
  a = swap_rows32(fmaxf(a.x, a.y));
  return fmaxf(a.x, a.y);
}
__device__ __forceinline__ float quad_sum_rs(float v) {
  float2 a = swap_rows16(v);
  a = swap_rows32(a.x + a.y);
  return a.x + a.y;
}

// Min / max over lanes 0..15 of each 16-lane row (all rows hold the same data).
__device__ __forceinline__ int row16_min(int v) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) v = min(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ int row16_max(int v) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) v = max(v, __shfl_xor(v, m, 64));
  return v;
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// Make this wave's LDS writes visible to its other lanes (and keep the compiler
// from moving LDS accesses across).  Waves of these kernels never share LDS.
__device__ __forceinline__ void wave_lds_fence() {
  __asm__ __volatile__("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

}  // namespace dsa3d
