// The offset predictor's pointwise layer (MegaSlide-DiT, section "3D Deformable Slide
// Attention": offsets come from a depthwise 3-D convolution followed by a linear layer,
// pointwise convolutions in the implementation paragraph): y = x W^T + b per token.
//
// k_gemm_nt  C[M][N] = A[M][K] B[N][K]^T (+ bias[N]) on the matrix cores: 128 x 128
//            block tiles, 32-deep K steps staged through LDS (the next tile's global
//            loads issued before this tile's products), four waves of 64 x 64, each as
//            2 x 2 tiles of v_mfma_f32_32x32x16_bf16 (fp32 inputs: v_mfma_f32_32x32x2_f32).
//            The 32 x 32 x 16 shape sustains about twice the bf16 rate of 16 x 16 x 32 on
//            gfx950.
// Backward: dx = dy W and dW = dy^T x are the same kernel on transposed copies (k_transpose,
// also the fp32 -> bf16 rounding of dy on the bf16 path); db is a two-stage column sum
// in a fixed order.
#include "dsa3d.h"
#include "internal.hpp"

namespace dsa3d {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int GB = 128, GK = 32;

template <typename T> struct GemmT;
template <> struct GemmT<u16> { static constexpr int EV = 8, PAD = 8; };
template <> struct GemmT<float> { static constexpr int EV = 4, PAD = 4; };

__device__ __forceinline__ float cvt_in(u16 v) { return to_f32(v); }
__device__ __forceinline__ float cvt_in(float v) { return v; }
template <typename T> __device__ __forceinline__ T cvt_out(float v);
template <> __device__ __forceinline__ float cvt_out<float>(float v) { return v; }
template <> __device__ __forceinline__ u16 cvt_out<u16>(float v) {
  return __builtin_bit_cast(u16, static_cast<__bf16>(v));
}

// One 16-byte chunk (EV elements) of row `row`, columns k .. k+EV-1 of a [rows][K]
// matrix, zero outside; vec: K is a multiple of EV (whole chunks, 16-byte aligned rows).
template <typename T>
__device__ __forceinline__ uint4 load_chunk(const T* p, int rows, int K, int row, int k, bool vec) {
  constexpr int EV = GemmT<T>::EV;
  uint4 u = {0u, 0u, 0u, 0u};
  if (row >= rows) return u;
  if (vec) {
    if (k < K) u = *reinterpret_cast<const uint4*>(p + (size_t)row * K + k);
    return u;
  }
  T tmp[EV];
#pragma unroll
  for (int e = 0; e < EV; ++e) tmp[e] = k + e < K ? p[(size_t)row * K + k + e] : T(0);
  __builtin_memcpy(&u, tmp, 16);
  return u;
}

template <typename T, typename OutT>
__global__ __launch_bounds__(256) void k_gemm_nt(const T* __restrict__ A, const T* __restrict__ B,
                                                 const float* __restrict__ bias, OutT* __restrict__ C, int M, int N,
                                                 int K) {
  constexpr int EV = GemmT<T>::EV, LS = GK + GemmT<T>::PAD;  // LDS row stride (elements)
  constexpr int CPR = GK / EV, NCH = GB * CPR / 256;          // chunks per row, per thread
  __shared__ __attribute__((aligned(16))) T As[GB * LS];
  __shared__ __attribute__((aligned(16))) T Bs[GB * LS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * GB, n0 = blockIdx.x * GB;
  const bool vec = (K % EV) == 0;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 ra[NCH], rb[NCH];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int id = tid + 256 * c, row = id / CPR, kc = (id % CPR) * EV;
      ra[c] = load_chunk<T>(A, M, K, m0 + row, k0 + kc, vec);
      rb[c] = load_chunk<T>(B, N, K, n0 + row, k0 + kc, vec);
    }
  };
  fetch(0);
  for (int k0 = 0; k0 < K; k0 += GK) {
    __syncthreads();  // the previous tile's reads are done
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int id = tid + 256 * c, row = id / CPR, kc = (id % CPR) * EV;
      *reinterpret_cast<uint4*>(As + row * LS + kc) = ra[c];
      *reinterpret_cast<uint4*>(Bs + row * LS + kc) = rb[c];
    }
    __syncthreads();
    if (k0 + GK < K) fetch(k0 + GK);  // in flight during this tile's products
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int ks = 0; ks < GK; ks += 16) {
        bf16x8_t af[2], bfr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint4 ua = *reinterpret_cast<const uint4*>(As + (wm * 64 + i * 32 + (lane & 31)) * LS + ks +
                                                           (lane >> 5) * 8);
          const uint4 ub = *reinterpret_cast<const uint4*>(Bs + (wn * 64 + i * 32 + (lane & 31)) * LS + ks +
                                                           (lane >> 5) * 8);
          __builtin_memcpy(&af[i], &ua, 16);
          __builtin_memcpy(&bfr[i], &ub, 16);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    } else {
      // lanes of half h take k = 16 h + s at step s (the same order for both operands)
      float av[2][16], bv[2][16];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float* pa = reinterpret_cast<const float*>(As) + (wm * 64 + i * 32 + (lane & 31)) * LS + (lane >> 5) * 16;
        const float* pb = reinterpret_cast<const float*>(Bs) + (wn * 64 + i * 32 + (lane & 31)) * LS + (lane >> 5) * 16;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          av[i][s] = pa[s];
          bv[i][s] = pb[s];
        }
      }
#pragma unroll
      for (int s = 0; s < 16; ++s)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i][s], bv[j][s], acc[i][j], 0, 0, 0);
    }
  }
  // result: lane l holds column l % 32 and rows 8 (r / 4) + 4 (l / 32) + r % 4 of each tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + (lane & 31);
      if (col >= N) continue;
      const float b = bias ? bias[col] : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (row < M) C[(size_t)row * N + col] = cvt_out<OutT>(acc[i][j][r] + b);
      }
    }
}

// out[c][r] = in[r][c] (converted), 32 x 32 tiles through LDS.
template <typename Tin, typename Tout>
__global__ __launch_bounds__(256) void k_transpose(const Tin* __restrict__ in, Tout* __restrict__ out, int R, int Cc) {
  __shared__ float tile[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    const int r = r0 + ty + i, c = c0 + tx;
    tile[ty + i][tx] = (r < R && c < Cc) ? cvt_in(in[(size_t)r * Cc + c]) : 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    const int c = c0 + ty + i, r = r0 + tx;
    if (c < Cc && r < R) out[(size_t)c * R + r] = cvt_out<Tout>(tile[tx][ty + i]);
  }
}

__global__ __launch_bounds__(256) void k_round_bf16(const float* __restrict__ in, u16* __restrict__ out, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = cvt_out<u16>(in[i]);
}

// Column sums of [R][Cc] fp32: stage 1 sums rows of chunk blockIdx.y (COLSUM_ROWS rows)
// in order; stage 2 adds the chunks in order.
constexpr int COLSUM_ROWS = 256;
__global__ __launch_bounds__(256) void k_colsum_part(const float* __restrict__ in, float* __restrict__ part, int R,
                                                     int Cc) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= Cc) return;
  const int r0 = blockIdx.y * COLSUM_ROWS, r1 = min(r0 + COLSUM_ROWS, R);
  float s = 0.f;
  for (int r = r0; r < r1; ++r) s += in[(size_t)r * Cc + c];
  part[(size_t)blockIdx.y * Cc + c] = s;
}
__global__ __launch_bounds__(256) void k_colsum_final(const float* __restrict__ part, float* __restrict__ out,
                                                      int chunks, int Cc) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= Cc) return;
  float s = 0.f;
  for (int i = 0; i < chunks; ++i) s += part[(size_t)i * Cc + c];
  out[c] = s;
}

template <typename T, typename OutT>
static hipError_t gemm(const T* A, const T* B, const float* bias, OutT* C, int M, int N, int K, hipStream_t s) {
  dim3 grid((N + GB - 1) / GB, (M + GB - 1) / GB);
  k_gemm_nt<T, OutT><<<grid, 256, 0, s>>>(A, B, bias, C, M, N, K);
  return hipGetLastError();
}

template <typename Tin, typename Tout>
static hipError_t transpose(const Tin* in, Tout* out, int R, int Cc, hipStream_t s) {
  dim3 grid((Cc + 31) / 32, (R + 31) / 32);
  k_transpose<Tin, Tout><<<grid, 256, 0, s>>>(in, out, R, Cc);
  return hipGetLastError();
}

struct LinWs {
  void* dy_t;   // dy in T, [M][O] (bf16 path only)
  void* dyT;    // dy^T in T, [O][M]
  void* wT;     // W^T in T, [K][O]
  void* xT;     // x^T in T, [K][M]
  float* part;  // column-sum partials [ceil(M / COLSUM_ROWS)][O]
};

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t linear_layout(int M, int Kd, int O, int dtype, char* base, LinWs* w) {
  const size_t es = dtype == DSA3D_BF16 ? 2 : 4;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += al256(bytes);
    return p;
  };
  LinWs l;
  l.dy_t = dtype == DSA3D_BF16 ? take((size_t)M * O * es) : nullptr;
  l.dyT = take((size_t)O * M * es);
  l.wT = take((size_t)Kd * O * es);
  l.xT = take((size_t)Kd * M * es);
  l.part = (float*)take((size_t)((M + COLSUM_ROWS - 1) / COLSUM_ROWS) * O * 4);
  if (w) *w = l;
  return off;
}

template <typename T>
static hipError_t linear_bwd(const T* x, const T* w, const float* dy, int M, int Kd, int O, T* dx, float* dw,
                             float* db, const LinWs& l, hipStream_t s) {
  hipError_t e;
  const T* dyA;  // dy as the A operand of dx = dy W
  if constexpr (sizeof(T) == 2) {
    const size_t n = (size_t)M * O;
    k_round_bf16<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(dy, (u16*)l.dy_t, n);
    dyA = (const T*)l.dy_t;
  } else {
    dyA = (const T*)dy;
  }
  if ((e = transpose<float, T>(dy, (T*)l.dyT, M, O, s)) != hipSuccess) return e;
  if ((e = transpose<T, T>(w, (T*)l.wT, O, Kd, s)) != hipSuccess) return e;
  if ((e = transpose<T, T>(x, (T*)l.xT, M, Kd, s)) != hipSuccess) return e;
  if ((e = gemm<T, T>(dyA, (const T*)l.wT, nullptr, dx, M, Kd, O, s)) != hipSuccess) return e;
  if ((e = gemm<T, float>((const T*)l.dyT, (const T*)l.xT, nullptr, dw, O, Kd, M, s)) != hipSuccess) return e;
  if (db) {
    const int chunks = (M + COLSUM_ROWS - 1) / COLSUM_ROWS;
    k_colsum_part<<<dim3((O + 255) / 256, chunks), 256, 0, s>>>(dy, l.part, M, O);
    k_colsum_final<<<(O + 255) / 256, 256, 0, s>>>(l.part, db, chunks, O);
  }
  return hipGetLastError();
}

}  // namespace dsa3d

using namespace dsa3d;

namespace {

int check_linear(const void* x, const void* w, int M, int Kd, int O, int dtype) {
  if (!x || !w) return DSA3D_ERR_NULL;
  if (dtype != DSA3D_F32 && dtype != DSA3D_BF16) return DSA3D_ERR_DTYPE;
  if (M < 1 || Kd < 1 || O < 1 || (long long)M * Kd >= (1LL << 31) || (long long)M * O >= (1LL << 31) ||
      (long long)Kd * O >= (1LL << 31))
    return DSA3D_ERR_GRID;
  if ((((uintptr_t)x) | ((uintptr_t)w)) & 15u) return DSA3D_ERR_ALIGN;
  return DSA3D_OK;
}

}  // namespace

extern "C" {

int dsa3d_linear_forward(const void* x, const void* weight, const float* bias, int M, int Kd, int O, int dtype,
                         float* y, hipStream_t stream) {
  const int st = check_linear(x, weight, M, Kd, O, dtype);
  if (st != DSA3D_OK) return st;
  if (!y) return DSA3D_ERR_NULL;
  if (((uintptr_t)y | (uintptr_t)bias) & 3u) return DSA3D_ERR_ALIGN;
  const hipError_t e = dtype == DSA3D_BF16
                           ? gemm<u16, float>((const u16*)x, (const u16*)weight, bias, y, M, O, Kd, stream)
                           : gemm<float, float>((const float*)x, (const float*)weight, bias, y, M, O, Kd, stream);
  return e == hipSuccess ? DSA3D_OK : DSA3D_ERR_LAUNCH;
}

size_t dsa3d_linear_workspace_bytes(int M, int Kd, int O, int dtype) {
  const int P = 256;
  if (check_linear((void*)(uintptr_t)P, (void*)(uintptr_t)P, M, Kd, O, dtype) != DSA3D_OK) return 0;
  return linear_layout(M, Kd, O, dtype, nullptr, nullptr);
}

int dsa3d_linear_backward(const void* x, const void* weight, const float* dy, int M, int Kd, int O, int dtype,
                          void* dx, float* dweight, float* dbias, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  const int st = check_linear(x, weight, M, Kd, O, dtype);
  if (st != DSA3D_OK) return st;
  if (!dy || !dx || !dweight || !workspace) return DSA3D_ERR_NULL;
  if (((uintptr_t)dy | (uintptr_t)dweight | (uintptr_t)dbias) & 3u || ((uintptr_t)dx & 15u) ||
      ((uintptr_t)workspace & 15u))
    return DSA3D_ERR_ALIGN;
  if (workspace_bytes < linear_layout(M, Kd, O, dtype, nullptr, nullptr)) return DSA3D_ERR_WORKSPACE;
  LinWs l;
  linear_layout(M, Kd, O, dtype, static_cast<char*>(workspace), &l);
  const hipError_t e =
      dtype == DSA3D_BF16
          ? linear_bwd<u16>((const u16*)x, (const u16*)weight, dy, M, Kd, O, (u16*)dx, dweight, dbias, l, stream)
          : linear_bwd<float>((const float*)x, (const float*)weight, dy, M, Kd, O, (float*)dx, dweight, dbias, l,
                              stream);
  return e == hipSuccess ? DSA3D_OK : DSA3D_ERR_LAUNCH;
}

}  // extern "C"
