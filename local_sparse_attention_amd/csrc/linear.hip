// The offset predictor's pointwise layer (MegaSlide-DiT, section "3D Deformable Slide
// Attention": offsets come from a depthwise 3-D convolution followed by a linear layer,
// pointwise convolutions in the implementation paragraph): y = x W^T + b per token.
//
// k_gemm_nt  C[M][N] = A[M][K] B[N][K]^T (+ bias[N]) on the matrix cores: 128 x 256
//            block tiles for bf16 (128 x 128 for fp32 inputs or N < 256), 32-deep K steps
//            staged through LDS (the next tile's global loads issued before this tile's
//            products), four waves of 64 x 128 (64 x 64), each as 2 x 4 (2 x 2) tiles of
//            v_mfma_f32_32x32x16_bf16 (fp32 inputs: v_mfma_f32_32x32x2_f32).  Products
//            with few output tiles and a long K split K over grid layers and add the
//            parts in a fixed order.
//            Both bf16 shapes run at the same rate on gfx950; the 32 x 32 x 16 one covers a
//            64 x 64 wave tile in a quarter of the instructions.
// Backward: dx = dy W and dW = dy^T x are the same kernel on transposed copies (one pass
// over dy, k_dy_prep, writes its bf16 rounding, its transpose and the per-tile column
// sums of db; k_transpose the copies of W and x); db's column sums add in a fixed order.
#include "dsa3d.h"
#include "internal.hpp"
#include "tube.hpp"

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
// matrix stored with row stride ld, zero outside; vec: K and ld are multiples of EV
// (whole chunks, 16-byte aligned rows).
template <typename T>
__device__ __forceinline__ uint4 load_chunk(const T* p, int rows, int K, size_t ld, int row, int k, bool vec) {
  constexpr int EV = GemmT<T>::EV;
  uint4 u = {0u, 0u, 0u, 0u};
  if (row >= rows) return u;
  if (vec) {
    if (k < K) u = *reinterpret_cast<const uint4*>(p + (size_t)row * ld + k);
    return u;
  }
  T tmp[EV];
#pragma unroll
  for (int e = 0; e < EV; ++e) tmp[e] = k + e < K ? p[(size_t)row * ld + k + e] : T(0);
  __builtin_memcpy(&u, tmp, 16);
  return u;
}

// Split K (gridDim.z > 1): block z takes the columns kc z .. kc (z + 1) - 1 of A and B
// (kc a multiple of GK) and writes its partial product to C + z M N (no bias);
// k_splitk_sum adds the parts.  WN: 32-column tiles per wave along N, so a block is
// GB x (64 WN) and a wave 64 x 32 WN (WN = 4 reads a quarter fewer fragment bytes per
// product than WN = 2 and stages half the bytes per product).
template <typename T, typename OutT, int WN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm_nt(const T* __restrict__ A, const T* __restrict__ B,
                                                 const float* __restrict__ bias, OutT* __restrict__ C, int M, int N,
                                                 int Kfull, int kc) {
  constexpr int BN = 64 * WN;
  const size_t ld = (size_t)Kfull;
  const int kbeg = blockIdx.z * kc, K = min(kc, Kfull - kbeg);
  A += kbeg;
  B += kbeg;
  C += (size_t)blockIdx.z * M * N;
  constexpr int EV = GemmT<T>::EV, LS = GK + GemmT<T>::PAD;  // LDS row stride (elements)
  constexpr int CPR = GK / EV;                                // chunks per row
  constexpr int NCA = GB * CPR / 256, NCB = BN * CPR / 256;   // chunks per thread
  __shared__ __attribute__((aligned(16))) T As[GB * LS];
  __shared__ __attribute__((aligned(16))) T Bs[BN * LS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * GB, n0 = blockIdx.x * BN;
  const bool vec = (Kfull % EV) == 0;

  f32x16_t acc[2][WN];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  float bcol[WN];
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const int col = n0 + wn * 32 * WN + j * 32 + (lane & 31);
    bcol[j] = bias && col < N ? bias[col] : 0.f;
  }

  uint4 ra[NCA], rb[NCB];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int c = 0; c < NCA; ++c) {
      const int id = tid + 256 * c, row = id / CPR, ck = (id % CPR) * EV;
      ra[c] = load_chunk<T>(A, M, K, ld, m0 + row, k0 + ck, vec);
    }
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const int id = tid + 256 * c, row = id / CPR, ck = (id % CPR) * EV;
      rb[c] = load_chunk<T>(B, N, K, ld, n0 + row, k0 + ck, vec);
    }
  };
  fetch(0);
  for (int k0 = 0; k0 < K; k0 += GK) {
    __syncthreads();  // the previous tile's reads are done
#pragma unroll
    for (int c = 0; c < NCA; ++c) {
      const int id = tid + 256 * c, row = id / CPR, ck = (id % CPR) * EV;
      *reinterpret_cast<uint4*>(As + row * LS + ck) = ra[c];
    }
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const int id = tid + 256 * c, row = id / CPR, ck = (id % CPR) * EV;
      *reinterpret_cast<uint4*>(Bs + row * LS + ck) = rb[c];
    }
    __syncthreads();
    if (k0 + GK < K) fetch(k0 + GK);  // in flight during this tile's products
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int ks = 0; ks < GK; ks += 16) {
        bf16x8_t af[2], bfr[WN];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint4 ua = *reinterpret_cast<const uint4*>(As + (wm * 64 + i * 32 + (lane & 31)) * LS + ks +
                                                           (lane >> 5) * 8);
          __builtin_memcpy(&af[i], &ua, 16);
        }
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          const uint4 ub = *reinterpret_cast<const uint4*>(Bs + (wn * 32 * WN + j * 32 + (lane & 31)) * LS + ks +
                                                           (lane >> 5) * 8);
          __builtin_memcpy(&bfr[j], &ub, 16);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    } else {
      // lanes of half h take k = 16 h + s at step s (the same order for both operands)
      float av[2][16], bv[WN][16];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float* pa = reinterpret_cast<const float*>(As) + (wm * 64 + i * 32 + (lane & 31)) * LS + (lane >> 5) * 16;
#pragma unroll
        for (int s = 0; s < 16; ++s) av[i][s] = pa[s];
      }
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const float* pb =
            reinterpret_cast<const float*>(Bs) + (wn * 32 * WN + j * 32 + (lane & 31)) * LS + (lane >> 5) * 16;
#pragma unroll
        for (int s = 0; s < 16; ++s) bv[j][s] = pb[s];
      }
#pragma unroll
      for (int s = 0; s < 16; ++s)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i][s], bv[j][s], acc[i][j], 0, 0, 0);
    }
  }
  // every load done (a wait the compiler sees, so that it adds none before each of the
  // conditional stores below, which would make each store wait for the one before it)
  __builtin_amdgcn_s_waitcnt(0);
  // result: lane l holds column l % 32 and rows 8 (r / 4) + 4 (l / 32) + r % 4 of each tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int col = n0 + wn * 32 * WN + j * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (row < M) C[(size_t)row * N + col] = cvt_out<OutT>(acc[i][j][r] + bcol[j]);
      }
    }
}

// Pipelined form for bf16 with K a multiple of 8 (rows of 16-byte chunks): 128 x 256
// blocks, 64-deep K steps in a ring of RING_ST LDS stages filled by direct global->LDS
// loads two steps ahead (each wave issues 12 per stage: 8 rows of 128 bytes a load, rows
// swizzled as sw() so that the 16-byte fragment reads do not collide on LDS banks),
// four waves of 64 x 128 as 2 x 4 tiles of v_mfma_f32_32x32x16_bf16.  Chunks outside
// the matrix (rows past M or N, columns past K) load 16 zero bytes from zero16, so every
// stage holds zeros there and every wave issues the same number of loads.
constexpr int RING_ST = 3, RK = 64, RBN = 256, RING_GY = 8;
constexpr int RING_STAGE = (GB + RBN) * RK * 2;  // bytes: A rows, then B rows
static __device__ __attribute__((aligned(16))) uint4 zero16[1];

template <typename OutT>
__global__ __launch_bounds__(256) void k_gemm_ring(const u16* __restrict__ A, const u16* __restrict__ B,
                                                   const float* __restrict__ bias, OutT* __restrict__ C, int M,
                                                   int N, int Kfull, int kc) {
  __shared__ __attribute__((aligned(1024))) char ring[RING_ST][RING_STAGE];
  const size_t ld = (size_t)Kfull;
  const int kbeg = blockIdx.z * kc, K = min(kc, Kfull - kbeg);
  A += kbeg;
  B += kbeg;
  C += (size_t)blockIdx.z * M * N;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  // block order: each XCD takes a contiguous range of blocks (xcd_remap), walked in
  // groups of RING_GY block rows with the column index outer, so the A rows and B
  // columns of the blocks in flight on one XCD stay in its L2
  const int nbx = (N + RBN - 1) / RBN, nby = (M + GB - 1) / GB;
  const int L = xcd_remap(blockIdx.x, nbx * nby);
  const int g0 = (L / (RING_GY * nbx)) * RING_GY, gy = min(RING_GY, nby - g0);
  const int rr = L - g0 * nbx;
  const int m0 = (g0 + rr % gy) * GB, n0 = (rr / gy) * RBN;
  const int nk = (K + RK - 1) / RK;
  // this wave's 12 loads of a stage: load i covers stage rows 8 (4 i + wave) .. + 7
  // (rows 0-127 are A's, 128-383 B's); lane l takes row + l / 8, physical chunk l % 8,
  // which holds logical chunk (l % 8) ^ (row & 7)
  // kmax[i]: the load's chunks are inside the matrix for K steps kt with kt RK < kmax[i]
  // (0 for rows past the edge); src[i] points at row 0 then, never read.
  const u16* src[12];
  int kmax[12];
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    const int r = 8 * (4 * i + wave) + (lane >> 3);  // i < 4: A's rows (wave-uniform)
    const int c = ((lane & 7) ^ r) & 7;
    const int grow = i < 4 ? m0 + r : n0 + (r - GB);
    const bool rin = grow < (i < 4 ? M : N);
    src[i] = (i < 4 ? A : B) + (rin ? (size_t)grow * ld : 0) + c * 8;
    kmax[i] = rin ? K - c * 8 : 0;
  }
  // loads i0 .. i1 - 1 of stage kt
  auto issue = [&](int kt, int i0, int i1) {
    char* st = ring[kt % RING_ST];
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      if (i < i0 || i >= i1) continue;
      const bool ok = kt * RK < kmax[i];
      const uintptr_t g = ok ? reinterpret_cast<uintptr_t>(src[i] + (size_t)kt * RK)
                             : reinterpret_cast<uintptr_t>(&zero16[0]);
      dma16(reinterpret_cast<const void*>(g), st + 1024 * (4 * i + wave));
    }
  };
  float bcol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = n0 + wn * 128 + j * 32 + (lane & 31);
    bcol[j] = bias && col < N ? bias[col] : 0.f;
  }

  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

#pragma unroll
  for (int s = 0; s < RING_ST - 1; ++s) issue(s, 0, 12);
  for (int kt = 0; kt < nk; ++kt) {
    wait_vmcnt_c<(RING_ST - 2) * 12>();  // this wave's loads of stage kt have landed
    lds_barrier();                       // everyone's have, and stage kt - 1 is read
    typedef __attribute__((address_space(3))) char lds_char;
    const lds_char* st = (const lds_char*)ring[kt % RING_ST];
#pragma unroll
    for (int ks = 0; ks < RK / 16; ++ks) {
      // a quarter of stage kt + 2's loads (into the slot of stage kt - 1) before each
      // 16-deep step, so that the CU's load issue spreads over the stage
      issue(kt + RING_ST - 1, 3 * ks, 3 * ks + 3);
      const int cb = (2 * ks + (lane >> 5)) * 16;  // logical byte of this lane's 16 bytes
      bf16x8_t af[2], bfr[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + (lane & 31);
        af[i] = *(const __attribute__((address_space(3))) bf16x8_t*)(st + sw(r, cb));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = GB + wn * 128 + j * 32 + (lane & 31);
        bfr[j] = *(const __attribute__((address_space(3))) bf16x8_t*)(st + sw(r, cb));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }
  // the zero loads of the last stages and the bias values: a wait the compiler sees, so
  // that it adds none before each of the conditional stores below
  __builtin_amdgcn_s_waitcnt(0);
  // result: lane l holds column l % 32 and rows 8 (r / 4) + 4 (l / 32) + r % 4 of each tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + j * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (row < M) C[(size_t)row * N + col] = cvt_out<OutT>(acc[i][j][r] + bcol[j]);
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

// One pass over dy [R][Cc] fp32 in 32 x 32 tiles through LDS: its rounded copy in T
// (rounded, when not null), its transpose in T ([Cc][R]), and the column sums of each
// tile's rows, added in row order, into part[R / 32 tile row][Cc] (k_colsum_final then
// adds the tile rows in order: a fixed order, so the result does not depend on the
// launch).
constexpr int COLSUM_ROWS = 32;
template <typename T>
__global__ __launch_bounds__(256) void k_dy_prep(const float* __restrict__ dy, T* __restrict__ rounded,
                                                 T* __restrict__ dyT, float* __restrict__ part, int R, int Cc) {
  __shared__ float tile[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    const int r = r0 + ty + i, c = c0 + tx;
    const bool in = r < R && c < Cc;
    const float v = in ? dy[(size_t)r * Cc + c] : 0.f;
    tile[ty + i][tx] = v;
    if (rounded && in) rounded[(size_t)r * Cc + c] = cvt_out<T>(v);
  }
  __syncthreads();
  if (ty == 0 && c0 + tx < Cc) {
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 32; ++r) sum += tile[r][tx];
    part[(size_t)blockIdx.y * Cc + c0 + tx] = sum;
  }
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    const int c = c0 + ty + i, r = r0 + tx;
    if (c < Cc && r < R) dyT[(size_t)c * R + r] = cvt_out<T>(tile[tx][ty + i]);
  }
}
__global__ __launch_bounds__(256) void k_colsum_final(const float* __restrict__ part, float* __restrict__ out,
                                                      int chunks, int Cc) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= Cc) return;
  float s = 0.f;
#pragma unroll 8
  for (int i = 0; i < chunks; ++i) s += part[(size_t)i * Cc + c];
  out[c] = s;
}

// C[i] = sum over z of part[z][i] in order z = 0, 1, .. (fixed, so the result does not
// depend on the launch), four consecutive elements a thread; vec: n is a multiple of 4
// and C 16-byte aligned (16-byte loads and stores), else one element at a time.
__global__ __launch_bounds__(256) void k_splitk_sum(const float* __restrict__ part, float* __restrict__ C, size_t n,
                                                    int parts, int vec) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  if (vec) {
    float4 a = *reinterpret_cast<const float4*>(part + i);
    for (int z = 1; z < parts; ++z) {
      const float4 b = *reinterpret_cast<const float4*>(part + (size_t)z * n + i);
      a.x += b.x;
      a.y += b.y;
      a.z += b.z;
      a.w += b.w;
    }
    *reinterpret_cast<float4*>(C + i) = a;
    return;
  }
  for (size_t j = i; j < min(i + 4, n); ++j) {
    float a = part[j];
    for (int z = 1; z < parts; ++z) a += part[(size_t)z * n + j];
    C[j] = a;
  }
}

// Block width: 256 columns (WN = 4) for bf16 inputs when N fills it, else 128.
template <typename T>
static int gemm_wn(int N) { return sizeof(T) == 2 && N >= 256 ? 4 : 2; }

// K split in parts of kc (a multiple of GK) for products with few output tiles and a long
// K: each part a grid layer of its own, so that the launch fills the chip.
template <typename T>
static int splitk_parts(int M, int N, int K) {
  const int bn = 64 * gemm_wn<T>(N);
  const long long tiles = (long long)((N + bn - 1) / bn) * ((M + GB - 1) / GB);
  if (tiles >= 512 || K < 4096) return 1;
  return (int)min((long long)(K / 1024), (768 + tiles - 1) / tiles);
}
static int splitk_chunk(int K, int parts) { return ((K + parts - 1) / parts + GK - 1) / GK * GK; }

// The pipelined bf16 form loads whole 16-byte chunks: rows of K elements must start on
// 16 bytes.
template <typename T>
static bool Kfull_ok(int K, const T* A, const T* B) {
  return K % 8 == 0 && ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B)) & 15u) == 0;
}

template <typename T, typename OutT>
static void launch_gemm(const T* A, const T* B, const float* bias, OutT* C, int M, int N, int K, int kc, int layers,
                        hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    if (N >= RBN && Kfull_ok(K, A, B)) {
      k_gemm_ring<OutT><<<dim3(((N + RBN - 1) / RBN) * ((M + GB - 1) / GB), 1, layers), 256, 0, s>>>(A, B, bias, C, M,
                                                                                                       N, K, kc);
      return;
    }
    if (gemm_wn<T>(N) == 4) {
      k_gemm_nt<T, OutT, 4><<<dim3((N + 255) / 256, (M + GB - 1) / GB, layers), 256, 0, s>>>(A, B, bias, C, M, N, K,
                                                                                             kc);
      return;
    }
  }
  k_gemm_nt<T, OutT, 2><<<dim3((N + 127) / 128, (M + GB - 1) / GB, layers), 256, 0, s>>>(A, B, bias, C, M, N, K, kc);
}

template <typename T, typename OutT>
static hipError_t gemm(const T* A, const T* B, const float* bias, OutT* C, int M, int N, int K, hipStream_t s) {
  launch_gemm<T, OutT>(A, B, bias, C, M, N, K, K, 1, s);
  return hipGetLastError();
}

// C (fp32, no bias) with K split as splitk_parts() says, the parts in part (parts M N
// floats) when there are several.
template <typename T>
static hipError_t gemm_split(const T* A, const T* B, float* C, int M, int N, int K, float* part, hipStream_t s) {
  const int parts = splitk_parts<T>(M, N, K);
  if (parts == 1) return gemm<T, float>(A, B, nullptr, C, M, N, K, s);
  const int kc = splitk_chunk(K, parts);
  const int used = (K + kc - 1) / kc;
  launch_gemm<T, float>(A, B, nullptr, part, M, N, K, kc, used, s);
  const size_t n = (size_t)M * N;
  const int vec = (n % 4) == 0 && (reinterpret_cast<uintptr_t>(C) & 15u) == 0;
  k_splitk_sum<<<(unsigned)((n + 1023) / 1024), 256, 0, s>>>(part, C, n, used, vec);
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
  float* kpart; // split-K partials of dW [parts][O][Kd] (null when dW is not split)
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
  const int parts = dtype == DSA3D_BF16 ? splitk_parts<u16>(O, Kd, M) : splitk_parts<float>(O, Kd, M);
  l.kpart = parts > 1 ? (float*)take((size_t)parts * O * Kd * 4) : nullptr;
  if (w) *w = l;
  return off;
}

template <typename T>
static hipError_t linear_bwd(const T* x, const T* w, const float* dy, int M, int Kd, int O, T* dx, float* dw,
                             float* db, const LinWs& l, hipStream_t s) {
  hipError_t e;
  // dy once: rounded to T (the A operand of dx = dy W; fp32 inputs use dy itself),
  // transposed (the A operand of dW = dy^T x), column sums (db)
  const int chunks = (M + COLSUM_ROWS - 1) / COLSUM_ROWS;
  T* rounded = sizeof(T) == 2 ? (T*)l.dy_t : nullptr;
  k_dy_prep<T><<<dim3((O + 31) / 32, chunks), 256, 0, s>>>(dy, rounded, (T*)l.dyT, l.part, M, O);
  const T* dyA = sizeof(T) == 2 ? (const T*)l.dy_t : (const T*)dy;
  if ((e = transpose<T, T>(w, (T*)l.wT, O, Kd, s)) != hipSuccess) return e;
  if ((e = transpose<T, T>(x, (T*)l.xT, M, Kd, s)) != hipSuccess) return e;
  if ((e = gemm<T, T>(dyA, (const T*)l.wT, nullptr, dx, M, Kd, O, s)) != hipSuccess) return e;
  if ((e = gemm_split<T>((const T*)l.dyT, (const T*)l.xT, dw, O, Kd, M, l.kpart, s)) != hipSuccess) return e;
  if (db) k_colsum_final<<<(O + 255) / 256, 256, 0, s>>>(l.part, db, chunks, O);
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
