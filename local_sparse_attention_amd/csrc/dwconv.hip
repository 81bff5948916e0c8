// Depthwise 3-D convolution over the token grid (MegaSlide-DiT, section "3D Deformable
// Slide Attention": the DWConv3D term of Eq. (1), and the first stage of the offset
// predictor, which the implementation paragraph builds from nn.Conv3d with groups equal
// to the hidden size).  One ct x cy x cx filter per channel, cross-correlation, zero
// padding that keeps the grid:
//   y[n, c] = b[c] + sum_taps w[c][tap] x[n + shift(tap), c]
// Tensors are [N][C] (token n = (t * Hp + y) * Wp + x, channels contiguous).  The
// stencil is HBM-bound: the kernels keep a block's filters in LDS and take each input
// row from L1/L2 for the taps that reuse it.
//   k_dwconv      one thread per (4 tokens of a row, 8 channels); forward (optionally adding into y:
//                 the attention output plus the convolution term in one pass) and, with
//                 the taps mirrored, the input gradient dx.
//   k_dwconv_dw   filter and bias gradients: a block sums dy[n, c] x[n + shift, c] over a
//                 span of one frame's rows for 2048 channels and up to 8 taps; the spans'
//                 partial sums are added in a fixed order by k_dwconv_dw_sum
//                 (deterministic, no atomics).
#include "dsa3d.h"
#include "internal.hpp"
#include "tube.hpp"

#include <algorithm>

namespace dsa3d {

struct CGeom {
  int F, Hp, Wp, C;
  int ct, cy, cx, taps;
  int N;
};

constexpr int CONV_CB = 64;      // channels per forward block
constexpr int CONV_TOK = 32;     // token quads (4 tokens of a row) per forward block
constexpr int CONV_MAX_TAPS = 512;

// 32 bytes of zeros: the row a masked tap reads (8 bf16 or 8 fp32 zero elements), so the
// load itself yields 0 and needs no select afterwards.
__device__ __align__(32) const uint4 g_zero_row[2] = {};

__device__ __forceinline__ void ld8(const u16* p, float* x) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void ld8(const float* p, float* x) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void st8(u16* p, const float* x) {
  store4(p, x[0], x[1], x[2], x[3]);
  store4(p + 4, x[4], x[5], x[6], x[7]);
}
__device__ __forceinline__ void st8(float* p, const float* x) {
  store4(p, x[0], x[1], x[2], x[3]);
  store4(p + 4, x[4], x[5], x[6], x[7]);
}

// Packed tap shift (da, de, df), each biased by 512 into 10 bits.
__device__ __forceinline__ int pack_shift(int da, int de, int df) {
  return ((da + 512) << 20) | ((de + 512) << 10) | (df + 512);
}
__device__ __forceinline__ void unpack_shift(int s, int& da, int& de, int& df) {
  da = (s >> 20) - 512;
  de = ((s >> 10) & 1023) - 512;
  df = (s & 1023) - 512;
}

// flip = 0: y = conv(x) + b (+ y when accumulating).  flip = 1: the transpose (taps
// mirrored, no bias): dx from dy.  A thread takes 8 channels of CONV_Q consecutive tokens
// of one grid row, so a tap's row test, row address and filter values serve CONV_Q
// outputs; a tap's CONV_Q loads are issued before their products (a token outside the
// grid reads a row of zeros).
constexpr int CONV_Q = 4;

template <typename T>
__global__ __launch_bounds__(256) void k_dwconv(const T* __restrict__ x, const float* __restrict__ w,
                                                const float* __restrict__ b, T* __restrict__ y, CGeom g,
                                                int accumulate, int flip) {
  extern __shared__ float lw[];  // [taps][CONV_CB] filters, then [taps] packed shifts
  int* lsh = reinterpret_cast<int*>(lw + g.taps * CONV_CB);
  const int tid = threadIdx.x;
  // each XCD takes a contiguous run of quad blocks of one channel block, so the rows of
  // neighbouring frames and rows that a block's taps reach sit in the same L2
  const int nqx = (g.Wp + CONV_Q - 1) / CONV_Q;         // quads per grid row
  const long long nquads = (long long)g.F * g.Hp * nqx;
  const int nqb = (int)((nquads + CONV_TOK - 1) / CONV_TOK), ncb = (g.C + CONV_CB - 1) / CONV_CB;
  const int L = xcd_remap(blockIdx.x, nqb * ncb);
  const int cb = L / nqb, qb = L - cb * nqb;
  const int c0 = cb * CONV_CB;
  const int rt = (g.ct - 1) / 2, ry = (g.cy - 1) / 2, rx = (g.cx - 1) / 2;
  const int sgn = flip ? -1 : 1;
  for (int i = tid; i < g.taps * CONV_CB; i += 256) {
    const int tap = i / CONV_CB, cl = i - tap * CONV_CB;
    lw[i] = c0 + cl < g.C ? w[(size_t)(c0 + cl) * g.taps + tap] : 0.f;
  }
  for (int tap = tid; tap < g.taps; tap += 256) {
    const int a = tap / (g.cy * g.cx), r = tap - a * (g.cy * g.cx), e = r / g.cx, f = r - e * g.cx;
    lsh[tap] = pack_shift(sgn * (a - rt), sgn * (e - ry), sgn * (f - rx));
  }
  __syncthreads();
  const int cg = tid & 7, ql = tid >> 3;
  const long long qd = (long long)qb * CONV_TOK + ql;
  const int c = c0 + cg * 8;
  if (qd >= nquads || c >= g.C) return;
  const int qx = (int)(qd % nqx);
  const int ty = (int)(qd / nqx);  // t * Hp + y
  const int t = ty / g.Hp, yy = ty - t * g.Hp, x0 = qx * CONV_Q;
  const size_t n0 = (size_t)ty * g.Wp + x0;
  float acc[CONV_Q][8];
#pragma unroll
  for (int q = 0; q < CONV_Q; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[q][e] = (b && !flip) ? b[c + e] : 0.f;
  for (int tap = 0; tap < g.taps; ++tap) {
    int da, de, df;
    unpack_shift(lsh[tap], da, de, df);
    const int ts = t + da, ys = yy + de;
    const bool row_ok = (unsigned)ts < (unsigned)g.F && (unsigned)ys < (unsigned)g.Hp;
    const T* row = x + ((size_t)(ts * g.Hp + ys) * g.Wp) * g.C + c;
    const T* zero = reinterpret_cast<const T*>(g_zero_row);
    float v[CONV_Q][8];
#pragma unroll
    for (int q = 0; q < CONV_Q; ++q) {
      const int xs = x0 + q + df;
      const bool ok = row_ok && x0 + q < g.Wp && (unsigned)xs < (unsigned)g.Wp;
      ld8(ok ? row + (size_t)xs * g.C : zero, v[q]);
    }
    const float4 w0 = *reinterpret_cast<const float4*>(lw + tap * CONV_CB + cg * 8);
    const float4 w1 = *reinterpret_cast<const float4*>(lw + tap * CONV_CB + cg * 8 + 4);
    const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int q = 0; q < CONV_Q; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[q][e] = fmaf(wv[e], v[q][e], acc[q][e]);
  }
#pragma unroll
  for (int q = 0; q < CONV_Q; ++q) {
    if (x0 + q >= g.Wp) break;
    T* out = y + (n0 + q) * g.C + c;
    if (accumulate) {
      float v[8];
      ld8(out, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[q][e] += v[e];
    }
    st8(out, acc[q]);
  }
}

// The same, specialised on the filter width CX: per (da, de) row pair a thread loads the
// CONV_Q + CX - 1 row positions its CONV_Q tokens reach once and takes all CX taps from
// them (CONV_Q + CX - 1 loads instead of CONV_Q * CX).  Filters in LDS as [taps][CONV_CB].
template <typename T, int CX>
__global__ __launch_bounds__(256) void k_dwconv_w(const T* __restrict__ x, const float* __restrict__ w,
                                                  const float* __restrict__ b, T* __restrict__ y, CGeom g,
                                                  int accumulate, int flip) {
  extern __shared__ float lw[];  // [taps][CONV_CB]
  constexpr int NV = CONV_Q + CX - 1;
  const int tid = threadIdx.x;
  const int nqx = (g.Wp + CONV_Q - 1) / CONV_Q;
  const long long nquads = (long long)g.F * g.Hp * nqx;
  const int nqb = (int)((nquads + CONV_TOK - 1) / CONV_TOK), ncb = (g.C + CONV_CB - 1) / CONV_CB;
  const int L = xcd_remap(blockIdx.x, nqb * ncb);
  const int cb = L / nqb, qb = L - cb * nqb;
  const int c0 = cb * CONV_CB;
  for (int i = tid; i < g.taps * CONV_CB; i += 256) {
    const int tap = i / CONV_CB, cl = i - tap * CONV_CB;
    lw[i] = c0 + cl < g.C ? w[(size_t)(c0 + cl) * g.taps + tap] : 0.f;
  }
  __syncthreads();
  const int cg = tid & 7, ql = tid >> 3;
  const long long qd = (long long)qb * CONV_TOK + ql;
  const int c = c0 + cg * 8;
  if (qd >= nquads || c >= g.C) return;
  const int qx = (int)(qd % nqx);
  const int ty = (int)(qd / nqx);
  const int t = ty / g.Hp, yy = ty - t * g.Hp, x0 = qx * CONV_Q;
  const size_t n0 = (size_t)ty * g.Wp + x0;
  const int rt = (g.ct - 1) / 2, ry = (g.cy - 1) / 2, rx = (CX - 1) / 2;
  const int sgn = flip ? -1 : 1;
  const T* zero = reinterpret_cast<const T*>(g_zero_row);
  float acc[CONV_Q][8];
#pragma unroll
  for (int q = 0; q < CONV_Q; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[q][e] = (b && !flip) ? b[c + e] : 0.f;
  for (int a = 0; a < g.ct; ++a)
    for (int e2 = 0; e2 < g.cy; ++e2) {
      const int ts = t + sgn * (a - rt), ys = yy + sgn * (e2 - ry);
      const bool row_ok = (unsigned)ts < (unsigned)g.F && (unsigned)ys < (unsigned)g.Hp;
      const T* row = x + ((size_t)(ts * g.Hp + ys) * g.Wp) * g.C + c;
      // positions x0 - rx .. x0 + CONV_Q - 1 + rx
      float v[NV][8];
#pragma unroll
      for (int p = 0; p < NV; ++p) {
        const int xs = x0 - rx + p;
        const bool ok = row_ok && (unsigned)xs < (unsigned)g.Wp;
        ld8(ok ? row + (size_t)xs * g.C : zero, v[p]);
      }
      const int tap_row = (a * g.cy + e2) * CX;
#pragma unroll
      for (int f = 0; f < CX; ++f) {
        // flip mirrors the tap: output x reads x - (f - rx), i.e. position index 2 rx - f
        const int tap = tap_row + f;
        const float4 w0 = *reinterpret_cast<const float4*>(lw + tap * CONV_CB + cg * 8);
        const float4 w1 = *reinterpret_cast<const float4*>(lw + tap * CONV_CB + cg * 8 + 4);
        const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
        for (int q = 0; q < CONV_Q; ++q) {
          const int pidx = q + (flip ? 2 * rx - f : f);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[q][e] = fmaf(wv[e], v[pidx][e], acc[q][e]);
        }
      }
    }
#pragma unroll
  for (int q = 0; q < CONV_Q; ++q) {
    if (x0 + q >= g.Wp) break;
    T* out = y + (n0 + q) * g.C + c;
    if (accumulate) {
      float v[8];
      ld8(out, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[q][e] += v[e];
    }
    st8(out, acc[q]);
  }
}

// Filter / bias gradient partial sums.  A block takes one frame t, a span of its rows
// (yc of nyc spans), 2048 channels (8 a thread) and up to DW_TAPS taps (chunk tc); each
// thread walks the span's tokens in order, loading its 8 channels of dy and, per tap, of x
// (a tap outside the grid reads a row of zeros), and keeps 8 x DW_TAPS sums.  Blocks are
// ordered (channel block, tap chunk, row span, frame) with frames fastest and each XCD
// given a contiguous run, so neighbouring frames' rows meet in one L2.
// part[((t * nyc + yc) * C + c) * (taps + 1) + tap], the bias sum at index taps.
constexpr int DW_CPB = 2048, DW_TAPS = 8;

struct DwSplit {
  int ncb, ntc, nyc, rows;  // channel blocks, tap chunks, row spans, rows per span
};

template <typename T>
__global__ __launch_bounds__(256) void k_dwconv_dw(const T* __restrict__ x, const T* __restrict__ dy,
                                                   float* __restrict__ part, CGeom g, DwSplit sp) {
  const int total = sp.ncb * sp.ntc * sp.nyc * g.F;
  int L = xcd_remap(blockIdx.x, total);
  const int t = L % g.F;
  L /= g.F;
  const int yc = L % sp.nyc;
  L /= sp.nyc;
  const int tc = L % sp.ntc, cb = L / sp.ntc;
  const int c = cb * DW_CPB + 8 * threadIdx.x;
  if (c >= g.C) return;
  const int tap0 = tc * DW_TAPS, ntap = min(DW_TAPS, g.taps - tap0);
  const int rt = (g.ct - 1) / 2, ry = (g.cy - 1) / 2, rx = (g.cx - 1) / 2;
  const T* zero = reinterpret_cast<const T*>(g_zero_row);
  float acc[DW_TAPS][8], bs[8];
  int sh[DW_TAPS];  // packed (da, de, df) shifts of this chunk's taps
#pragma unroll
  for (int i = 0; i < DW_TAPS; ++i) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
    const int tap = tap0 + min(i, ntap - 1);
    const int a = tap / (g.cy * g.cx), r = tap - a * (g.cy * g.cx), e = r / g.cx, f = r - e * g.cx;
    sh[i] = pack_shift(a - rt, e - ry, f - rx);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) bs[e] = 0.f;
  const int y0 = yc * sp.rows, y1 = min(y0 + sp.rows, g.Hp);
  for (int yy = y0; yy < y1; ++yy)
    for (int xx = 0; xx < g.Wp; ++xx) {
      const int n = (t * g.Hp + yy) * g.Wp + xx;
      float d[8], v[DW_TAPS][8];
      ld8(dy + (size_t)n * g.C + c, d);
      // every tap's load first (taps past ntap repeat the last one and are never written)
#pragma unroll
      for (int i = 0; i < DW_TAPS; ++i) {
        int da, de, df;
        unpack_shift(sh[i], da, de, df);
        const int ts = t + da, ys = yy + de, xs = xx + df;
        const bool ok = (unsigned)ts < (unsigned)g.F && (unsigned)ys < (unsigned)g.Hp && (unsigned)xs < (unsigned)g.Wp;
        ld8(ok ? x + (size_t)((ts * g.Hp + ys) * g.Wp + xs) * g.C + c : zero, v[i]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) bs[e] += d[e];
#pragma unroll
      for (int i = 0; i < DW_TAPS; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] = fmaf(d[e], v[i][e], acc[i][e]);
    }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float* p = part + (((size_t)t * sp.nyc + yc) * g.C + c + e) * (g.taps + 1);
#pragma unroll
    for (int i = 0; i < DW_TAPS; ++i)
      if (i < ntap) p[tap0 + i] = acc[i][e];
    if (tc == 0) p[g.taps] = bs[e];
  }
}

// The filter gradient specialised on the filter width CX: a block takes one frame t, a
// span of rows, 2048 channels (8 a thread) and ROWS consecutive filter rows (da, de) of
// one frame offset (chunk tc of ct * cy / ROWS); each thread slides along its rows keeping,
// per filter row, the CX input positions x - rx .. x + rx in registers, so each step loads
// one dy row and one new input row per filter row (instead of one per tap).
template <typename T, int ROWS, int CX>
__global__ __launch_bounds__(256) void k_dwconv_dw_w(const T* __restrict__ x, const T* __restrict__ dy,
                                                     float* __restrict__ part, CGeom g, DwSplit sp) {
  const int total = sp.ncb * sp.ntc * sp.nyc * g.F;
  int L = xcd_remap(blockIdx.x, total);
  const int t = L % g.F;
  L /= g.F;
  const int yc = L % sp.nyc;
  L /= sp.nyc;
  const int tc = L % sp.ntc, cb = L / sp.ntc;
  const int c = cb * DW_CPB + 8 * threadIdx.x;
  if (c >= g.C) return;
  constexpr int rx = (CX - 1) / 2;
  const int rt = (g.ct - 1) / 2, ry = (g.cy - 1) / 2;
  const int row0 = tc * ROWS;  // filter rows (a * cy + e) row0 .. row0 + ROWS - 1
  const T* zero = reinterpret_cast<const T*>(g_zero_row);
  float acc[ROWS][CX][8], win[ROWS][CX][8], bs[8];
  int da[ROWS], de[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int fr = min(row0 + r, g.ct * g.cy - 1);  // rows past the filter repeat the last, never written
    da[r] = fr / g.cy - rt;
    de[r] = fr % g.cy - ry;
#pragma unroll
    for (int f = 0; f < CX; ++f)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][f][e] = 0.f;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) bs[e] = 0.f;
  const int y0 = yc * sp.rows, y1 = min(y0 + sp.rows, g.Hp);
  for (int yy = y0; yy < y1; ++yy) {
    const T* rows[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const int ts = t + da[r], ys = yy + de[r];
      const bool ok = (unsigned)ts < (unsigned)g.F && (unsigned)ys < (unsigned)g.Hp;
      rows[r] = ok ? x + ((size_t)(ts * g.Hp + ys) * g.Wp) * g.C + c : nullptr;
      // the window before the row's first token: positions -rx - 1 .. rx - 1
#pragma unroll
      for (int f = 1; f < CX; ++f) {
        const int xs = f - 1 - rx;
        ld8(rows[r] && (unsigned)xs < (unsigned)g.Wp ? rows[r] + (size_t)xs * g.C : zero, win[r][f]);
      }
    }
    for (int xx = 0; xx < g.Wp; ++xx) {
      float d[8];
      ld8(dy + ((size_t)(t * g.Hp + yy) * g.Wp + xx) * g.C + c, d);
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        // slide: positions xx - rx .. xx + rx
#pragma unroll
        for (int f = 0; f < CX - 1; ++f)
#pragma unroll
          for (int e = 0; e < 8; ++e) win[r][f][e] = win[r][f + 1][e];
        const int xs = xx + rx;
        ld8(rows[r] && xs < g.Wp ? rows[r] + (size_t)xs * g.C : zero, win[r][CX - 1]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) bs[e] += d[e];
#pragma unroll
      for (int r = 0; r < ROWS; ++r)
#pragma unroll
        for (int f = 0; f < CX; ++f)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[r][f][e] = fmaf(d[e], win[r][f][e], acc[r][f][e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float* p = part + (((size_t)t * sp.nyc + yc) * g.C + c + e) * (g.taps + 1);
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
      if (row0 + r < g.ct * g.cy)
#pragma unroll
        for (int f = 0; f < CX; ++f) p[(row0 + r) * CX + f] = acc[r][f][e];
    if (tc == 0) p[g.taps] = bs[e];
  }
}

// dw[c][tap] (and db[c]) = sum of the partial sums, frames and row spans in order.
__global__ __launch_bounds__(256) void k_dwconv_dw_sum(const float* __restrict__ part, float* __restrict__ dw,
                                                       float* __restrict__ db, CGeom g, int nparts) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long per = (long long)g.C * (g.taps + 1);
  if (i >= per) return;
  float s = 0.f;
  for (int t = 0; t < nparts; ++t) s += part[(size_t)t * per + i];
  const int c = (int)(i / (g.taps + 1)), tap = (int)(i - (long long)c * (g.taps + 1));
  if (tap < g.taps) {
    dw[(size_t)c * g.taps + tap] = s;
  } else if (db) {
    db[c] = s;
  }
}

// ---- frame-sweeping forms: filters up to 3 x 3 x 3, C a multiple of 64 ------------
// A block owns a TB_Y x TB_X tile of token positions and TB_C channels and sweeps a
// run of frames.  The input slices of the frames its taps read -- the tile plus a halo
// of (cy - 1) / 2 rows and (cx - 1) / 2 columns, [token][TB_C] in LDS -- sit in a ring
// of TB_RING slices, one new slice per output frame, so every input row comes from
// memory about once (halo aside) instead of once per tap row.  The next frame's slice is
// loaded into registers while the current frame is computed.
constexpr int TB_Y = 8, TB_X = 16, TB_C = 64, TB_RING = 3;

template <typename T, int CY, int CX>
struct Tube {
  static constexpr int SY = TB_Y + CY - 1, SX = TB_X + CX - 1, SLICE = SY * SX;  // slice rows, columns, tokens
  static constexpr int CH = SLICE * (TB_C / 8);   // 8-channel chunks per slice
  static constexpr int LOADS = (CH + 255) / 256;  // chunks per thread
};

// 8 consecutive elements as one or two 16-byte words
template <typename T> struct Chunk8;
template <> struct Chunk8<u16> { uint4 a; };
template <> struct Chunk8<float> { uint4 a, b; };
__device__ __forceinline__ Chunk8<u16> ld_chunk(const u16* p) { return {*reinterpret_cast<const uint4*>(p)}; }
__device__ __forceinline__ Chunk8<float> ld_chunk(const float* p) {
  return {reinterpret_cast<const uint4*>(p)[0], reinterpret_cast<const uint4*>(p)[1]};
}
__device__ __forceinline__ void st_chunk(u16* p, const Chunk8<u16>& c) { *reinterpret_cast<uint4*>(p) = c.a; }
__device__ __forceinline__ void st_chunk(float* p, const Chunk8<float>& c) {
  reinterpret_cast<uint4*>(p)[0] = c.a;
  reinterpret_cast<uint4*>(p)[1] = c.b;
}

// Block order: tile column fastest, then tile row, frame run, channel block, each XCD
// given a contiguous run (neighbouring tiles share their halo rows in one L2).
struct TubeBlock {
  int c0, y0, x0, t0, t1;
};
__device__ __forceinline__ TubeBlock tube_block(const CGeom& g, int fchunk) {
  const int ntx = (g.Wp + TB_X - 1) / TB_X, nty = (g.Hp + TB_Y - 1) / TB_Y;
  const int nfc = (g.F + fchunk - 1) / fchunk, ncb = g.C / TB_C;
  int L = xcd_remap(blockIdx.x, ncb * nfc * nty * ntx);
  TubeBlock b;
  const int tx = L % ntx;
  L /= ntx;
  const int ty = L % nty;
  L /= nty;
  const int fc = L % nfc;
  b.c0 = (L / nfc) * TB_C;
  b.y0 = ty * TB_Y;
  b.x0 = tx * TB_X;
  b.t0 = fc * fchunk;
  b.t1 = min(b.t0 + fchunk, g.F);
  return b;
}

// A thread's share of a block's frame slices: U::LOADS chunks at offsets within a frame
// that are fixed per block.  Every load is issued (chunks outside the grid read the
// tensor's first chunk) and every chunk written to LDS (those past the slice to a dummy
// chunk), the ones outside the grid zeroed by a mask on the way: no branch around a load
// or its use, so the compiler's wait for a slice's loads sits at one unconditional place
// rather than being repeated, conservatively, at the top of the next frame.
__device__ __forceinline__ Chunk8<u16> mask_chunk(const Chunk8<u16>& c, uint32_t m) {
  return {make_uint4(c.a.x & m, c.a.y & m, c.a.z & m, c.a.w & m)};
}
__device__ __forceinline__ Chunk8<float> mask_chunk(const Chunk8<float>& c, uint32_t m) {
  return {make_uint4(c.a.x & m, c.a.y & m, c.a.z & m, c.a.w & m), make_uint4(c.b.x & m, c.b.y & m, c.b.z & m, c.b.w & m)};
}
template <typename T, int CY, int CX>
struct TubeSlices {
  using U = Tube<T, CY, CX>;
  long long off[U::LOADS];  // element offset within a frame, -1 outside the grid or past the slice
  long long fstride;
  int F;
  __device__ __forceinline__ TubeSlices(const CGeom& g, const TubeBlock& b) {
    constexpr int ry = (CY - 1) / 2, rx = (CX - 1) / 2;
    fstride = (long long)g.Hp * g.Wp * g.C;
    F = g.F;
#pragma unroll
    for (int k = 0; k < U::LOADS; ++k) {
      const int j = threadIdx.x + 256 * k;
      const int tok = j >> 3, sy = tok / U::SX, sx = tok - sy * U::SX;
      const int gy = b.y0 - ry + sy, gx = b.x0 - rx + sx;
      const bool ok = j < U::CH && (unsigned)gy < (unsigned)g.Hp && (unsigned)gx < (unsigned)g.Wp;
      off[k] = ok ? ((long long)gy * g.Wp + gx) * g.C + b.c0 + (j & 7) * 8 : -1;
    }
  }
  __device__ __forceinline__ void load(const T* __restrict__ x, int f, Chunk8<T>* buf) const {
    const bool fin = (unsigned)f < (unsigned)F;
#pragma unroll
    for (int k = 0; k < U::LOADS; ++k)
      buf[k] = ld_chunk(x + ((fin && off[k] >= 0) ? (size_t)f * fstride + off[k] : (size_t)0));
  }
  __device__ __forceinline__ void store(T* slot, T* dummy, int f, const Chunk8<T>* buf) const {
    const bool fin = (unsigned)f < (unsigned)F;
#pragma unroll
    for (int k = 0; k < U::LOADS; ++k) {
      const int j = threadIdx.x + 256 * k;
      st_chunk(j < U::CH ? slot + (size_t)j * 8 : dummy, mask_chunk(buf[k], (fin && off[k] >= 0) ? ~0u : 0u));
    }
  }
};
__device__ __forceinline__ int ring_slot(int f) { return ((f % TB_RING) + TB_RING) % TB_RING; }

template <typename T> struct Dy2;  // 2 consecutive elements
template <> struct Dy2<u16> { uint32_t v; };
template <> struct Dy2<float> { float2 v; };
__device__ __forceinline__ void dy2_unpack(const Dy2<u16>& d, float* x) {
  x[0] = __uint_as_float(d.v << 16);
  x[1] = __uint_as_float(d.v & 0xffff0000u);
}
__device__ __forceinline__ void dy2_unpack(const Dy2<float>& d, float* x) {
  x[0] = d.v.x;
  x[1] = d.v.y;
}
__device__ __forceinline__ void ld2(const u16* p, float* x) { dy2_unpack(Dy2<u16>{*reinterpret_cast<const uint32_t*>(p)}, x); }
__device__ __forceinline__ void ld2(const float* p, float* x) { dy2_unpack(Dy2<float>{*reinterpret_cast<const float2*>(p)}, x); }

__device__ __forceinline__ void store2(u16* p, float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  *reinterpret_cast<bf16x2_t*>(p) = __builtin_convertvector((f32x2_t{a, b}), bf16x2_t);
}
__device__ __forceinline__ void store2(float* p, float a, float b) { *reinterpret_cast<float2*>(p) = make_float2(a, b); }

// Forward (or, with the filters mirrored, the input gradient): thread (cg2, patch)
// computes a 4 x 4 patch of the tile (rows 4 (cp >> 2) .. + 3, columns 4 (cp & 3) .. + 3)
// for 2 channels, with those channels' filters in registers (read once from the block's
// copy in LDS, [tap][channel] fp32).  Per frame offset and window row it widens the
// 4 + cx - 1 input columns once and uses each for every (filter row, filter column,
// patch column) that reads it: 4 products per widened value, where a thread that owns a
// column of 8 rows gets 2.4 (a wave reads two neighbouring tokens' 128 bytes at a time).
// Every global load of a frame -- the next slice and, with accumulate, the output's old
// values -- is issued at the frame's start and its data used only after the products;
// no load, LDS write or register copy of the frame loop sits behind a branch (chunks
// outside the grid are loaded from a valid address and zeroed by a mask on the way to
// LDS; the last frame of a run loads and writes to its free ring slot a slice nobody
// reads), so the compiler's waits for the loads sit where the data is used.
template <typename T, int CY, int CX, bool ACC>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) void k_dwconv_tube(
    const T* __restrict__ x, const float* __restrict__ w, const float* __restrict__ b, T* __restrict__ y, CGeom g,
    int fchunk, int flip) {
  using U = Tube<T, CY, CX>;
  constexpr int NT = 3 * CY * CX;  // tap slots (ct <= 3)
  constexpr int PR = 4, PC = 4;    // patch rows, columns
  constexpr int WR = PR + CY - 1, WC = PC + CX - 1;  // input window rows, columns
  static_assert(PR * 2 == TB_Y && PC * 4 == TB_X, "8 patches of 4 x 4 tokens per tile");
  __shared__ __attribute__((aligned(16))) T ring[TB_RING][U::SLICE * TB_C];
  __shared__ __attribute__((aligned(16))) float wl[NT + 1][TB_C];  // taps, then the bias
  __shared__ __attribute__((aligned(16))) T dummy[8];
  const int tid = threadIdx.x;
  const TubeBlock bk = tube_block(g, fchunk);
  const int rt = (g.ct - 1) / 2;
  const int cg2 = tid & 31, cp = tid >> 5;
  const int pr0 = PR * (cp >> 2), pc0 = PC * (cp & 3);  // the patch's first tile row, column
  const int c = bk.c0 + cg2 * 2;
  // filters (the tap index runs fastest in global memory; mirrored for the input
  // gradient) and bias through LDS, so that every load of the prologue is complete before
  // the frame loop
  for (int i = tid; i < TB_C * g.taps; i += 256) {
    const int ch = i / g.taps, tap = i - ch * g.taps;
    wl[flip ? g.taps - 1 - tap : tap][ch] = w[(size_t)bk.c0 * g.taps + i];
  }
  for (int i = g.taps * TB_C + tid; i < NT * TB_C; i += 256) wl[i / TB_C][i % TB_C] = 0.f;
  if (tid < TB_C) wl[NT][tid] = (b && !flip) ? b[bk.c0 + tid] : 0.f;
  const TubeSlices<T, CY, CX> sl_io(g, bk);
  const long long fstride = sl_io.fstride;
  Chunk8<T> pre[U::LOADS];
  for (int f = bk.t0 - rt; f <= bk.t0 + rt; ++f) {
    sl_io.load(x, f, pre);
    sl_io.store(ring[ring_slot(f)], dummy, f, pre);
  }
  __syncthreads();
  float wr[NT][2];
#pragma unroll
  for (int tap = 0; tap < NT; ++tap) {
    const float2 t2 = *reinterpret_cast<const float2*>(&wl[tap][cg2 * 2]);
    wr[tap][0] = t2.x;
    wr[tap][1] = t2.y;
  }
  const float2 bv = *reinterpret_cast<const float2*>(&wl[NT][cg2 * 2]);
  // this thread's output tokens: offsets within a frame (first element of its 2 channels)
  // and whether they lie inside the grid
  uint32_t omask = 0;  // bit i * PC + j
#pragma unroll
  for (int i = 0; i < PR; ++i)
#pragma unroll
    for (int j = 0; j < PC; ++j)
      if (bk.y0 + pr0 + i < g.Hp && bk.x0 + pc0 + j < g.Wp) omask |= 1u << (i * PC + j);
  const size_t obase = ((size_t)(bk.y0 + pr0) * g.Wp + bk.x0 + pc0) * g.C + c;
  auto oofs = [&](int i, int j) { return obase + ((size_t)i * g.Wp + j) * g.C; };
  for (int t = bk.t0; t < bk.t1; ++t) {
    sl_io.load(x, t + 1 + rt, pre);
    Dy2<T> old[PR * PC];
    if constexpr (ACC) {
#pragma unroll
      for (int i = 0; i < PR; ++i)
#pragma unroll
        for (int j = 0; j < PC; ++j) {
          const bool in = (omask >> (i * PC + j)) & 1u;
          old[i * PC + j] =
              *reinterpret_cast<const Dy2<T>*>(y + (in ? (size_t)t * fstride + oofs(i, j) : (size_t)0));
        }
    }
    float acc[PR][PC][2];
#pragma unroll
    for (int i = 0; i < PR; ++i)
#pragma unroll
      for (int j = 0; j < PC; ++j) {
        acc[i][j][0] = bv.x;
        acc[i][j][1] = bv.y;
      }
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      if (a >= g.ct) break;
      const T* sl = ring[ring_slot(t - rt + a)];
#pragma unroll
      for (int p = 0; p < WR; ++p) {
        // input window row p (patch row p - e2 for filter row e2), columns 0 .. WC - 1
        float xw[WC][2];
#pragma unroll
        for (int q = 0; q < WC; ++q) ld2(sl + ((pr0 + p) * U::SX + pc0 + q) * TB_C + cg2 * 2, xw[q]);
#pragma unroll
        for (int e2 = 0; e2 < CY; ++e2) {
          const int i = p - e2;
          if (i < 0 || i >= PR) continue;
#pragma unroll
          for (int f = 0; f < CX; ++f) {
            const int tap = (a * CY + e2) * CX + f;
#pragma unroll
            for (int j = 0; j < PC; ++j) {
              acc[i][j][0] = fmaf(wr[tap][0], xw[j + f][0], acc[i][j][0]);
              acc[i][j][1] = fmaf(wr[tap][1], xw[j + f][1], acc[i][j][1]);
            }
          }
        }
      }
    }
    __syncthreads();  // every read of the leaving frame's slice is done
    // the next slice into LDS before the output stores, so that waiting for its loads
    // never means waiting for stores
    sl_io.store(ring[ring_slot(t + 1 + rt)], dummy, t + 1 + rt, pre);
    if constexpr (ACC) {
#pragma unroll
      for (int i = 0; i < PR; ++i)
#pragma unroll
        for (int j = 0; j < PC; ++j) {
          float o[2];
          dy2_unpack(old[i * PC + j], o);
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            acc[i][j][e] += o[e];
            // keeps the add (and so the wait for the old value) out of the conditional
            // store below, where the compiler would otherwise sink it
            __asm__ __volatile__("" ::"v"(acc[i][j][e]));
          }
        }
    }
#pragma unroll
    for (int i = 0; i < PR; ++i)
#pragma unroll
      for (int j = 0; j < PC; ++j)
        if ((omask >> (i * PC + j)) & 1u) store2(y + (size_t)t * fstride + oofs(i, j), acc[i][j][0], acc[i][j][1]);
    __syncthreads();
  }
}

// Filter / bias gradient over the same tiles: thread (cg2, cp) keeps the partial sums of
// all taps for 2 channels over a 4 x 4 patch of the tile (rows 4 (cp >> 2) .. + 3,
// columns 4 (cp & 3) .. + 3), its dy values in registers, loaded a frame ahead like the
// slices.  Per frame offset and window row it unpacks the 4 + cx - 1 input columns once
// and uses each for every (filter row, filter column, patch column) that reads it (a
// wave reads two neighbouring tokens' 128 bytes at a time).  At the end the 8 patches'
// sums are added pairwise in LDS in a fixed order and the block writes its part,
// [part][C][taps + 1] as k_dwconv_dw_sum reads it (part = (frame run, tile row, tile
// column)).
template <typename T, int CY, int CX>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) void k_dwconv_dw_tube(const T* __restrict__ x, const T* __restrict__ dy,
                                                           float* __restrict__ part, CGeom g, int fchunk) {
  using U = Tube<T, CY, CX>;
  constexpr int NT = 3 * CY * CX;  // tap slots (ct <= 3)
  constexpr int PR = 4, PC = 4;    // patch rows, columns
  constexpr int WR = PR + CY - 1, WC = PC + CX - 1;  // input window rows, columns
  static_assert(PR * 2 == TB_Y && PC * 4 == TB_X, "8 patches of 4 x 4 tokens per tile");
  __shared__ __attribute__((aligned(16))) T ring[TB_RING][U::SLICE * TB_C];
  __shared__ __attribute__((aligned(16))) T dummy[8];
  const int tid = threadIdx.x;
  const TubeBlock bk = tube_block(g, fchunk);
  const int rt = (g.ct - 1) / 2;
  const int cg2 = tid & 31, cp = tid >> 5;
  const int pr0 = PR * (cp >> 2), pc0 = PC * (cp & 3);  // the patch's first tile row, column
  const int c = bk.c0 + cg2 * 2;
  const TubeSlices<T, CY, CX> sl_io(g, bk);
  // this thread's dy values of frame f: the patch's PR x PC tokens, loaded unconditionally
  // (from the tensor's start outside the grid) and zeroed by dmask on use
  uint32_t dmask = 0;  // bit i * PC + j: patch token (i, j) is inside the grid
#pragma unroll
  for (int i = 0; i < PR; ++i)
#pragma unroll
    for (int j = 0; j < PC; ++j)
      if (bk.y0 + pr0 + i < g.Hp && bk.x0 + pc0 + j < g.Wp) dmask |= 1u << (i * PC + j);
  auto dy_fetch = [&](int f, Dy2<T>* buf) {
#pragma unroll
    for (int i = 0; i < PR; ++i)
#pragma unroll
      for (int j = 0; j < PC; ++j) {
        const bool in = ((dmask >> (i * PC + j)) & 1u) && f < g.F;
        const size_t o = ((size_t)(f * g.Hp + bk.y0 + pr0 + i) * g.Wp + bk.x0 + pc0 + j) * g.C + c;
        buf[i * PC + j] = *reinterpret_cast<const Dy2<T>*>(dy + (in ? o : (size_t)0));
      }
  };
  Chunk8<T> pre[U::LOADS];
  Dy2<T> dcur[PR * PC], dnext[PR * PC];
  for (int f = bk.t0 - rt; f <= bk.t0 + rt; ++f) {
    sl_io.load(x, f, pre);
    sl_io.store(ring[ring_slot(f)], dummy, f, pre);
  }
  dy_fetch(bk.t0, dcur);
  // the first frame's dy arrives before the frame loop, as every later frame's does (its
  // copy into dcur waits for it), so the loop's products need no wait for the loads in flight
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  float acc[NT + 1][2];  // taps, then the bias
#pragma unroll
  for (int i = 0; i <= NT; ++i) acc[i][0] = acc[i][1] = 0.f;
  // as in the forward, the last frame of the run loads and stores a slice (and loads dy
  // rows) that are never used, so that no load, LDS write or copy sits behind a branch
  for (int t = bk.t0; t < bk.t1; ++t) {
    sl_io.load(x, t + 1 + rt, pre);
    dy_fetch(t + 1, dnext);
    float d[PR][PC][2];
#pragma unroll
    for (int i = 0; i < PR; ++i)
#pragma unroll
      for (int j = 0; j < PC; ++j) {
        dy2_unpack(dcur[i * PC + j], d[i][j]);
        if (!((dmask >> (i * PC + j)) & 1u)) d[i][j][0] = d[i][j][1] = 0.f;
        acc[NT][0] += d[i][j][0];
        acc[NT][1] += d[i][j][1];
      }
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      if (a >= g.ct) break;
      const T* sl = ring[ring_slot(t - rt + a)];
#pragma unroll
      for (int p = 0; p < WR; ++p) {
        // input window row p (patch row p - e2 for filter row e2), columns 0 .. WC - 1
        float xw[WC][2];
#pragma unroll
        for (int q = 0; q < WC; ++q) ld2(sl + ((pr0 + p) * U::SX + pc0 + q) * TB_C + cg2 * 2, xw[q]);
#pragma unroll
        for (int e2 = 0; e2 < CY; ++e2) {
          const int i = p - e2;
          if (i < 0 || i >= PR) continue;
#pragma unroll
          for (int f = 0; f < CX; ++f) {
            const int tap = (a * CY + e2) * CX + f;
#pragma unroll
            for (int j = 0; j < PC; ++j) {
              acc[tap][0] = fmaf(d[i][j][0], xw[j + f][0], acc[tap][0]);
              acc[tap][1] = fmaf(d[i][j][1], xw[j + f][1], acc[tap][1]);
            }
          }
        }
      }
    }
    __syncthreads();
    sl_io.store(ring[ring_slot(t + 1 + rt)], dummy, t + 1 + rt, pre);
#pragma unroll
    for (int i = 0; i < PR * PC; ++i) dcur[i] = dnext[i];
    __syncthreads();
  }
  // patches 0 .. 7: add patch cp + h into patch cp for h = 4, 2, 1, through LDS
  float* red = reinterpret_cast<float*>(&ring[0][0]);  // [pair][NT + 1][32 cg2][2]
  constexpr int PER = (NT + 1) * 64;                   // floats per pair
  static_assert(4 * PER * 4 <= (int)sizeof(ring), "the reduction fits in the ring");
  for (int h = 4; h >= 1; h >>= 1) {
    if (cp >= h && cp < 2 * h)
#pragma unroll
      for (int i = 0; i <= NT; ++i)
        *reinterpret_cast<float2*>(red + (cp - h) * PER + (i * 32 + cg2) * 2) = make_float2(acc[i][0], acc[i][1]);
    __syncthreads();
    if (cp < h)
#pragma unroll
      for (int i = 0; i <= NT; ++i) {
        const float2 o = *reinterpret_cast<const float2*>(red + cp * PER + (i * 32 + cg2) * 2);
        acc[i][0] += o.x;
        acc[i][1] += o.y;
      }
    __syncthreads();
  }
  if (cp == 0) {
    const int ntx = (g.Wp + TB_X - 1) / TB_X, nty = (g.Hp + TB_Y - 1) / TB_Y;
    const int pidx = ((bk.t0 / fchunk) * nty + bk.y0 / TB_Y) * ntx + bk.x0 / TB_X;
    float* out = part + ((size_t)pidx * g.C + c) * (g.taps + 1);
    // tap slot (a, e, f) of this kernel is filter tap (a * cy + e) * cx + f (cy = CY, cx = CX)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      static_for<0, NT>([&](auto TC) {
        constexpr int tap = decltype(TC)::value;
        if (tap < g.taps) out[(size_t)e * (g.taps + 1) + tap] = acc[tap][e];
      });
      out[(size_t)e * (g.taps + 1) + g.taps] = acc[NT][e];
    }
  }
}

// The frame-sweeping forms: filters up to 3 x 3 x 3 (odd sides), C a multiple of 64.
static bool tube_ok(const CGeom& g) {
  return g.C % TB_C == 0 && g.ct <= 3 && (g.cy == 1 || g.cy == 3) && (g.cx == 1 || g.cx == 3);
}
// Frames per block: the run length, among the clip split into 1 .. 64 runs, whose blocks
// fill the chip's block slots (256 CUs x 2 resident blocks) in whole rounds best, weighed
// against the ct - 1 extra frames each run loads (a last, partly filled round of blocks
// leaves CUs idle).  A function of the geometry only: the filter gradient's workspace is
// sized with it.
static int tube_fchunk(const CGeom& g) {
  constexpr long long SLOTS = 512;
  const long long tiles =
      (long long)(g.C / TB_C) * ((g.Hp + TB_Y - 1) / TB_Y) * ((g.Wp + TB_X - 1) / TB_X);
  int best = g.F;
  double best_eff = -1.0;
  for (int nfc = 1; nfc <= std::min(g.F, 64); ++nfc) {
    const int fchunk = (g.F + nfc - 1) / nfc;
    const long long blocks = tiles * ((g.F + fchunk - 1) / fchunk);
    const long long rounds = (blocks + SLOTS - 1) / SLOTS;
    const double eff = (double)blocks / (double)(rounds * SLOTS) * fchunk / (double)(fchunk + g.ct - 1);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = fchunk;
    }
  }
  return best;
}
static long long tube_parts(const CGeom& g) {  // filter-gradient parts per channel
  const int fchunk = tube_fchunk(g);
  return (long long)((g.F + fchunk - 1) / fchunk) * ((g.Hp + TB_Y - 1) / TB_Y) * ((g.Wp + TB_X - 1) / TB_X);
}
static unsigned tube_blocks(const CGeom& g) { return (unsigned)(tube_parts(g) * (g.C / TB_C)); }

template <typename T, int CY, int CX>
static hipError_t tube_conv(const void* x, const float* w, const float* b, void* y, const CGeom& g, int acc,
                            int flip, hipStream_t s) {
  if (acc)
    k_dwconv_tube<T, CY, CX, true><<<tube_blocks(g), 256, 0, s>>>((const T*)x, w, b, (T*)y, g, tube_fchunk(g), flip);
  else
    k_dwconv_tube<T, CY, CX, false><<<tube_blocks(g), 256, 0, s>>>((const T*)x, w, b, (T*)y, g, tube_fchunk(g), flip);
  return hipGetLastError();
}
template <typename T, int CY, int CX>
static hipError_t tube_dw(const void* x, const void* dy, float* part, const CGeom& g, hipStream_t s) {
  k_dwconv_dw_tube<T, CY, CX><<<tube_blocks(g), 256, 0, s>>>((const T*)x, (const T*)dy, part, g, tube_fchunk(g));
  return hipGetLastError();
}
template <typename T>
static hipError_t tube_conv_dispatch(const void* x, const float* w, const float* b, void* y, const CGeom& g, int acc,
                                     int flip, hipStream_t s) {
  if (g.cy == 1) return g.cx == 1 ? tube_conv<T, 1, 1>(x, w, b, y, g, acc, flip, s) : tube_conv<T, 1, 3>(x, w, b, y, g, acc, flip, s);
  return g.cx == 1 ? tube_conv<T, 3, 1>(x, w, b, y, g, acc, flip, s) : tube_conv<T, 3, 3>(x, w, b, y, g, acc, flip, s);
}
template <typename T>
static hipError_t tube_dw_dispatch(const void* x, const void* dy, float* part, const CGeom& g, hipStream_t s) {
  if (g.cy == 1) return g.cx == 1 ? tube_dw<T, 1, 1>(x, dy, part, g, s) : tube_dw<T, 1, 3>(x, dy, part, g, s);
  return g.cx == 1 ? tube_dw<T, 3, 1>(x, dy, part, g, s) : tube_dw<T, 3, 3>(x, dy, part, g, s);
}

template <typename T, int CX>
static hipError_t conv_launch_w(const void* x, const float* w, const float* b, void* y, const CGeom& g, int acc,
                                int flip, hipStream_t s) {
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dwconv_w<T, CX>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     CONV_MAX_TAPS * CONV_CB * 4);
  if (attr != hipSuccess) return attr;
  const long long nquads = (long long)g.F * g.Hp * ((g.Wp + CONV_Q - 1) / CONV_Q);
  const long long total = ((nquads + CONV_TOK - 1) / CONV_TOK) * ((g.C + CONV_CB - 1) / CONV_CB);
  k_dwconv_w<T, CX><<<(unsigned)total, 256, (size_t)g.taps * CONV_CB * 4, s>>>((const T*)x, w, b, (T*)y, g, acc,
                                                                              flip);
  return hipGetLastError();
}

template <typename T>
static hipError_t conv_launch(const void* x, const float* w, const float* b, void* y, const CGeom& g, int acc,
                              int flip, hipStream_t s) {
  if (tube_ok(g)) return tube_conv_dispatch<T>(x, w, b, y, g, acc, flip, s);
  switch (g.cx) {
    case 1: return conv_launch_w<T, 1>(x, w, b, y, g, acc, flip, s);
    case 3: return conv_launch_w<T, 3>(x, w, b, y, g, acc, flip, s);
    case 5: return conv_launch_w<T, 5>(x, w, b, y, g, acc, flip, s);
    case 7: return conv_launch_w<T, 7>(x, w, b, y, g, acc, flip, s);
    case 9: return conv_launch_w<T, 9>(x, w, b, y, g, acc, flip, s);
    default: break;
  }
  const size_t lds = (size_t)g.taps * (CONV_CB + 1) * 4;  // filters and tap shifts, up to 130 KiB
  // dynamic LDS past 64 KiB needs the kernel's limit raised (a host-side attribute)
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dwconv<T>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     CONV_MAX_TAPS * (CONV_CB + 1) * 4);
  if (attr != hipSuccess) return attr;
  const long long nquads = (long long)g.F * g.Hp * ((g.Wp + CONV_Q - 1) / CONV_Q);
  const long long total = ((nquads + CONV_TOK - 1) / CONV_TOK) * ((g.C + CONV_CB - 1) / CONV_CB);
  k_dwconv<T><<<(unsigned)total, 256, lds, s>>>((const T*)x, w, b, (T*)y, g, acc, flip);
  return hipGetLastError();
}

// Filter rows per block of the sliding-window filter-gradient kernel (at most 9 taps a
// thread), 0 where the width has no specialisation.
static int dw_rows(int cx) { return cx == 1 ? 9 : cx == 3 ? 3 : (cx == 5 || cx == 7 || cx == 9) ? 1 : 0; }

// The filter-gradient blocks: channel blocks, tap chunks (filter-row groups for the
// sliding-window kernel, DW_TAPS taps otherwise) and row spans per frame, enough blocks
// to fill the chip (>= 1024) without splitting rows.
static DwSplit dw_split(const CGeom& g) {
  DwSplit sp;
  sp.ncb = (g.C + DW_CPB - 1) / DW_CPB;
  const int rows = dw_rows(g.cx);
  sp.ntc = rows ? (g.ct * g.cy + rows - 1) / rows : (g.taps + DW_TAPS - 1) / DW_TAPS;
  const long long base = (long long)sp.ncb * sp.ntc * g.F;
  sp.nyc = (int)std::min<long long>(g.Hp, std::max<long long>(1, (1024 + base - 1) / base));
  sp.rows = (g.Hp + sp.nyc - 1) / sp.nyc;
  sp.nyc = (g.Hp + sp.rows - 1) / sp.rows;
  return sp;
}

template <typename T>
static hipError_t dw_launch(const void* x, const void* dy, float* part, const CGeom& g, const DwSplit& sp,
                            hipStream_t s) {
  const long long total = (long long)sp.ncb * sp.ntc * sp.nyc * g.F;
  k_dwconv_dw<T><<<(unsigned)total, 256, 0, s>>>((const T*)x, (const T*)dy, part, g, sp);
  return hipGetLastError();
}

// Filter rows per block for the sliding-window kernel: at most 9 taps a thread.
template <typename T, int ROWS, int CX>
static hipError_t dw_launch_w(const void* x, const void* dy, float* part, const CGeom& g, hipStream_t s) {
  const DwSplit sp = dw_split(g);  // ntc = filter-row groups of ROWS (dw_rows(CX) == ROWS)
  const long long total = (long long)sp.ncb * sp.ntc * sp.nyc * g.F;
  k_dwconv_dw_w<T, ROWS, CX><<<(unsigned)total, 256, 0, s>>>((const T*)x, (const T*)dy, part, g, sp);
  return hipGetLastError();
}

template <typename T>
static hipError_t dw_dispatch(const void* x, const void* dy, float* part, const CGeom& g, hipStream_t s) {
  switch (g.cx) {
    case 1: return dw_launch_w<T, 9, 1>(x, dy, part, g, s);
    case 3: return dw_launch_w<T, 3, 3>(x, dy, part, g, s);
    case 5: return dw_launch_w<T, 1, 5>(x, dy, part, g, s);
    case 7: return dw_launch_w<T, 1, 7>(x, dy, part, g, s);
    case 9: return dw_launch_w<T, 1, 9>(x, dy, part, g, s);
    default: return dw_launch<T>(x, dy, part, g, dw_split(g), s);
  }
}

}  // namespace dsa3d

using namespace dsa3d;

namespace {

int check_conv(const void* x, const float* w, int F, int Hp, int Wp, int C, int ct, int cy, int cx, int dtype,
               CGeom* g) {
  if (!x || !w) return DSA3D_ERR_NULL;
  if (dtype != DSA3D_F32 && dtype != DSA3D_BF16) return DSA3D_ERR_DTYPE;
  if (F < 1 || Hp < 1 || Wp < 1 || C < 8 || (C & 7) || (long long)F * Hp * Wp >= (1LL << 30) ||
      (long long)F * Hp * Wp * C >= (1LL << 40))
    return DSA3D_ERR_GRID;
  if (ct < 1 || cy < 1 || cx < 1 || !(ct & 1) || !(cy & 1) || !(cx & 1) || ct * cy * cx > CONV_MAX_TAPS)
    return DSA3D_ERR_WINDOW;
  if (((uintptr_t)x & 15u) || ((uintptr_t)w & 3u)) return DSA3D_ERR_ALIGN;
  g->F = F; g->Hp = Hp; g->Wp = Wp; g->C = C;
  g->ct = ct; g->cy = cy; g->cx = cx; g->taps = ct * cy * cx;
  g->N = F * Hp * Wp;
  return DSA3D_OK;
}

// filter-gradient parts: [parts][C][taps + 1] fp32
long long conv_parts(const CGeom& g) { return tube_ok(g) ? tube_parts(g) : (long long)g.F * dw_split(g).nyc; }
size_t conv_ws(const CGeom& g) { return (((size_t)conv_parts(g) * g.C * (g.taps + 1) * 4) + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

int dsa3d_dwconv3d_forward(const void* x, const float* weight, const float* bias, int F, int Hp, int Wp, int C, int ct,
                           int cy, int cx, int dtype, void* y, int accumulate, hipStream_t stream) {
  CGeom g;
  const int st = check_conv(x, weight, F, Hp, Wp, C, ct, cy, cx, dtype, &g);
  if (st != DSA3D_OK) return st;
  if (!y) return DSA3D_ERR_NULL;
  if (((uintptr_t)y & 15u) || ((uintptr_t)bias & 3u)) return DSA3D_ERR_ALIGN;
  const hipError_t e = dtype == DSA3D_BF16 ? conv_launch<u16>(x, weight, bias, y, g, accumulate != 0, 0, stream)
                                           : conv_launch<float>(x, weight, bias, y, g, accumulate != 0, 0, stream);
  return e == hipSuccess ? DSA3D_OK : DSA3D_ERR_LAUNCH;
}

size_t dsa3d_dwconv3d_workspace_bytes(int F, int Hp, int Wp, int C, int ct, int cy, int cx) {
  CGeom g;
  const int P = 256;
  if (check_conv((void*)(uintptr_t)P, (const float*)(uintptr_t)P, F, Hp, Wp, C, ct, cy, cx, DSA3D_BF16, &g) !=
      DSA3D_OK)
    return 0;
  return conv_ws(g);
}

int dsa3d_dwconv3d_backward(const void* x, const float* weight, const void* dy, int F, int Hp, int Wp, int C, int ct,
                            int cy, int cx, int dtype, void* dx, float* dweight, float* dbias, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  CGeom g;
  const int st = check_conv(x, weight, F, Hp, Wp, C, ct, cy, cx, dtype, &g);
  if (st != DSA3D_OK) return st;
  if (!dy || !dx || !dweight || !workspace) return DSA3D_ERR_NULL;
  if (((uintptr_t)dy & 15u) || ((uintptr_t)dx & 15u) || ((uintptr_t)dweight & 3u) || ((uintptr_t)dbias & 3u) ||
      ((uintptr_t)workspace & 15u))
    return DSA3D_ERR_ALIGN;
  if (workspace_bytes < conv_ws(g)) return DSA3D_ERR_WORKSPACE;
  float* part = static_cast<float*>(workspace);
  const bool bf = dtype == DSA3D_BF16;
  hipError_t e = bf ? conv_launch<u16>(dy, weight, nullptr, dx, g, 0, 1, stream)
                    : conv_launch<float>(dy, weight, nullptr, dx, g, 0, 1, stream);
  if (e != hipSuccess) return DSA3D_ERR_LAUNCH;
  if (tube_ok(g))
    e = bf ? tube_dw_dispatch<u16>(x, dy, part, g, stream) : tube_dw_dispatch<float>(x, dy, part, g, stream);
  else
    e = bf ? dw_dispatch<u16>(x, dy, part, g, stream) : dw_dispatch<float>(x, dy, part, g, stream);
  if (e != hipSuccess) return DSA3D_ERR_LAUNCH;
  const long long per = (long long)g.C * (g.taps + 1);
  k_dwconv_dw_sum<<<(unsigned)((per + 255) / 256), 256, 0, stream>>>(part, dweight, dbias, g, (int)conv_parts(g));
  return hipGetLastError() == hipSuccess ? DSA3D_OK : DSA3D_ERR_LAUNCH;
}

}  // extern "C"
