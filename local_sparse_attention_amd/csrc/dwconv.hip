// Depthwise 3-D convolution over the token grid (MegaSlide-DiT, section "3D Deformable
// Slide Attention": the DWConv3D term of Eq. (1), and the first stage of the offset
// predictor, which the implementation paragraph builds from nn.Conv3d with groups equal
// to the hidden size).  One ct x cy x cx filter per channel, cross-correlation, zero
// padding that keeps the grid:
//   y[n, c] = b[c] + sum_taps w[c][tap] x[n + shift(tap), c]
// Tensors are [N][C] (token n = (t * Hp + y) * Wp + x, channels contiguous).  The
// stencil is HBM-bound: the kernels keep a block's filters in LDS and take each input
// row from L1/L2 for the taps that reuse it.
//   k_dwconv      one thread per (token, 8 channels); forward (optionally adding into y:
//                 the attention output plus the convolution term in one pass) and, with
//                 the taps mirrored, the input gradient dx.
//   k_dwconv_dw   filter and bias gradients, per frame: a block of 32 channels x 8 tap
//                 groups sums dy[n, c] x[n + shift, c] over one frame's tokens; the frames'
//                 partial sums are added in frame order by k_dwconv_dw_sum (deterministic,
//                 no atomics).
#include "dsa3d.h"
#include "internal.hpp"

namespace dsa3d {

struct CGeom {
  int F, Hp, Wp, C;
  int ct, cy, cx, taps;
  int N;
};

constexpr int CONV_CB = 64;      // channels per forward block
constexpr int CONV_TOK = 32;     // tokens per forward block
constexpr int CONV_MAX_TAPS = 512;

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

// flip = 0: y = conv(x) + b (+ y when accumulating).  flip = 1: the transpose (taps
// mirrored, no bias): dx from dy.
template <typename T>
__global__ __launch_bounds__(256) void k_dwconv(const T* __restrict__ x, const float* __restrict__ w,
                                                const float* __restrict__ b, T* __restrict__ y, CGeom g,
                                                int accumulate, int flip) {
  extern __shared__ float lw[];  // [taps][CONV_CB]
  const int tid = threadIdx.x;
  const int c0 = blockIdx.y * CONV_CB;
  for (int i = tid; i < g.taps * CONV_CB; i += 256) {
    const int tap = i / CONV_CB, cl = i - tap * CONV_CB;
    lw[i] = c0 + cl < g.C ? w[(size_t)(c0 + cl) * g.taps + tap] : 0.f;
  }
  __syncthreads();
  const int cg = tid & 7, tl = tid >> 3;
  const int n = blockIdx.x * CONV_TOK + tl;
  const int c = c0 + cg * 8;
  if (n >= g.N || c >= g.C) return;
  const int plane = g.Hp * g.Wp;
  const int t = n / plane, yy = (n - t * plane) / g.Wp, xx = n - t * plane - yy * g.Wp;
  const int rt = (g.ct - 1) / 2, ry = (g.cy - 1) / 2, rx = (g.cx - 1) / 2;
  const int sgn = flip ? -1 : 1;
  float acc[8], v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = (b && !flip) ? b[c + e] : 0.f;
  int tap = 0;
  for (int a = 0; a < g.ct; ++a) {
    const int ts = t + sgn * (a - rt);
    for (int e = 0; e < g.cy; ++e) {
      const int ys = yy + sgn * (e - ry);
      const bool row_in = (unsigned)ts < (unsigned)g.F && (unsigned)ys < (unsigned)g.Hp;
      for (int f = 0; f < g.cx; ++f, ++tap) {
        const int xs = xx + sgn * (f - rx);
        if (!row_in || (unsigned)xs >= (unsigned)g.Wp) continue;
        ld8(x + (size_t)((ts * g.Hp + ys) * g.Wp + xs) * g.C + c, v);
        const float4 w0 = *reinterpret_cast<const float4*>(lw + tap * CONV_CB + cg * 8);
        const float4 w1 = *reinterpret_cast<const float4*>(lw + tap * CONV_CB + cg * 8 + 4);
        acc[0] = fmaf(w0.x, v[0], acc[0]); acc[1] = fmaf(w0.y, v[1], acc[1]);
        acc[2] = fmaf(w0.z, v[2], acc[2]); acc[3] = fmaf(w0.w, v[3], acc[3]);
        acc[4] = fmaf(w1.x, v[4], acc[4]); acc[5] = fmaf(w1.y, v[5], acc[5]);
        acc[6] = fmaf(w1.z, v[6], acc[6]); acc[7] = fmaf(w1.w, v[7], acc[7]);
      }
    }
  }
  T* out = y + (size_t)n * g.C + c;
  if (accumulate) {
    ld8(out, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += v[e];
  }
  st8(out, acc);
}

// Filter / bias gradient partial sums of frame blockIdx.x for 32 channels.  Thread
// (channel lane cl, tap group tg) owns taps tg, tg + 8, ...; tap group 0 also sums dy
// for the bias.  part[(t * C + c) * (taps + 1) + tap], the bias at index taps.
constexpr int DW_CH = 32, DW_TG = 8, DW_MAXT = (CONV_MAX_TAPS + DW_TG - 1) / DW_TG;

template <typename T, int MT>
__global__ __launch_bounds__(256) void k_dwconv_dw(const T* __restrict__ x, const T* __restrict__ dy,
                                                   float* __restrict__ part, CGeom g) {
  const int t = blockIdx.x;
  const int cl = threadIdx.x & (DW_CH - 1), tg = threadIdx.x / DW_CH;
  const int c = blockIdx.y * DW_CH + cl;
  if (c >= g.C) return;
  const int rt = (g.ct - 1) / 2, ry = (g.cy - 1) / 2, rx = (g.cx - 1) / 2;
  float acc[MT], bsum = 0.f;
  int ta[MT], te[MT], tf[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    acc[i] = 0.f;
    const int tap = tg + i * DW_TG;
    const int a = tap / (g.cy * g.cx), r = tap - a * (g.cy * g.cx);
    ta[i] = tap < g.taps ? a - rt : 1 << 20;  // taps past the filter never land in the grid
    te[i] = r / g.cx - ry;
    tf[i] = r - (r / g.cx) * g.cx - rx;
  }
  for (int yy = 0; yy < g.Hp; ++yy)
    for (int xx = 0; xx < g.Wp; ++xx) {
      const int n = (t * g.Hp + yy) * g.Wp + xx;
      const float d = to_f32(dy[(size_t)n * g.C + c]);
      bsum += d;
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int ts = t + ta[i], ys = yy + te[i], xs = xx + tf[i];
        if ((unsigned)ts < (unsigned)g.F && (unsigned)ys < (unsigned)g.Hp && (unsigned)xs < (unsigned)g.Wp)
          acc[i] = fmaf(d, to_f32(x[(size_t)((ts * g.Hp + ys) * g.Wp + xs) * g.C + c]), acc[i]);
      }
    }
  float* pp = part + ((size_t)t * g.C + c) * (g.taps + 1);
#pragma unroll
  for (int i = 0; i < MT; ++i)
    if (tg + i * DW_TG < g.taps) pp[tg + i * DW_TG] = acc[i];
  if (tg == 0) pp[g.taps] = bsum;
}

// dw[c][tap] (and db[c]) = sum over frames in order of the partial sums.
__global__ __launch_bounds__(256) void k_dwconv_dw_sum(const float* __restrict__ part, float* __restrict__ dw,
                                                       float* __restrict__ db, CGeom g) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long per = (long long)g.C * (g.taps + 1);
  if (i >= per) return;
  float s = 0.f;
  for (int t = 0; t < g.F; ++t) s += part[(size_t)t * per + i];
  const int c = (int)(i / (g.taps + 1)), tap = (int)(i - (long long)c * (g.taps + 1));
  if (tap < g.taps) {
    dw[(size_t)c * g.taps + tap] = s;
  } else if (db) {
    db[c] = s;
  }
}

template <typename T>
static hipError_t conv_launch(const void* x, const float* w, const float* b, void* y, const CGeom& g, int acc,
                              int flip, hipStream_t s) {
  const size_t lds = (size_t)g.taps * CONV_CB * 4;  // the block's filters, up to 128 KiB
  // dynamic LDS past 64 KiB needs the kernel's limit raised (a host-side attribute)
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dwconv<T>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     CONV_MAX_TAPS * CONV_CB * 4);
  if (attr != hipSuccess) return attr;
  dim3 grid((g.N + CONV_TOK - 1) / CONV_TOK, (g.C + CONV_CB - 1) / CONV_CB);
  k_dwconv<T><<<grid, 256, lds, s>>>((const T*)x, w, b, (T*)y, g, acc, flip);
  return hipGetLastError();
}

template <typename T, int MT>
static void dw_launch(const void* x, const void* dy, float* part, const CGeom& g, hipStream_t s) {
  dim3 grid(g.F, (g.C + DW_CH - 1) / DW_CH);
  k_dwconv_dw<T, MT><<<grid, 256, 0, s>>>((const T*)x, (const T*)dy, part, g);
}

template <typename T>
static hipError_t dw_dispatch(const void* x, const void* dy, float* part, const CGeom& g, hipStream_t s) {
  const int mt = (g.taps + DW_TG - 1) / DW_TG;
  if (mt <= 4) dw_launch<T, 4>(x, dy, part, g, s);
  else if (mt <= 8) dw_launch<T, 8>(x, dy, part, g, s);
  else if (mt <= 16) dw_launch<T, 16>(x, dy, part, g, s);
  else if (mt <= 32) dw_launch<T, 32>(x, dy, part, g, s);
  else dw_launch<T, DW_MAXT>(x, dy, part, g, s);
  return hipGetLastError();
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

size_t conv_ws(const CGeom& g) { return (((size_t)g.F * g.C * (g.taps + 1) * 4) + 255) & ~(size_t)255; }

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
  e = bf ? dw_dispatch<u16>(x, dy, part, g, stream) : dw_dispatch<float>(x, dy, part, g, stream);
  if (e != hipSuccess) return DSA3D_ERR_LAUNCH;
  const long long per = (long long)g.C * (g.taps + 1);
  k_dwconv_dw_sum<<<(unsigned)((per + 255) / 256), 256, 0, stream>>>(part, dweight, dbias, g);
  return hipGetLastError() == hipSuccess ? DSA3D_OK : DSA3D_ERR_LAUNCH;
}

}  // extern "C"
