// Sampled windows of 3D Deformable Slide Attention (MegaSlide-DiT, section "3D
// Deformable Slide Attention": keys and values sampled at real offset positions by
// trilinear interpolation, softmax over the kt x kh x kw samples, Eq. (1) attention
// term; the implementation paragraph samples with grid_sample, bilinear mode, 5-D).
//
// A sample at position P (token units along t, y, x) blends the 8 grid rows
// floor(P) + {0,1}^3 with weights prod_d (bit_d ? f_d : 1 - f_d), f = P - floor(P);
// rows outside the grid are zero.  Two ways of placing sample (u, v, w) of the query
// at p, with offsets o read at element strides (sn, sh, ss) per token, head, sample:
//   box:  one offset per (query, head); s_d = clamp(p_d + o_d - (k_d - 1)/2, 0, G_d - k_d)
//         and the sample sits at s + (u, v, w)  (integer offsets: the integer windows);
//   free: the sample sits at p + (u, v, w) - (k - 1)/2 + its own offset.
// Positions are kept as integer part plus fraction: the fraction of p + integer + o is
// o - floor(o), exact in fp32, so the weights do not lose bits at large coordinates.
//
// Kernels (all VALU and gathers: with per-sample positions there is no shared key tile
// for matrix cores to work on):
//   forward     one wave per (query, head); D/8 lanes per sample (8 elements a lane),
//               64/(D/8) samples in flight, an online softmax per lane group, groups
//               merged at the end; writes O and the log-sum-exp.
//   dQ side     the same mapping: recomputes the weights from the log-sum-exp, Delta =
//               dO . O, dz = alpha (dO . v~ - Delta); writes dQ, the offset gradient of
//               every sample (through the interpolation weights) and, per sample, alpha
//               and scale * dz for the key side.
//   dK/dV side  deterministic, no atomics: samples are sorted (stable radix sort) by
//               (head, floor(P)); the wave of key m visits the 8 cells m - {0,1}^3 in a
//               fixed order and their samples in sorted order, adding w alpha dO and
//               w scale dz q.
//   offsets     the per-sample gradients summed over the heads / samples that share an
//               offset entry, in a fixed order.
#include <math.h>

#include "dsa3d.h"
#include "internal.hpp"

namespace dsa3d {

struct SGeom {
  int F, Hp, Wp;
  int kt, ky, kx, K;
  int H, N;
  int mode;               // DSA3D_SAMPLE_BOX / DSA3D_SAMPLE_FREE
  long long sn, sh, ss;   // offset strides in floats (0 = shared)
  float scale;
};

constexpr int EL = 8;  // row elements per lane

__device__ __forceinline__ void load8(const u16* p, float* x) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float* x) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void store8(u16* p, const float* x) {
  store4(p, x[0], x[1], x[2], x[3]);
  store4(p + 4, x[4], x[5], x[6], x[7]);
}
__device__ __forceinline__ void store8(float* p, const float* x) {
  store4(p, x[0], x[1], x[2], x[3]);
  store4(p + 4, x[4], x[5], x[6], x[7]);
}

// Raw 16- (bf16) or 32-byte (fp32) loads of 8 row elements, converted after all the loads
// of a batch are issued, so a lane keeps a batch of corner rows in flight.
template <typename T> struct Raw8;
template <> struct Raw8<u16> { uint4 u; };
template <> struct Raw8<float> { float4 a, b; };
__device__ __forceinline__ Raw8<u16> ldraw(const u16* p) { return {*reinterpret_cast<const uint4*>(p)}; }
__device__ __forceinline__ Raw8<float> ldraw(const float* p) {
  return {reinterpret_cast<const float4*>(p)[0], reinterpret_cast<const float4*>(p)[1]};
}
__device__ __forceinline__ void unraw(const Raw8<u16>& r, float* x) {
  const uint32_t w[4] = {r.u.x, r.u.y, r.u.z, r.u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unraw(const Raw8<float>& r, float* x) {
  x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
  x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
}

__device__ __forceinline__ float dot8(const float* a, const float* b) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < EL; ++i) s = fmaf(a[i], b[i], s);
  return s;
}

// Sum over the G lanes of a sample group (8 or 16 lanes: a half row or a row of the
// wave's DPP rows) by DPP moves, every lane getting the sum: the lanes of a quad swap in
// pairs and then halves (quad_perm 1,0,3,2 and 2,3,0,1), then quads and half rows swap by
// mirroring the half row and the row.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int G>
__device__ __forceinline__ float gsum(float v) {
  static_assert(G == 8 || G == 16, "lane groups are half rows or rows");
  v += dpp_mov<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  if constexpr (G == 16) v += dpp_mov<0x140>(v);  // row_mirror
  return v;
}

// Box start along one axis: integer part, fraction, and whether the clamp is inactive
// (the start then moves with the offset).  |o| <= 2G gives the same start as any larger
// offset and keeps the integer part in range.
__device__ __forceinline__ void box_axis(int p, float o, int k, int G, int& si, float& sf, bool& active) {
  o = fminf(fmaxf(o, -2.f * G), 2.f * G);
  const float fl = floorf(o);
  const int xi = p - (k - 1) / 2 + (int)fl;
  const float xf = o - fl;
  if (xi < 0) {
    si = 0; sf = 0.f; active = false;
  } else if (xi > G - k || (xi == G - k && xf > 0.f)) {
    si = G - k; sf = 0.f; active = false;
  } else {
    si = xi; sf = xf;
    active = (xi > 0 || xf > 0.f) && xi < G - k;
  }
}

// Wave order on the query side: a wave per (token, head), head-major, so that the waves
// of a block and their neighbours in launch order take neighbouring tokens of one head,
// whose windows (and the key rows they read) overlap, and share those rows in the caches
// (3-7% faster than token-major; the key-side kernels keep token-major order, which
// measured faster for them).
struct QPos {
  int p[3];       // query position
  int si[3];      // box: start (integer part)
  float sf[3];    //      start (fraction)
  bool act[3];    //      clamp inactive
  const float* o; // offsets of (query, head)
};

__device__ __forceinline__ QPos query_pos(const SGeom& g, const float* off, int n, int h) {
  QPos q;
  const int plane = g.Hp * g.Wp;
  q.p[0] = n / plane;
  q.p[1] = (n - q.p[0] * plane) / g.Wp;
  q.p[2] = n - q.p[0] * plane - q.p[1] * g.Wp;
  q.o = off + (long long)n * g.sn + (long long)h * g.sh;
  if (g.mode == DSA3D_SAMPLE_BOX) {
    box_axis(q.p[0], q.o[0], g.kt, g.F, q.si[0], q.sf[0], q.act[0]);
    box_axis(q.p[1], q.o[1], g.ky, g.Hp, q.si[1], q.sf[1], q.act[1]);
    box_axis(q.p[2], q.o[2], g.kx, g.Wp, q.si[2], q.sf[2], q.act[2]);
  }
  return q;
}

// Position of sample j = (u, v, w) (lat packs u << 20 | v << 10 | w): floor (i) and
// fraction (f) per axis.
__device__ __forceinline__ void sample_pos_lat(const SGeom& g, const QPos& q, int j, int packed, int* i, float* f) {
  const int lat[3] = {packed >> 20, (packed >> 10) & 1023, packed & 1023};
  if (g.mode == DSA3D_SAMPLE_BOX) {
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      i[d] = q.si[d] + lat[d];
      f[d] = q.sf[d];
    }
  } else {
    const int kk[3] = {g.kt, g.ky, g.kx};
    const int G[3] = {g.F, g.Hp, g.Wp};
    const float* o = q.o + (long long)j * g.ss;
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      const float od = fminf(fmaxf(o[d], -2.f * G[d] - kk[d]), 2.f * G[d] + kk[d]);
      const float fl = floorf(od);
      i[d] = q.p[d] + lat[d] - (kk[d] - 1) / 2 + (int)fl;
      f[d] = od - fl;
    }
  }
}

__device__ __forceinline__ int lattice_of(const SGeom& g, int j) {
  const int u = j / (g.ky * g.kx), r = j - u * (g.ky * g.kx), v = r / g.kx, w = r - v * g.kx;
  return (u << 20) | (v << 10) | w;
}

__device__ __forceinline__ void sample_pos(const SGeom& g, const QPos& q, int j, int* i, float* f) {
  sample_pos_lat(g, q, j, lattice_of(g, j), i, f);
}

// The lattice of every sample (window extents < 1024) in LDS, shared by a block's waves.
constexpr int MAX_SAMPLES = 4096;
__device__ __forceinline__ void fill_lattice(const SGeom& g, int* lat) {
  for (int j = threadIdx.x; j < g.K; j += blockDim.x) lat[j] = lattice_of(g, j);
  __syncthreads();
}

// Corner c (bits t, y, x) of a sample: token (-1 outside the grid) and weight.
__device__ __forceinline__ int corner_tok(const SGeom& g, const int* i, int c) {
  const int t = i[0] + ((c >> 2) & 1), y = i[1] + ((c >> 1) & 1), x = i[2] + (c & 1);
  if ((unsigned)t >= (unsigned)g.F || (unsigned)y >= (unsigned)g.Hp || (unsigned)x >= (unsigned)g.Wp) return -1;
  return (t * g.Hp + y) * g.Wp + x;
}
__device__ __forceinline__ float corner_w(const float* f, int c) {
  const float a = (c & 4) ? f[0] : 1.f - f[0];
  const float b = (c & 2) ? f[1] : 1.f - f[1];
  const float e = (c & 1) ? f[2] : 1.f - f[2];
  return a * b * e;
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void k_sampled_fwd(const T* __restrict__ q, const T* __restrict__ k,
                                                     const T* __restrict__ v, const float* __restrict__ off,
                                                     T* __restrict__ out, float* __restrict__ lse, SGeom g) {
  constexpr int G = D / EL, NG = 64 / G;
  __shared__ int lat[MAX_SAMPLES];
  fill_lattice(g, lat);
  const long long wv = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wv >= (long long)g.N * g.H) return;
  const int h = (int)(wv / g.N), n = (int)(wv - (long long)h * g.N);  // head-major: see wave order
  const int lane = threadIdx.x & 63, grp = lane / G, gl = lane % G;
  const size_t row = ((size_t)n * g.H + h) * D + gl * EL;
  float qf[EL];
  load8(q + row, qf);
  const float sl2 = g.scale * LOG2E;
  const QPos qp = query_pos(g, off, n, h);

  float m = -INFINITY, l = 0.f, acc[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) acc[e] = 0.f;
  for (int j = grp; j < g.K; j += NG) {
    int i[3];
    float f[3];
    sample_pos_lat(g, qp, j, lat[j], i, f);
    float ks[EL], vs[EL], x[EL], wc[8];
    size_t rr[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      // a corner outside the grid or of zero weight reads the query's own row (w = 0)
      const int tok = corner_tok(g, i, c);
      const float w = corner_w(f, c);
      const bool ok = tok >= 0 && w != 0.f;
      wc[c] = ok ? w : 0.f;
      rr[c] = ((size_t)(ok ? tok : n) * g.H + h) * D + gl * EL;
    }
    Raw8<T> kr[8], vr[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) kr[c] = ldraw(k + rr[c]);
#pragma unroll
    for (int c = 0; c < 8; ++c) vr[c] = ldraw(v + rr[c]);
#pragma unroll
    for (int e = 0; e < EL; ++e) ks[e] = vs[e] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      unraw(kr[c], x);
#pragma unroll
      for (int e = 0; e < EL; ++e) ks[e] = fmaf(wc[c], x[e], ks[e]);
      unraw(vr[c], x);
#pragma unroll
      for (int e = 0; e < EL; ++e) vs[e] = fmaf(wc[c], x[e], vs[e]);
    }
    const float s = gsum<G>(dot8(qf, ks)) * sl2;
    const float mn = fmaxf(m, s);
    const float a = exp2f(m - mn), p = exp2f(s - mn);
    l = l * a + p;
#pragma unroll
    for (int e = 0; e < EL; ++e) acc[e] = fmaf(p, vs[e], acc[e] * a);
    m = mn;
  }
  // merge the lane groups (a fixed tree)
#pragma unroll
  for (int mask = G; mask < 64; mask <<= 1) {
    const float m2 = __shfl_xor(m, mask, 64), l2 = __shfl_xor(l, mask, 64);
    const float mn = fmaxf(m, m2);
    const float a1 = m == -INFINITY ? 0.f : exp2f(m - mn), a2 = m2 == -INFINITY ? 0.f : exp2f(m2 - mn);
    l = l * a1 + l2 * a2;
#pragma unroll
    for (int e = 0; e < EL; ++e) acc[e] = acc[e] * a1 + __shfl_xor(acc[e], mask, 64) * a2;
    m = mn;
  }
  if (grp == 0) {
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < EL; ++e) acc[e] *= inv;
    store8(out + row, acc);
    if (gl == 0) lse[(size_t)h * g.N + n] = (m + log2f(l)) * LN2;
  }
}

// ---------------------------------------------------------------------------
// backward, query side: dQ, per-sample coefficients, offset gradients
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void k_sampled_bwd_q(const T* __restrict__ q, const T* __restrict__ k,
                                                       const T* __restrict__ v, const T* __restrict__ o,
                                                       const T* __restrict__ dout, const float* __restrict__ lse,
                                                       const float* __restrict__ off, T* __restrict__ dq,
                                                       float* __restrict__ coef_a, float* __restrict__ coef_g,
                                                       float* __restrict__ gpos, SGeom g) {
  constexpr int G = D / EL, NG = 64 / G;
  __shared__ int lat[MAX_SAMPLES];
  fill_lattice(g, lat);
  const long long wv = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wv >= (long long)g.N * g.H) return;
  const int h = (int)(wv / g.N), n = (int)(wv - (long long)h * g.N);  // head-major: see wave order
  const int lane = threadIdx.x & 63, grp = lane / G, gl = lane % G;
  const size_t row = ((size_t)n * g.H + h) * D + gl * EL;
  float qf[EL], df[EL], x[EL];
  load8(q + row, qf);
  load8(dout + row, df);
  load8(o + row, x);
  const float delta = gsum<G>(dot8(df, x));
  const float sl2 = g.scale * LOG2E;
  const float l2 = lse[(size_t)h * g.N + n] * LOG2E;
  const QPos qp = query_pos(g, off, n, h);
  const size_t e0 = ((size_t)h * g.N + n) * g.K;

  float dqa[EL], gb[3] = {0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < EL; ++e) dqa[e] = 0.f;
  for (int j = grp; j < g.K; j += NG) {
    int i[3];
    float f[3];
    sample_pos_lat(g, qp, j, lat[j], i, f);
    // the 8 corners' weights and weight derivatives (0 for corners outside the grid,
    // which read the query's own row); all 16 corner rows are loaded before any product
    float wc[8], dwc[8][3];
    size_t rr[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int tok = corner_tok(g, i, c);
      const bool ok = tok >= 0;
      const float pt = (c & 4) ? f[0] : 1.f - f[0], py = (c & 2) ? f[1] : 1.f - f[1],
                  px = (c & 1) ? f[2] : 1.f - f[2];
      wc[c] = ok ? pt * py * px : 0.f;
      dwc[c][0] = ok ? ((c & 4) ? 1.f : -1.f) * py * px : 0.f;
      dwc[c][1] = ok ? ((c & 2) ? 1.f : -1.f) * pt * px : 0.f;
      dwc[c][2] = ok ? ((c & 1) ? 1.f : -1.f) * pt * py : 0.f;
      rr[c] = ((size_t)(ok ? tok : n) * g.H + h) * D + gl * EL;
    }
    Raw8<T> kr[8], vr[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) kr[c] = ldraw(k + rr[c]);
#pragma unroll
    for (int c = 0; c < 8; ++c) vr[c] = ldraw(v + rr[c]);
    // Every quantity of the sample is a weighted sum over the corners of the corner dots
    // q . k_c and dO . v_c: K~ . q = sum w_c (q . k_c), and the position derivatives take
    // the weight derivatives instead -- 16 dots rather than 8 blended rows.
    float tk[8], tv[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      unraw(kr[c], x);
      tk[c] = dot8(qf, x);
      unraw(vr[c], x);
      tv[c] = dot8(df, x);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      tk[c] = gsum<G>(tk[c]);
      tv[c] = gsum<G>(tv[c]);
    }
    float z = 0.f, da = 0.f, qk[3] = {0.f, 0.f, 0.f}, dv_[3] = {0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      z = fmaf(wc[c], tk[c], z);
      da = fmaf(wc[c], tv[c], da);
#pragma unroll
      for (int d = 0; d < 3; ++d) {
        qk[d] = fmaf(dwc[c][d], tk[c], qk[d]);
        dv_[d] = fmaf(dwc[c][d], tv[c], dv_[d]);
      }
    }
    const float alpha = exp2f(z * sl2 - l2);
    const float gz = g.scale * alpha * (da - delta);  // scale * dz
    // dQ += scale dz K~, corner by corner
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      unraw(kr[c], x);
      const float sc = gz * wc[c];
#pragma unroll
      for (int e = 0; e < EL; ++e) dqa[e] = fmaf(sc, x[e], dqa[e]);
    }
    float gp[3];
#pragma unroll
    for (int d = 0; d < 3; ++d) gp[d] = gz * qk[d] + alpha * dv_[d];
    if (gl == 0) {
      coef_a[e0 + j] = alpha;
      coef_g[e0 + j] = gz;
      if (g.mode == DSA3D_SAMPLE_FREE) {
        float* gq = gpos + (e0 + j) * 3;
        gq[0] = gp[0]; gq[1] = gp[1]; gq[2] = gp[2];
      }
    }
    gb[0] += gp[0]; gb[1] += gp[1]; gb[2] += gp[2];
  }
#pragma unroll
  for (int mask = G; mask < 64; mask <<= 1) {
#pragma unroll
    for (int e = 0; e < EL; ++e) dqa[e] += __shfl_xor(dqa[e], mask, 64);
#pragma unroll
    for (int d = 0; d < 3; ++d) gb[d] += __shfl_xor(gb[d], mask, 64);
  }
  if (grp == 0) {
    store8(dq + row, dqa);
    if (g.mode == DSA3D_SAMPLE_BOX && gl == 0) {
      float* gq = gpos + ((size_t)h * g.N + n) * 3;
#pragma unroll
      for (int d = 0; d < 3; ++d) gq[d] = qp.act[d] ? gb[d] : 0.f;
    }
  }
}

// ---------------------------------------------------------------------------
// box windows on the start's lattice
// ---------------------------------------------------------------------------
// With one offset per (query, head) every sample shares the fraction f of the start s,
// so sample (u, v, w) blends the rows s_i + (u, v, w) + c, c in {0,1}^3, with the same
// 8 weights: all samples read the (kt+1)(ky+1)(kx+1) rows of the lattice s_i + [0, k]^3.
// Since the blend is linear, q . K~(sample) is the same blend of the lattice dots
// T_l = q . K[l], and sum_j p_j V~(sample j) = sum_l A_l V[l] with A_l the blend's
// transpose applied to p.  A wave per (query, head) reads each lattice row once
// instead of each sample's 8 corners (147 samples: 256 rows against 1176).  The backward
// hands the key side the lattice weights of dO and q per lattice point, so the key side
// too visits L rows per (query, head) rather than 8 K corners.
constexpr int BOX_LDS_BYTES = 65536;  // a block's 4 waves: lattice and sample arrays

struct BoxLat {
  int e1, e2;        // lattice extents: ky + 1, kx + 1 (lattice index (lt e1 + ly) e2 + lx)
  int L;             // (kt + 1) e1 e2
  int coff[8];       // lattice index offset of corner c
  float w[8];        // corner weights
  float dw[8][3];    // their derivatives by f_t, f_y, f_x
};
__device__ __forceinline__ BoxLat box_lattice(const SGeom& g, const QPos& qp) {
  BoxLat b;
  b.e1 = g.ky + 1;
  b.e2 = g.kx + 1;
  b.L = (g.kt + 1) * b.e1 * b.e2;
  const float* f = qp.sf;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int ct = (c >> 2) & 1, cy = (c >> 1) & 1, cx = c & 1;
    b.coff[c] = (ct * b.e1 + cy) * b.e2 + cx;
    const float pt = ct ? f[0] : 1.f - f[0], py = cy ? f[1] : 1.f - f[1], px = cx ? f[2] : 1.f - f[2];
    b.w[c] = pt * py * px;
    b.dw[c][0] = (ct ? 1.f : -1.f) * py * px;
    b.dw[c][1] = (cy ? 1.f : -1.f) * pt * px;
    b.dw[c][2] = (cx ? 1.f : -1.f) * pt * py;
  }
  return b;
}
// grid token of lattice point l, -1 outside the grid
__device__ __forceinline__ int box_tok(const SGeom& g, const QPos& qp, const BoxLat& b, int l) {
  const int lt = l / (b.e1 * b.e2), r = l - lt * b.e1 * b.e2, ly = r / b.e2, lx = r - ly * b.e2;
  const int t = qp.si[0] + lt, y = qp.si[1] + ly, x = qp.si[2] + lx;
  if ((unsigned)t >= (unsigned)g.F || (unsigned)y >= (unsigned)g.Hp || (unsigned)x >= (unsigned)g.Wp) return -1;
  return (t * g.Hp + y) * g.Wp + x;
}
// lattice index of sample j's base corner
__device__ __forceinline__ int box_base(const SGeom& g, const BoxLat& b, int j) {
  const int u = j / (g.ky * g.kx), r = j - u * (g.ky * g.kx), v = r / g.kx, w = r - v * g.kx;
  return (u * b.e1 + v) * b.e2 + w;
}
// sum over the samples j with base corner l - coff[c] of wc[c] x[j] (the blend's transpose)
__device__ __forceinline__ float box_gather(const SGeom& g, const BoxLat& b, const float* wc, const float* x, int l) {
  const int lt = l / (b.e1 * b.e2), r = l - lt * b.e1 * b.e2, ly = r / b.e2, lx = r - ly * b.e2;
  float a = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int u = lt - ((c >> 2) & 1), v = ly - ((c >> 1) & 1), w = lx - (c & 1);
    if ((unsigned)u < (unsigned)g.kt && (unsigned)v < (unsigned)g.ky && (unsigned)w < (unsigned)g.kx)
      a = fmaf(wc[c], x[(u * g.ky + v) * g.kx + w], a);
  }
  return a;
}
// wave-wide sum / max
__device__ __forceinline__ float wsum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}
__device__ __forceinline__ float wmax(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
// LDS written by some lanes of the wave, read by others: order the accesses
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
// The lattice rows of (n, h) for a wave's lane groups, BU rows per group in flight:
// f(l, values of row l for this lane, tok >= 0) is called for every lattice point.
template <int BU, typename T, int D, typename Fn>
__device__ __forceinline__ void box_rows(const SGeom& g, const QPos& qp, const BoxLat& b, const T* __restrict__ src,
                                         int h, int grp, int gl, Fn&& fn) {
  constexpr int G = D / EL, NG = 64 / G;
  for (int l0 = grp; l0 < b.L; l0 += NG * BU) {
    Raw8<T> raw[BU];
    int ok[BU];
#pragma unroll
    for (int u = 0; u < BU; ++u) {
      const int l = l0 + u * NG;
      const int tok = l < b.L ? box_tok(g, qp, b, l) : -1;
      ok[u] = tok >= 0;
      raw[u] = ldraw(src + ((size_t)(ok[u] ? tok : 0) * g.H + h) * D + gl * EL);
    }
#pragma unroll
    for (int u = 0; u < BU; ++u) {
      const int l = l0 + u * NG;
      if (l < b.L) {
        float x[EL];
        unraw(raw[u], x);
        fn(l, x, ok[u] != 0);
      }
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void k_box_fwd(const T* __restrict__ q, const T* __restrict__ k,
                                                 const T* __restrict__ v, const float* __restrict__ off,
                                                 T* __restrict__ out, float* __restrict__ lse, SGeom g) {
  constexpr int G = D / EL;
  extern __shared__ float box_lds[];  // per wave: L lattice values (T_l, then A_l), K samples (scores, then p_j)
  const int wq = threadIdx.x >> 6;
  const long long wv = (long long)blockIdx.x * 4 + wq;
  if (wv >= (long long)g.N * g.H) return;
  const int h = (int)(wv / g.N), n = (int)(wv - (long long)h * g.N);  // head-major: see wave order
  const int lane = threadIdx.x & 63, grp = lane / G, gl = lane % G;
  const QPos qp = query_pos(g, off, n, h);
  const BoxLat b = box_lattice(g, qp);
  float* sl = box_lds + (size_t)wq * (b.L + g.K);
  float* ss = sl + b.L;
  const size_t row = ((size_t)n * g.H + h) * D + gl * EL;
  float qf[EL];
  load8(q + row, qf);
  // lattice dots q . K[l] (0 outside the grid)
  box_rows<4, T, D>(g, qp, b, k, h, grp, gl, [&](int l, const float* x, bool ok) {
    const float t = gsum<G>(dot8(qf, x));
    if (gl == 0) sl[l] = ok ? t : 0.f;
  });
  wave_lds_sync();
  // sample scores (log2 units), their max, p and its sum
  const float sl2 = g.scale * LOG2E;
  float mx = -INFINITY;
  for (int j = lane; j < g.K; j += 64) {
    const int lb = box_base(g, b, j);
    float z = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) z = fmaf(b.w[c], sl[lb + b.coff[c]], z);
    ss[j] = z * sl2;
    mx = fmaxf(mx, z * sl2);
  }
  mx = wmax(mx);
  float sum = 0.f;
  for (int j = lane; j < g.K; j += 64) {
    const float p = exp2f(ss[j] - mx);
    ss[j] = p;
    sum += p;
  }
  sum = wsum(sum);
  wave_lds_sync();
  // A_l, the lattice weights of V
  for (int l = lane; l < b.L; l += 64) sl[l] = box_gather(g, b, b.w, ss, l);
  wave_lds_sync();
  float acc[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) acc[e] = 0.f;
  box_rows<4, T, D>(g, qp, b, v, h, grp, gl, [&](int l, const float* x, bool ok) {
    const float a = ok ? sl[l] : 0.f;
#pragma unroll
    for (int e = 0; e < EL; ++e) acc[e] = fmaf(a, x[e], acc[e]);
  });
#pragma unroll
  for (int mask = G; mask < 64; mask <<= 1)
#pragma unroll
    for (int e = 0; e < EL; ++e) acc[e] += __shfl_xor(acc[e], mask, 64);
  if (grp == 0) {
    const float inv = 1.f / sum;
#pragma unroll
    for (int e = 0; e < EL; ++e) acc[e] *= inv;
    store8(out + row, acc);
    if (gl == 0) lse[(size_t)h * g.N + n] = (mx + log2f(sum)) * LN2;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void k_box_bwd_q(const T* __restrict__ q, const T* __restrict__ k,
                                                   const T* __restrict__ v, const T* __restrict__ o,
                                                   const T* __restrict__ dout, const float* __restrict__ lse,
                                                   const float* __restrict__ off, T* __restrict__ dq,
                                                   float* __restrict__ coef_a, float* __restrict__ coef_g,
                                                   float* __restrict__ gpos, SGeom g) {
  constexpr int G = D / EL;
  // per wave: L values T_l = q . K[l] (then B_l), L values U_l = dO . V[l] (then A_l),
  // K values scale * dS and K values alpha
  extern __shared__ float box_lds[];
  const int wq = threadIdx.x >> 6;
  const long long wv = (long long)blockIdx.x * 4 + wq;
  if (wv >= (long long)g.N * g.H) return;
  const int h = (int)(wv / g.N), n = (int)(wv - (long long)h * g.N);  // head-major: see wave order
  const int lane = threadIdx.x & 63, grp = lane / G, gl = lane % G;
  const QPos qp = query_pos(g, off, n, h);
  const BoxLat b = box_lattice(g, qp);
  float* st = box_lds + (size_t)wq * 2 * (b.L + g.K);
  float* su = st + b.L;
  float* sg = su + b.L;
  float* sa = sg + g.K;
  const size_t row = ((size_t)n * g.H + h) * D + gl * EL;
  float qf[EL], df[EL], x0[EL];
  load8(q + row, qf);
  load8(dout + row, df);
  load8(o + row, x0);
  const float delta = gsum<G>(dot8(df, x0));
  const float sl2 = g.scale * LOG2E;
  const float l2 = lse[(size_t)h * g.N + n] * LOG2E;
  box_rows<4, T, D>(g, qp, b, k, h, grp, gl, [&](int l, const float* x, bool ok) {
    const float t = gsum<G>(dot8(qf, x));
    if (gl == 0) st[l] = ok ? t : 0.f;
  });
  box_rows<4, T, D>(g, qp, b, v, h, grp, gl, [&](int l, const float* x, bool ok) {
    const float u = gsum<G>(dot8(df, x));
    if (gl == 0) su[l] = ok ? u : 0.f;
  });
  wave_lds_sync();
  // per sample: alpha, scale * dS, and the position gradient through the weights
  float gp[3] = {0.f, 0.f, 0.f};
  for (int j = lane; j < g.K; j += 64) {
    const int lb = box_base(g, b, j);
    float z = 0.f, da = 0.f, qk[3] = {0.f, 0.f, 0.f}, dv_[3] = {0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float t = st[lb + b.coff[c]], u = su[lb + b.coff[c]];
      z = fmaf(b.w[c], t, z);
      da = fmaf(b.w[c], u, da);
#pragma unroll
      for (int d = 0; d < 3; ++d) {
        qk[d] = fmaf(b.dw[c][d], t, qk[d]);
        dv_[d] = fmaf(b.dw[c][d], u, dv_[d]);
      }
    }
    const float alpha = exp2f(z * sl2 - l2);
    const float gz = g.scale * alpha * (da - delta);
    sg[j] = gz;
    sa[j] = alpha;
#pragma unroll
    for (int d = 0; d < 3; ++d) gp[d] += gz * qk[d] + alpha * dv_[d];
  }
  wave_lds_sync();
  // B_l, the lattice weights of K for dQ and of q for dK, and A_l, those of dO for dV
  // (into st and su: every T_l and U_l has been read); the key side takes both
  const size_t e0 = ((size_t)h * g.N + n) * b.L;
  for (int l = lane; l < b.L; l += 64) {
    const float bl = box_gather(g, b, b.w, sg, l), al = box_gather(g, b, b.w, sa, l);
    st[l] = bl;
    coef_a[e0 + l] = al;
    coef_g[e0 + l] = bl;
  }
  wave_lds_sync();
  float dqa[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) dqa[e] = 0.f;
  box_rows<4, T, D>(g, qp, b, k, h, grp, gl, [&](int l, const float* x, bool ok) {
    const float bl = ok ? st[l] : 0.f;
#pragma unroll
    for (int e = 0; e < EL; ++e) dqa[e] = fmaf(bl, x[e], dqa[e]);
  });
#pragma unroll
  for (int mask = G; mask < 64; mask <<= 1)
#pragma unroll
    for (int e = 0; e < EL; ++e) dqa[e] += __shfl_xor(dqa[e], mask, 64);
#pragma unroll
  for (int d = 0; d < 3; ++d) gp[d] = wsum(gp[d]);
  if (grp == 0) {
    store8(dq + row, dqa);
    if (gl == 0) {
      float* gq = gpos + ((size_t)h * g.N + n) * 3;
#pragma unroll
      for (int d = 0; d < 3; ++d) gq[d] = qp.act[d] ? gp[d] : 0.f;
    }
  }
}

// ---------------------------------------------------------------------------
// backward, key side
// ---------------------------------------------------------------------------
// Sort key of sample e = (h * N + n) * K + j: (head, base cell floor(P) + 1), base cells
// in [-1, G-1] per axis; samples whose 8 corners all lie outside the grid get the
// sentinel H * ncell and are never visited.
__global__ __launch_bounds__(256) void k_sampled_keys(const float* __restrict__ off, SGeom g,
                                                      uint32_t* __restrict__ keys) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long E = (long long)g.N * g.H * g.K;
  if (e >= E) return;
  const int j = (int)(e % g.K);
  const long long hn = e / g.K;
  const int n = (int)(hn % g.N), h = (int)(hn / g.N);
  const QPos qp = query_pos(g, off, n, h);
  int i[3];
  float f[3];
  sample_pos(g, qp, j, i, f);
  const int ncell = (g.F + 1) * (g.Hp + 1) * (g.Wp + 1);
  uint32_t key = (uint32_t)g.H * ncell;
  if (i[0] >= -1 && i[0] < g.F && i[1] >= -1 && i[1] < g.Hp && i[2] >= -1 && i[2] < g.Wp)
    key = (uint32_t)(h * ncell + ((i[0] + 1) * (g.Hp + 1) + (i[1] + 1)) * (g.Wp + 1) + (i[2] + 1));
  keys[e] = key;
}

// The sorted samples as contiguous records for the key side: sorted position i holds
// (query token, fractions f_t, f_y, f_x of its position) and (alpha, scale * dz), so a
// key's wave reads its samples in order with no index arithmetic.
__global__ __launch_bounds__(256) void k_sampled_pack(const float* __restrict__ off, const int* __restrict__ ids,
                                                      const float* __restrict__ coef_a,
                                                      const float* __restrict__ coef_g, int n_sorted,
                                                      int4* __restrict__ rec, float2* __restrict__ rcoef, SGeom g) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n_sorted) return;
  const int e = ids[i];
  const int j = e % g.K;
  const int hn = e / g.K;
  const int n = hn % g.N, h = hn / g.N;
  const QPos qp = query_pos(g, off, n, h);
  int ip[3];
  float f[3];
  sample_pos(g, qp, j, ip, f);
  rec[i] = make_int4(n, __float_as_int(f[0]), __float_as_int(f[1]), __float_as_int(f[2]));
  rcoef[i] = make_float2(coef_a[e], coef_g[e]);
}

constexpr int DK_B = 4;  // samples per lane group in flight on the key side

template <typename T, int D>
__global__ __launch_bounds__(256) void k_sampled_dkdv(const T* __restrict__ q, const T* __restrict__ dout,
                                                      const int4* __restrict__ rec,
                                                      const float2* __restrict__ rcoef,
                                                      const int* __restrict__ cell_ptr, T* __restrict__ dk,
                                                      T* __restrict__ dv, SGeom g) {
  constexpr int G = D / EL, NG = 64 / G;
  const long long wv = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wv >= (long long)g.N * g.H) return;
  const int m = (int)(wv / g.H), h = (int)(wv - (long long)m * g.H);  // key side: token-major (measured faster)
  const int lane = threadIdx.x & 63, grp = lane / G, gl = lane % G;
  const int plane = g.Hp * g.Wp;
  const int mt = m / plane, my = (m - mt * plane) / g.Wp, mx = m - mt * plane - my * g.Wp;
  const int ncell = (g.F + 1) * (g.Hp + 1) * (g.Wp + 1);

  float dka[EL], dva[EL], x[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) dka[e] = dva[e] = 0.f;
  for (int c = 0; c < 8; ++c) {
    // samples whose corner c is key m have base cell m - bits(c)
    const int bt = (c >> 2) & 1, by = (c >> 1) & 1, bx = c & 1;
    const int cell = h * ncell + ((mt - bt + 1) * (g.Hp + 1) + (my - by + 1)) * (g.Wp + 1) + (mx - bx + 1);
    const int beg = cell_ptr[cell], end = cell_ptr[cell + 1];
    // DK_B samples per lane group at a time: their records, then all their q / dO rows,
    // then the products (samples past the cell add zero)
    for (int base = beg; base < end; base += NG * DK_B) {
      int nn[DK_B];
      float a[DK_B], gz[DK_B];
#pragma unroll
      for (int b = 0; b < DK_B; ++b) {
        const int it = base + grp + b * NG;
        const bool ok = it < end;
        const int4 r = rec[ok ? it : beg];
        const float2 cf = rcoef[ok ? it : beg];
        const float f[3] = {__int_as_float(r.y), __int_as_float(r.z), __int_as_float(r.w)};
        const float w = ok ? corner_w(f, c) : 0.f;
        nn[b] = r.x;
        a[b] = w * cf.x;
        gz[b] = w * cf.y;
      }
      Raw8<T> dr[DK_B], qr[DK_B];
#pragma unroll
      for (int b = 0; b < DK_B; ++b) {
        const size_t r = ((size_t)nn[b] * g.H + h) * D + gl * EL;
        dr[b] = ldraw(dout + r);
        qr[b] = ldraw(q + r);
      }
#pragma unroll
      for (int b = 0; b < DK_B; ++b) {
        unraw(dr[b], x);
#pragma unroll
        for (int t = 0; t < EL; ++t) dva[t] = fmaf(a[b], x[t], dva[t]);
        unraw(qr[b], x);
#pragma unroll
        for (int t = 0; t < EL; ++t) dka[t] = fmaf(gz[b], x[t], dka[t]);
      }
    }
  }
#pragma unroll
  for (int mask = G; mask < 64; mask <<= 1) {
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      dka[e] += __shfl_xor(dka[e], mask, 64);
      dva[e] += __shfl_xor(dva[e], mask, 64);
    }
  }
  if (grp == 0) {
    const size_t r = ((size_t)m * g.H + h) * D + gl * EL;
    store8(dk + r, dka);
    store8(dv + r, dva);
  }
}

// Box windows on the lattice: entry e = (h * N + n) * L + l is lattice point l of
// (query n, head h), keyed by its grid token inside head h's segment; points outside the
// grid, and those of zero weight (the far slice of an axis whose fraction is 0), get the
// sentinel N and are never visited.
__global__ __launch_bounds__(256) void k_box_keys(const float* __restrict__ off, SGeom g,
                                                  uint32_t* __restrict__ keys) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  const int L = (g.kt + 1) * (g.ky + 1) * (g.kx + 1);
  if (e >= (long long)g.N * g.H * L) return;
  const int l = (int)(e % L);
  const long long hn = e / L;
  const int n = (int)(hn % g.N), h = (int)(hn / g.N);
  const QPos qp = query_pos(g, off, n, h);
  const int e1 = g.ky + 1, e2 = g.kx + 1;
  const int lt = l / (e1 * e2), r = l - lt * e1 * e2, ly = r / e2, lx = r - ly * e2;
  const bool dead = (lt == g.kt && qp.sf[0] == 0.f) || (ly == g.ky && qp.sf[1] == 0.f) || (lx == g.kx && qp.sf[2] == 0.f);
  const int t = qp.si[0] + lt, y = qp.si[1] + ly, x = qp.si[2] + lx;
  const bool in = (unsigned)t < (unsigned)g.F && (unsigned)y < (unsigned)g.Hp && (unsigned)x < (unsigned)g.Wp;
  keys[e] = (in && !dead) ? (uint32_t)((t * g.Hp + y) * g.Wp + x) : (uint32_t)g.N;
}

// sorted lattice entries as records (query token, A_l, B_l)
__global__ __launch_bounds__(256) void k_box_pack(const int* __restrict__ ids, const float* __restrict__ coef_a,
                                                  const float* __restrict__ coef_g, int n_sorted,
                                                  int4* __restrict__ rec, SGeom g) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n_sorted) return;
  const int e = ids[i];
  const int L = (g.kt + 1) * (g.ky + 1) * (g.kx + 1);
  const int n = (e / L) % g.N;
  rec[i] = make_int4(n, __float_as_int(coef_a[e]), __float_as_int(coef_g[e]), 0);
}

// dK[m] = sum B_l q_n, dV[m] = sum A_l dO_n over the lattice entries on key m, in sorted
// (query, lattice point) order; a wave per (key, head)
template <typename T, int D>
__global__ __launch_bounds__(256) void k_box_dkdv(const T* __restrict__ q, const T* __restrict__ dout,
                                                  const int4* __restrict__ rec, const int* __restrict__ cell_ptr,
                                                  T* __restrict__ dk, T* __restrict__ dv, SGeom g) {
  constexpr int G = D / EL, NG = 64 / G;
  const long long wv = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wv >= (long long)g.N * g.H) return;
  const int m = (int)(wv / g.H), h = (int)(wv - (long long)m * g.H);  // key side: token-major (measured faster)
  const int lane = threadIdx.x & 63, grp = lane / G, gl = lane % G;
  const int cell = h * (g.N + 1) + m;
  const int beg = cell_ptr[cell], end = cell_ptr[cell + 1];
  float dka[EL], dva[EL], x[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) dka[e] = dva[e] = 0.f;
  for (int base = beg; base < end; base += NG * DK_B) {
    int nn[DK_B];
    float a[DK_B], bq[DK_B];
#pragma unroll
    for (int u = 0; u < DK_B; ++u) {
      const int it = base + grp + u * NG;
      const bool ok = it < end;
      const int4 r = rec[ok ? it : beg];
      nn[u] = r.x;
      a[u] = ok ? __int_as_float(r.y) : 0.f;
      bq[u] = ok ? __int_as_float(r.z) : 0.f;
    }
    Raw8<T> dr[DK_B], qr[DK_B];
#pragma unroll
    for (int u = 0; u < DK_B; ++u) {
      const size_t r = ((size_t)nn[u] * g.H + h) * D + gl * EL;
      dr[u] = ldraw(dout + r);
      qr[u] = ldraw(q + r);
    }
#pragma unroll
    for (int u = 0; u < DK_B; ++u) {
      unraw(dr[u], x);
#pragma unroll
      for (int t = 0; t < EL; ++t) dva[t] = fmaf(a[u], x[t], dva[t]);
      unraw(qr[u], x);
#pragma unroll
      for (int t = 0; t < EL; ++t) dka[t] = fmaf(bq[u], x[t], dka[t]);
    }
  }
#pragma unroll
  for (int mask = G; mask < 64; mask <<= 1) {
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      dka[e] += __shfl_xor(dka[e], mask, 64);
      dva[e] += __shfl_xor(dva[e], mask, 64);
    }
  }
  if (grp == 0) {
    const size_t r = ((size_t)m * g.H + h) * D + gl * EL;
    store8(dk + r, dka);
    store8(dv + r, dva);
  }
}

// Offset gradients in the caller's layout: entry (n, ho, jo) sums the per-sample (free)
// or per-(query, head) (box) gradients over the heads (sh == 0) and samples (ss == 0)
// that share it, heads then samples in ascending order.
__global__ __launch_bounds__(256) void k_sampled_doff(const float* __restrict__ gpos, float* __restrict__ doff,
                                                      SGeom g) {
  const int hb = g.sh == 0 ? 1 : g.H;
  const int kb = (g.mode == DSA3D_SAMPLE_BOX || g.ss == 0) ? 1 : g.K;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long long)g.N * hb * kb) return;
  const int jo = (int)(t % kb);
  const long long r = t / kb;
  const int ho = (int)(r % hb), n = (int)(r / hb);
  float s[3] = {0.f, 0.f, 0.f};
  for (int h = (hb == 1 ? 0 : ho); h < (hb == 1 ? g.H : ho + 1); ++h) {
    if (g.mode == DSA3D_SAMPLE_BOX) {
      const float* p = gpos + ((size_t)h * g.N + n) * 3;
      s[0] += p[0]; s[1] += p[1]; s[2] += p[2];
    } else {
      for (int j = (kb == 1 ? 0 : jo); j < (kb == 1 ? g.K : jo + 1); ++j) {
        const float* p = gpos + (((size_t)h * g.N + n) * g.K + j) * 3;
        s[0] += p[0]; s[1] += p[1]; s[2] += p[2];
      }
    }
  }
  float* d = doff + (long long)n * g.sn + (long long)ho * g.sh + (long long)jo * g.ss;
  d[0] = s[0]; d[1] = s[1]; d[2] = s[2];
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// Box windows whose lattice arrays fit a block's LDS run on the lattice kernels: a block
// of 4 waves holds nl lattice arrays and ns sample arrays per wave (the backward 2 and 2).
static long long box_lattice_points(const SGeom& g) { return (long long)(g.kt + 1) * (g.ky + 1) * (g.kx + 1); }
static size_t box_lds_bytes(const SGeom& g, int nl, int ns) {
  return (size_t)4 * (nl * box_lattice_points(g) + ns * g.K) * sizeof(float);
}
static bool box_on_lattice(const SGeom& g) {
  return g.mode == DSA3D_SAMPLE_BOX && box_lds_bytes(g, 2, 2) <= (size_t)BOX_LDS_BYTES;
}
// ... and their backward on the lattice when the N H L lattice entries fit 32-bit indices
static bool box_lattice_bwd(const SGeom& g) {
  return box_on_lattice(g) && (long long)g.N * g.H * box_lattice_points(g) < (1LL << 31);
}

struct SampledWs {
  uint32_t* keys[2];
  int* vals[2];
  uint32_t* ghist;
  uint32_t* scan_part;  // chunk totals of the histogram scans
  int* cell_ptr;
  float* coef_a;  // per sample alpha, or per lattice point A_l (box windows on the lattice)
  float* coef_g;  // per sample scale * dz, or per lattice point B_l
  float* gpos;
  int4* rec;      // sorted samples: (token, fractions), or lattice points: (token, A_l, B_l)
  float2* rcoef;  // sorted samples: (alpha, scale * dz)
  int passes;
  int nseg;       // sort segments: 1, or one per head (lattice points)
  int keyspace;   // keys per segment, the sentinel included
};

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t sampled_layout(const SGeom& g, char* base, SampledWs* w) {
  // sorted entries: samples keyed by (head, base cell) in one segment with the sentinel
  // H * ncell, or lattice points keyed by token in one segment per head, sentinel N
  const bool lat = box_lattice_bwd(g);
  const size_t E = (size_t)g.N * g.H * (lat ? box_lattice_points(g) : g.K);
  const int nseg = lat ? g.H : 1;
  const size_t seglen = E / nseg;
  const size_t nb = (seglen + RADIX_TILE - 1) / RADIX_TILE * nseg;
  const size_t ncell = (size_t)(g.F + 1) * (g.Hp + 1) * (g.Wp + 1);
  const size_t sentinel = lat ? (size_t)g.N : ncell * g.H;
  int bits = 1;
  while (((size_t)1 << bits) <= sentinel) ++bits;  // the sentinel sorts last
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  SampledWs s;
  s.keys[0] = (uint32_t*)take(E * 4);
  s.keys[1] = (uint32_t*)take(E * 4);
  s.vals[0] = (int*)take(E * 4);
  s.vals[1] = (int*)take(E * 4);
  s.ghist = (uint32_t*)take(256 * nb * 4);
  s.scan_part = (uint32_t*)take(scan_part_words(256 * nb) * 4);
  s.cell_ptr = (int*)take(((sentinel + 1) * nseg + 1) * 4);
  s.coef_a = (float*)take(E * 4);
  s.coef_g = (float*)take(E * 4);
  s.gpos = (float*)take((g.mode == DSA3D_SAMPLE_BOX ? (size_t)g.N * g.H : (size_t)g.N * g.H * g.K) * 3 * 4);
  s.rec = (int4*)take(E * sizeof(int4));
  s.rcoef = lat ? nullptr : (float2*)take(E * sizeof(float2));
  s.passes = (bits + 7) / 8;
  s.nseg = nseg;
  s.keyspace = lat ? (int)sentinel + 1 : (int)sentinel;
  if (w) *w = s;
  return off;
}

static unsigned nblocks(long long n, int per) { return (unsigned)((n + per - 1) / per); }


template <typename T, int D>
static hipError_t sampled_fwd_impl(const void* q, const void* k, const void* v, const float* off, void* out,
                                   float* lse, const SGeom& g, hipStream_t s) {
  if (box_on_lattice(g))
    k_box_fwd<T, D><<<nblocks((long long)g.N * g.H, 4), 256, box_lds_bytes(g, 1, 1), s>>>(
        (const T*)q, (const T*)k, (const T*)v, off, (T*)out, lse, g);
  else
    k_sampled_fwd<T, D><<<nblocks((long long)g.N * g.H, 4), 256, 0, s>>>(
        (const T*)q, (const T*)k, (const T*)v, off, (T*)out, lse, g);
  return hipGetLastError();
}

hipError_t launch_sampled_forward(int dtype, int D, const void* q, const void* k, const void* v, const float* off,
                                  void* out, float* lse, const SGeom& g, hipStream_t s) {
  if (dtype == DSA3D_BF16)
    return D == 64 ? sampled_fwd_impl<u16, 64>(q, k, v, off, out, lse, g, s)
                   : sampled_fwd_impl<u16, 128>(q, k, v, off, out, lse, g, s);
  return D == 64 ? sampled_fwd_impl<float, 64>(q, k, v, off, out, lse, g, s)
                 : sampled_fwd_impl<float, 128>(q, k, v, off, out, lse, g, s);
}

template <typename T, int D>
static hipError_t sampled_bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                   const float* lse, const float* off, void* dq, void* dk, void* dv, float* doff,
                                   const SGeom& g, const SampledWs& w, hipStream_t s) {
  const long long waves = (long long)g.N * g.H;
  const bool lat = box_lattice_bwd(g);
  const long long E = waves * (lat ? box_lattice_points(g) : g.K);
  if (lat)
    k_box_keys<<<nblocks(E, 256), 256, 0, s>>>(off, g, w.keys[0]);
  else
    k_sampled_keys<<<nblocks(E, 256), 256, 0, s>>>(off, g, w.keys[0]);
  uint32_t* keys[2] = {w.keys[0], w.keys[1]};
  int* vals[2] = {w.vals[0], w.vals[1]};
  const int seglen = (int)(E / w.nseg);
  const int cur = radix_sort(keys, vals, w.ghist, seglen, w.nseg, w.passes, s, w.scan_part);
  if (cur < 0) return hipErrorLaunchFailure;
  hipError_t e = launch_cell_ptr(keys[cur], seglen, w.nseg, w.keyspace, w.cell_ptr, s);
  if (e != hipSuccess) return e;
  // every entry is packed; those keyed by the sentinel sort after every key (of their
  // segment) and are never visited
  const int n_sorted = (int)E;
  if (lat) {
    k_box_bwd_q<T, D><<<nblocks(waves, 4), 256, box_lds_bytes(g, 2, 2), s>>>(
        (const T*)q, (const T*)k, (const T*)v, (const T*)o, (const T*)dout, lse, off, (T*)dq, w.coef_a, w.coef_g,
        w.gpos, g);
    k_box_pack<<<nblocks(n_sorted, 256), 256, 0, s>>>(vals[cur], w.coef_a, w.coef_g, n_sorted, w.rec, g);
    k_box_dkdv<T, D><<<nblocks(waves, 4), 256, 0, s>>>((const T*)q, (const T*)dout, w.rec, w.cell_ptr, (T*)dk,
                                                       (T*)dv, g);
  } else {
    k_sampled_bwd_q<T, D><<<nblocks(waves, 4), 256, 0, s>>>((const T*)q, (const T*)k, (const T*)v, (const T*)o,
                                                            (const T*)dout, lse, off, (T*)dq, w.coef_a, w.coef_g,
                                                            w.gpos, g);
    k_sampled_pack<<<nblocks(n_sorted, 256), 256, 0, s>>>(off, vals[cur], w.coef_a, w.coef_g, n_sorted, w.rec,
                                                          w.rcoef, g);
    k_sampled_dkdv<T, D><<<nblocks(waves, 4), 256, 0, s>>>((const T*)q, (const T*)dout, w.rec, w.rcoef,
                                                           w.cell_ptr, (T*)dk, (T*)dv, g);
  }
  const long long nout = (long long)g.N * (g.sh == 0 ? 1 : g.H) *
                         ((g.mode == DSA3D_SAMPLE_BOX || g.ss == 0) ? 1 : g.K);
  k_sampled_doff<<<nblocks(nout, 256), 256, 0, s>>>(w.gpos, doff, g);
  return hipGetLastError();
}

hipError_t launch_sampled_backward(int dtype, int D, const void* q, const void* k, const void* v, const void* o,
                                   const void* dout, const float* lse, const float* off, void* dq, void* dk,
                                   void* dv, float* doff, const SGeom& g, char* workspace, hipStream_t s) {
  SampledWs w;
  sampled_layout(g, workspace, &w);
  if (dtype == DSA3D_BF16)
    return D == 64 ? sampled_bwd_impl<u16, 64>(q, k, v, o, dout, lse, off, dq, dk, dv, doff, g, w, s)
                   : sampled_bwd_impl<u16, 128>(q, k, v, o, dout, lse, off, dq, dk, dv, doff, g, w, s);
  return D == 64 ? sampled_bwd_impl<float, 64>(q, k, v, o, dout, lse, off, dq, dk, dv, doff, g, w, s)
                 : sampled_bwd_impl<float, 128>(q, k, v, o, dout, lse, off, dq, dk, dv, doff, g, w, s);
}

}  // namespace dsa3d

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
using namespace dsa3d;

namespace {

bool odd_pos(int k) { return k >= 1 && (k & 1); }

// Offsets layout: three consecutive floats per entry at element strides (sn, sh, ss)
// >= 0, 0 meaning shared; the entries that are not shared must not overlap (checked as
// a strided array: sorted by stride, each level starts past the extent of the one
// inside it).  Box windows take one offset per (query, head): ss must be 0.
bool layout_ok(long long sn, long long sh, long long ss, int N, int H, int K, int mode) {
  if (sn < 3 || sh < 0 || ss < 0) return false;
  if (mode == DSA3D_SAMPLE_BOX && ss != 0) return false;
  struct Dim { long long stride, size; } d[3] = {{sn, N}, {sh, sh ? H : 1}, {ss, ss ? K : 1}};
  for (int a = 0; a < 3; ++a)
    for (int b = a + 1; b < 3; ++b)
      if (d[b].stride < d[a].stride) { const Dim t = d[a]; d[a] = d[b]; d[b] = t; }
  long long extent = 3;  // floats covered by one entry
  for (int a = 0; a < 3; ++a) {
    if (d[a].size == 1) continue;
    if (d[a].stride < extent) return false;
    extent = d[a].stride * (d[a].size - 1) + extent;
  }
  return true;
}

int check_sampled_geom(int mode, int F, int Hp, int Wp, int heads, int kt, int ky, int kx) {
  if (mode != DSA3D_SAMPLE_BOX && mode != DSA3D_SAMPLE_FREE) return DSA3D_ERR_MODE;
  if (F < 1 || Hp < 1 || Wp < 1 || heads < 1 || heads > 65535) return DSA3D_ERR_GRID;
  if ((long long)F * Hp * Wp >= (1LL << 30)) return DSA3D_ERR_GRID;
  if (!odd_pos(kt) || !odd_pos(ky) || !odd_pos(kx)) return DSA3D_ERR_WINDOW;
  if (mode == DSA3D_SAMPLE_BOX && (kt > F || ky > Hp || kx > Wp)) return DSA3D_ERR_WINDOW;
  if ((long long)kt * ky * kx > 4096) return DSA3D_ERR_WINDOW;
  return DSA3D_OK;
}

SGeom make_sgeom(int mode, int F, int Hp, int Wp, int heads, int kt, int ky, int kx, long long sn, long long sh,
                 long long ss, float scale) {
  SGeom g;
  g.F = F; g.Hp = Hp; g.Wp = Wp;
  g.kt = kt; g.ky = ky; g.kx = kx; g.K = kt * ky * kx;
  g.H = heads; g.N = F * Hp * Wp;
  g.mode = mode;
  g.sn = sn; g.sh = sh; g.ss = ss;
  g.scale = scale;
  return g;
}

int check_sampled(const void* q, const void* k, const void* v, const float* off, long long sn, long long sh,
                  long long ss, int mode, int F, int Hp, int Wp, int heads, int head_dim, int kt, int ky, int kx,
                  float scale, int dtype, SGeom* g) {
  if (!q || !k || !v || !off) return DSA3D_ERR_NULL;
  if (dtype != DSA3D_F32 && dtype != DSA3D_BF16) return DSA3D_ERR_DTYPE;
  if (head_dim != 64 && head_dim != 128) return DSA3D_ERR_HEAD_DIM;
  const int st = check_sampled_geom(mode, F, Hp, Wp, heads, kt, ky, kx);
  if (st != DSA3D_OK) return st;
  if (!isfinite(scale)) return DSA3D_ERR_SCALE;
  if (!layout_ok(sn, sh, ss, F * Hp * Wp, heads, kt * ky * kx, mode)) return DSA3D_ERR_LAYOUT;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v) & 15u) return DSA3D_ERR_ALIGN;
  if ((uintptr_t)off & 3u) return DSA3D_ERR_ALIGN;
  *g = make_sgeom(mode, F, Hp, Wp, heads, kt, ky, kx, sn, sh, ss, scale);
  return DSA3D_OK;
}

// the backward sorts N * H * L lattice points (box windows on the lattice) or N * H * K
// samples with 32-bit indices and (H * cells) 32-bit keys
bool backward_fits(const SGeom& g) {
  if (box_lattice_bwd(g)) return true;
  const long long E = (long long)g.N * g.H * g.K;
  const long long cells = (long long)(g.F + 1) * (g.Hp + 1) * (g.Wp + 1) * g.H;
  return E < (1LL << 31) && cells < (1LL << 31) - 1;
}

}  // namespace

extern "C" {

size_t dsa3d_sampled_workspace_bytes(int F, int Hp, int Wp, int heads, int kt, int ky, int kx, int mode,
                                     int backward) {
  if (check_sampled_geom(mode, F, Hp, Wp, heads, kt, ky, kx) != DSA3D_OK) return 0;
  if (!backward) return 256;  // the forward needs no scratch
  // the layout depends on the geometry and the mode only
  const SGeom g = make_sgeom(mode, F, Hp, Wp, heads, kt, ky, kx, 3, 0, 0, 1.f);
  if (!backward_fits(g)) return 0;
  return sampled_layout(g, nullptr, nullptr);
}

int dsa3d_sampled_forward(const void* q, const void* k, const void* v, const float* offsets, long long stride_token,
                          long long stride_head, long long stride_sample, int mode, int F, int Hp, int Wp, int heads,
                          int head_dim, int kt, int ky, int kx, float scale, int dtype, void* out, float* lse,
                          hipStream_t stream) {
  SGeom g;
  const int st = check_sampled(q, k, v, offsets, stride_token, stride_head, stride_sample, mode, F, Hp, Wp, heads,
                               head_dim, kt, ky, kx, scale, dtype, &g);
  if (st != DSA3D_OK) return st;
  if (!out || !lse) return DSA3D_ERR_NULL;
  if (((uintptr_t)out & 15u) || ((uintptr_t)lse & 3u)) return DSA3D_ERR_ALIGN;
  return launch_sampled_forward(dtype, head_dim, q, k, v, offsets, out, lse, g, stream) == hipSuccess
             ? DSA3D_OK
             : DSA3D_ERR_LAUNCH;
}

int dsa3d_sampled_backward(const void* q, const void* k, const void* v, const float* offsets, long long stride_token,
                           long long stride_head, long long stride_sample, int mode, const void* out,
                           const float* lse, const void* dout, int F, int Hp, int Wp, int heads, int head_dim, int kt,
                           int ky, int kx, float scale, int dtype, void* dq, void* dk, void* dv, float* doffsets,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  SGeom g;
  const int st = check_sampled(q, k, v, offsets, stride_token, stride_head, stride_sample, mode, F, Hp, Wp, heads,
                               head_dim, kt, ky, kx, scale, dtype, &g);
  if (st != DSA3D_OK) return st;
  if (!out || !lse || !dout || !dq || !dk || !dv || !doffsets || !workspace) return DSA3D_ERR_NULL;
  if (((uintptr_t)out | (uintptr_t)dout | (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv | (uintptr_t)workspace) &
      15u)
    return DSA3D_ERR_ALIGN;
  if (((uintptr_t)lse | (uintptr_t)doffsets) & 3u) return DSA3D_ERR_ALIGN;
  if (!backward_fits(g)) return DSA3D_ERR_GRID;
  if (workspace_bytes < sampled_layout(g, nullptr, nullptr)) return DSA3D_ERR_WORKSPACE;
  return launch_sampled_backward(dtype, head_dim, q, k, v, out, dout, lse, offsets, dq, dk, dv, doffsets, g,
                                 static_cast<char*>(workspace), stream) == hipSuccess
             ? DSA3D_OK
             : DSA3D_ERR_LAUNCH;
}

}  // extern "C"
