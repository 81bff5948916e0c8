// 3D Deformable Slide Attention kernels for gfx950 (MegaSlide-DiT, section "3D
// Deformable Slide Attention", Eq. (1) attention term and its softmax weights).
//
// Query-centric passes (forward, dQ): one wave per (query group, head).  A group
// holds up to 16 queries whose windows start in one 1 x 4 x 4 start blob; the
// union of their windows lies in the box [min start, max start + k) per axis (the
// "halo").  The halo is streamed 32 keys at a time: K and V rows are gathered into
// LDS (16-byte loads, one row of a head is contiguous), S^T = K Q^T and the value
// products run on 16x16x32 bf16 MFMA (16x16x4 fp32 MFMA on the fp32 path), keys
// outside a query's own window are masked, and the softmax is kept online.
//
// Key-centric pass (dK, dV): one wave per (1 x 4 x 4 key blob, head).  The queries
// that can see a key of the blob have window starts in a box of start cells; the
// start-cell CSR is walked cell by cell in a fixed order, ascending query id inside
// a cell, 32 queries at a time.  dK and dV accumulate in registers: no atomics, so
// the result is bitwise reproducible.
#include "internal.hpp"

namespace dsa3d {

template <typename T, int D>
struct Tile {
  static constexpr int EV = 16 / (int)sizeof(T);  // elements per 16-byte vector
  static constexpr int RV = D / EV;                // 16-byte vectors per row
  static constexpr int RS = D + EV;                // LDS row stride (one vector of padding)
  static constexpr int NC = D / 32;                // 32-deep contraction steps over d
  static constexpr int NT = D / 16;                // 16-wide output tiles over d
};

// Slot j of a lane in quad `quad` <-> row of a 32-row chunk.  Matches the result
// layout of two stacked 16x16 tiles (lane holds rows 4*quad + i of each).
__device__ __forceinline__ void chunk_rows(int quad, int* rows) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    rows[j] = quad * 4 + j;
    rows[j + 4] = 16 + quad * 4 + j;
  }
}

__device__ __forceinline__ bool in_window(const int4& kp, const int4& s, const Geom& g) {
  return (unsigned)(kp.x - s.x) < (unsigned)g.kt && (unsigned)(kp.y - s.y) < (unsigned)g.ky &&
         (unsigned)(kp.z - s.z) < (unsigned)g.kx;
}

// Copies CHUNK rows (token ltok[r], or zeros when < 0) of head h into LDS.
template <typename T, int D>
__device__ __forceinline__ void stage_rows(T* __restrict__ lds, const T* __restrict__ src, const int* ltok, int H,
                                           int h, int lane) {
  using TL = Tile<T, D>;
#pragma unroll
  for (int it = 0; it < CHUNK * TL::RV / 64; ++it) {
    const int vi = it * 64 + lane;
    const int r = vi / TL::RV, cv = vi % TL::RV;
    const int tok = ltok[r];
    uint4 val = {0u, 0u, 0u, 0u};
    if (tok >= 0) val = *reinterpret_cast<const uint4*>(src + ((size_t)tok * H + h) * D + cv * TL::EV);
    *reinterpret_cast<uint4*>(lds + r * TL::RS + cv * TL::EV) = val;
  }
}

struct GroupInfo {
  int n;       // this lane's query token
  bool qv;     // lane holds a real query
  int4 s;      // its window start
  int4 h0;     // halo origin (t, y, x)
  int ny, nx;  // halo extent along y, x
  int nh;      // halo size in keys
};

__device__ __forceinline__ GroupInfo group_info(const Geom& g, const Prep& p, int grp_idx, int lane) {
  GroupInfo gi;
  const int2 grp = p.groups[grp_idx];
  const int qi = lane & 15;
  gi.qv = qi < grp.y;
  gi.n = p.perm[grp.x + (gi.qv ? qi : 0)];
  gi.s = p.starts[gi.n];
  const int t0 = row16_min(gi.s.x), t1 = row16_max(gi.s.x);
  const int y0 = row16_min(gi.s.y), y1 = row16_max(gi.s.y);
  const int x0 = row16_min(gi.s.z), x1 = row16_max(gi.s.z);
  gi.h0 = make_int4(t0, y0, x0, 0);
  const int nt = t1 - t0 + g.kt;
  gi.ny = y1 - y0 + g.ky;
  gi.nx = x1 - x0 + g.kx;
  gi.nh = nt * gi.ny * gi.nx;
  return gi;
}

// Lanes 0..CHUNK-1 decode halo keys base + lane into token ids and positions.
// Keys past the halo get token -1 and a position outside every window.
__device__ __forceinline__ void halo_chunk(const Geom& g, const GroupInfo& gi, int base, int lane, int* ltok,
                                           int4* lpos) {
  if (lane < CHUNK) {
    const int hi = base + lane;
    int tok = -1;
    int4 pos = make_int4(-(1 << 29), -(1 << 29), -(1 << 29), 0);
    if (hi < gi.nh) {
      const int nyx = gi.ny * gi.nx;
      const int dt = hi / nyx, rem = hi - dt * nyx, dy = rem / gi.nx, dx = rem - dy * gi.nx;
      pos = make_int4(gi.h0.x + dt, gi.h0.y + dy, gi.h0.z + dx, 0);
      tok = (pos.x * g.Hp + pos.y) * g.Wp + pos.z;
    }
    ltok[lane] = tok;
    lpos[lane] = pos;
  }
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void k_forward(const T* __restrict__ q, const T* __restrict__ k,
                                                const T* __restrict__ v, T* __restrict__ out,
                                                float* __restrict__ lse, Geom g, Prep p, float sl2) {
  using TL = Tile<T, D>;
  __shared__ __attribute__((aligned(16))) T lk[CHUNK * TL::RS];
  __shared__ __attribute__((aligned(16))) T lv[CHUNK * TL::RS];
  __shared__ int ltok[CHUNK];
  __shared__ int4 lpos[CHUNK];

  if ((int)blockIdx.x >= *p.ngroups) return;
  const int h = g.h0 + (int)blockIdx.y, lane = threadIdx.x, r16 = lane & 15, quad = lane >> 4;
  const GroupInfo gi = group_info(g, p, blockIdx.x, lane);

  Frag<T> qf[TL::NC];
  const T* qrow = q + ((size_t)gi.n * g.H + h) * D;
#pragma unroll
  for (int c = 0; c < TL::NC; ++c) load_frag(qf[c], qrow + c * 32 + quad * 8);

  f32x4_t oacc[TL::NT];
#pragma unroll
  for (int t = 0; t < TL::NT; ++t) oacc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  int rows[8];
  chunk_rows(quad, rows);

  for (int base = 0; base < gi.nh; base += CHUNK) {
    halo_chunk(g, gi, base, lane, ltok, lpos);
    wave_lds_fence();
    stage_rows<T, D>(lk, k, ltok, g.H, h, lane);
    stage_rows<T, D>(lv, v, ltok, g.H, h, lane);
    wave_lds_fence();

    float sv[8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < TL::NC; ++c) {
        Frag<T> a;
        load_frag(a, lk + (u * 16 + r16) * TL::RS + c * 32 + quad * 8);
        acc = mma(a, qf[c], acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = gi.qv && in_window(lpos[u * 16 + quad * 4 + i], gi.s, g);
        sv[u * 4 + i] = ok ? acc[i] * sl2 : -INFINITY;
      }
    }
    float cm = sv[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) cm = fmaxf(cm, sv[j]);
    cm = quad_max(cm);
    const float mn = fmaxf(m_run, cm);
    const float mref = (mn == -INFINITY) ? 0.f : mn;
    const float alpha = __builtin_amdgcn_exp2f(m_run - mref);
    float pr[8], ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pr[j] = __builtin_amdgcn_exp2f(sv[j] - mref);
      ps += pr[j];
    }
    ps = quad_sum(ps);
    l_run = l_run * alpha + ps;
    m_run = mn;
    Frag<T> pf;
    set_frag(pf, pr);
#pragma unroll
    for (int t = 0; t < TL::NT; ++t) {
      oacc[t] *= alpha;
      Frag<T> a;
      gather_frag<T>(a, lv, TL::RS, rows, t * 16 + r16);
      oacc[t] = mma(a, pf, oacc[t]);
    }
    wave_lds_fence();
  }

  if (gi.qv) {
    const float inv = 1.f / l_run;
    T* orow = out + ((size_t)gi.n * g.H + h) * D;
#pragma unroll
    for (int t = 0; t < TL::NT; ++t)
      store4(orow + t * 16 + quad * 4, oacc[t][0] * inv, oacc[t][1] * inv, oacc[t][2] * inv, oacc[t][3] * inv);
    if (quad == 0) lse[(size_t)h * g.N + gi.n] = (m_run + log2f(l_run)) * LN2;
  }
}

// ---------------------------------------------------------------------------
// Backward, query side: Delta and dQ
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void k_backward_dq(const T* __restrict__ q, const T* __restrict__ k,
                                                    const T* __restrict__ v, const T* __restrict__ o,
                                                    const T* __restrict__ dout, const float* __restrict__ lse,
                                                    T* __restrict__ dq, float* __restrict__ delta, Geom g, Prep p,
                                                    float sl2, float scale) {
  using TL = Tile<T, D>;
  __shared__ __attribute__((aligned(16))) T lk[CHUNK * TL::RS];
  __shared__ __attribute__((aligned(16))) T lv[CHUNK * TL::RS];
  __shared__ int ltok[CHUNK];
  __shared__ int4 lpos[CHUNK];

  if ((int)blockIdx.x >= *p.ngroups) return;
  const int h = g.h0 + (int)blockIdx.y, lane = threadIdx.x, r16 = lane & 15, quad = lane >> 4;
  const GroupInfo gi = group_info(g, p, blockIdx.x, lane);

  Frag<T> qf[TL::NC], dof[TL::NC];
  const size_t rbase = ((size_t)gi.n * g.H + h) * D;
  float dsum = 0.f;
#pragma unroll
  for (int c = 0; c < TL::NC; ++c) {
    load_frag(qf[c], q + rbase + c * 32 + quad * 8);
    load_frag(dof[c], dout + rbase + c * 32 + quad * 8);
    Frag<T> of;
    load_frag(of, o + rbase + c * 32 + quad * 8);
#pragma unroll
    for (int j = 0; j < 8; ++j) dsum += frag_elem(dof[c], j) * frag_elem(of, j);
  }
  dsum = quad_sum(dsum);  // Delta = <dO, O> of this lane's query
  if (gi.qv && quad == 0) delta[(size_t)h * g.N + gi.n] = dsum;
  const float lse2 = gi.qv ? lse[(size_t)h * g.N + gi.n] * LOG2E : 0.f;

  f32x4_t acc_dq[TL::NT];
#pragma unroll
  for (int t = 0; t < TL::NT; ++t) acc_dq[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  int rows[8];
  chunk_rows(quad, rows);

  for (int base = 0; base < gi.nh; base += CHUNK) {
    halo_chunk(g, gi, base, lane, ltok, lpos);
    wave_lds_fence();
    stage_rows<T, D>(lk, k, ltok, g.H, h, lane);
    stage_rows<T, D>(lv, v, ltok, g.H, h, lane);
    wave_lds_fence();

    float ds[8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4_t s_acc = {0.f, 0.f, 0.f, 0.f}, dp_acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < TL::NC; ++c) {
        Frag<T> a;
        load_frag(a, lk + (u * 16 + r16) * TL::RS + c * 32 + quad * 8);
        s_acc = mma(a, qf[c], s_acc);
        load_frag(a, lv + (u * 16 + r16) * TL::RS + c * 32 + quad * 8);
        dp_acc = mma(a, dof[c], dp_acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = gi.qv && in_window(lpos[u * 16 + quad * 4 + i], gi.s, g);
        const float pij = ok ? __builtin_amdgcn_exp2f(s_acc[i] * sl2 - lse2) : 0.f;
        ds[u * 4 + i] = pij * (dp_acc[i] - dsum);
      }
    }
    Frag<T> dsf;
    set_frag(dsf, ds);
#pragma unroll
    for (int t = 0; t < TL::NT; ++t) {
      Frag<T> a;
      gather_frag<T>(a, lk, TL::RS, rows, t * 16 + r16);
      acc_dq[t] = mma(a, dsf, acc_dq[t]);
    }
    wave_lds_fence();
  }

  if (gi.qv) {
    T* row = dq + rbase;
#pragma unroll
    for (int t = 0; t < TL::NT; ++t)
      store4(row + t * 16 + quad * 4, acc_dq[t][0] * scale, acc_dq[t][1] * scale, acc_dq[t][2] * scale,
             acc_dq[t][3] * scale);
  }
}

// ---------------------------------------------------------------------------
// Backward, key side: dK and dV
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void k_backward_dkdv(const T* __restrict__ q, const T* __restrict__ k,
                                                      const T* __restrict__ v, const T* __restrict__ dout,
                                                      const float* __restrict__ lse,
                                                      const float* __restrict__ delta, T* __restrict__ dk,
                                                      T* __restrict__ dv, Geom g, Prep p, float sl2, float scale) {
  using TL = Tile<T, D>;
  __shared__ __attribute__((aligned(16))) T lq[CHUNK * TL::RS];
  __shared__ __attribute__((aligned(16))) T ldo[CHUNK * TL::RS];
  __shared__ int ltok[CHUNK];
  __shared__ int4 lst[CHUNK];
  __shared__ float llse[CHUNK], ldel[CHUNK];

  const int h = g.h0 + (int)blockIdx.y, lane = threadIdx.x, r16 = lane & 15, quad = lane >> 4;
  // key blob -> this lane's key (lane & 15)
  const int kby = (g.Hp + 3) / 4, kbx = (g.Wp + 3) / 4;
  const int b = blockIdx.x;
  const int bt = b / (kby * kbx), brem = b - bt * (kby * kbx), byb = brem / kbx, bxb = brem - byb * kbx;
  const int4 kp = make_int4(bt, byb * 4 + (r16 >> 2), bxb * 4 + (r16 & 3), 0);
  const bool kvalid = kp.y < g.Hp && kp.z < g.Wp;
  const int ktok = kvalid ? (kp.x * g.Hp + kp.y) * g.Wp + kp.z : 0;

  Frag<T> kf[TL::NC], vf[TL::NC];
  const size_t kbase = ((size_t)ktok * g.H + h) * D;
#pragma unroll
  for (int c = 0; c < TL::NC; ++c) {
    if (kvalid) {
      load_frag(kf[c], k + kbase + c * 32 + quad * 8);
      load_frag(vf[c], v + kbase + c * 32 + quad * 8);
    } else {
      zero_frag(kf[c]);
      zero_frag(vf[c]);
    }
  }

  // start cells whose windows can hold a key of this blob
  const int yhi = min(byb * 4 + 3, g.Hp - 1), xhi = min(bxb * 4 + 3, g.Wp - 1);
  const int ct0 = max(bt - g.kt + 1, 0), ct1 = min(bt, g.Lt - 1);
  const int cy0 = max(byb * 4 - g.ky + 1, 0), cy1 = min(yhi, g.Ly - 1);
  const int cx0 = max(bxb * 4 - g.kx + 1, 0), cx1 = min(xhi, g.Lx - 1);
  const int nct = max(ct1 - ct0 + 1, 0), ncy = max(cy1 - cy0 + 1, 0), ncx = max(cx1 - cx0 + 1, 0);
  const int ncells = nct * ncy * ncx, ncyx = ncy * ncx;

  f32x4_t acc_dk[TL::NT], acc_dv[TL::NT];
#pragma unroll
  for (int t = 0; t < TL::NT; ++t) {
    acc_dk[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc_dv[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  int rows[8];
  chunk_rows(quad, rows);

  int ci = 0, oi = 0;  // cursor: next cell of the box, queries of it already taken
  for (;;) {
    // ---- next (up to) CHUNK queries, in cell order then query order
    int filled = 0;
    while (filled < CHUNK && ci < ncells) {
      const int c = ci + lane;
      int beg = 0, cnt = 0;
      if (c < ncells) {
        const int ct = c / ncyx, crem = c - ct * ncyx, cy = crem / ncx, cx = crem - cy * ncx;
        const int key = cell_key(g, ct0 + ct, cy0 + cy, cx0 + cx);
        beg = p.cell_ptr[key];
        cnt = p.cell_ptr[key + 1] - beg;
        if (lane == 0) {
          beg += oi;
          cnt -= oi;
        }
      }
      const int incl = wave_incl_scan(cnt, lane), excl = incl - cnt;
      const int total = __shfl(incl, 63, 64);
      const int need = CHUNK - filled;
      const int stop = min(incl, need);
      for (int e = excl; e < stop; ++e) ltok[filled + e] = p.perm[beg + (e - excl)];
      if (total <= need) {
        filled += total;
        ci += 64;
        oi = 0;
      } else {
        const unsigned long long over = __ballot(incl > need);
        const int ls = __ffsll((long long)over) - 1;
        const int excl_ls = __shfl(excl, ls, 64);
        oi = (ls == 0 ? oi : 0) + (need - excl_ls);
        ci += ls;
        filled = CHUNK;
      }
    }
    if (filled == 0) break;
    wave_lds_fence();
    if (lane < CHUNK) {
      if (lane < filled) {
        const int tok = ltok[lane];
        lst[lane] = p.starts[tok];
        llse[lane] = lse[(size_t)h * g.N + tok] * LOG2E;
        ldel[lane] = delta[(size_t)h * g.N + tok];
      } else {
        ltok[lane] = -1;
        lst[lane] = make_int4(-(1 << 29), -(1 << 29), -(1 << 29), 0);
        llse[lane] = 0.f;
        ldel[lane] = 0.f;
      }
    }
    wave_lds_fence();
    stage_rows<T, D>(lq, q, ltok, g.H, h, lane);
    stage_rows<T, D>(ldo, dout, ltok, g.H, h, lane);
    wave_lds_fence();

    float pr[8], ds[8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4_t s_acc = {0.f, 0.f, 0.f, 0.f}, dp_acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < TL::NC; ++c) {
        Frag<T> a;
        load_frag(a, lq + (u * 16 + r16) * TL::RS + c * 32 + quad * 8);
        s_acc = mma(a, kf[c], s_acc);
        load_frag(a, ldo + (u * 16 + r16) * TL::RS + c * 32 + quad * 8);
        dp_acc = mma(a, vf[c], dp_acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qr = u * 16 + quad * 4 + i;  // S[qr][key r16]
        const bool ok = in_window(kp, lst[qr], g);
        const float pij = ok ? __builtin_amdgcn_exp2f(s_acc[i] * sl2 - llse[qr]) : 0.f;
        pr[u * 4 + i] = pij;
        ds[u * 4 + i] = pij * (dp_acc[i] - ldel[qr]);
      }
    }
    Frag<T> pf, dsf;
    set_frag(pf, pr);
    set_frag(dsf, ds);
#pragma unroll
    for (int t = 0; t < TL::NT; ++t) {
      Frag<T> a;
      gather_frag<T>(a, ldo, TL::RS, rows, t * 16 + r16);
      acc_dv[t] = mma(a, pf, acc_dv[t]);
      gather_frag<T>(a, lq, TL::RS, rows, t * 16 + r16);
      acc_dk[t] = mma(a, dsf, acc_dk[t]);
    }
    wave_lds_fence();
    if (filled < CHUNK) break;
  }

  if (kvalid) {
    T* krow = dk + kbase;
    T* vrow = dv + kbase;
#pragma unroll
    for (int t = 0; t < TL::NT; ++t) {
      store4(krow + t * 16 + quad * 4, acc_dk[t][0] * scale, acc_dk[t][1] * scale, acc_dk[t][2] * scale,
             acc_dk[t][3] * scale);
      store4(vrow + t * 16 + quad * 4, acc_dv[t][0], acc_dv[t][1], acc_dv[t][2], acc_dv[t][3]);
    }
  }
}

// ---------------------------------------------------------------------------
// launches
// ---------------------------------------------------------------------------
template <typename T, int D>
static hipError_t fwd_impl(const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s) {
  dim3 grid(p.max_groups, g.nh);
  k_forward<T, D><<<grid, 64, 0, s>>>((const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse_out, g, p,
                                      a.scale * LOG2E);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t dq_impl(const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s) {
  dim3 grid_q(p.max_groups, g.nh);
  k_backward_dq<T, D><<<grid_q, 64, 0, s>>>((const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.o,
                                            (const T*)a.dout, a.lse, (T*)a.out, p.delta, g, p, a.scale * LOG2E,
                                            a.scale);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t dkdv_impl_v1(const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s) {
  const int nkb = g.F * ((g.Hp + 3) / 4) * ((g.Wp + 3) / 4);
  dim3 grid_k(nkb, g.nh);
  k_backward_dkdv<T, D><<<grid_k, 64, 0, s>>>((const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.dout,
                                              a.lse, p.delta, (T*)a.dk, (T*)a.dv, g, p, a.scale * LOG2E, a.scale);
  return hipGetLastError();
}

hipError_t launch_forward_v1(int dtype, int D, const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s) {
  if (dtype == 1) return D == 64 ? fwd_impl<u16, 64>(a, g, p, s) : fwd_impl<u16, 128>(a, g, p, s);
  return D == 64 ? fwd_impl<float, 64>(a, g, p, s) : fwd_impl<float, 128>(a, g, p, s);
}

hipError_t launch_backward_dq_v1(int dtype, int D, const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s) {
  if (dtype == 1) return D == 64 ? dq_impl<u16, 64>(a, g, p, s) : dq_impl<u16, 128>(a, g, p, s);
  return D == 64 ? dq_impl<float, 64>(a, g, p, s) : dq_impl<float, 128>(a, g, p, s);
}

hipError_t launch_backward_dkdv_v1(int dtype, int D, const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s) {
  if (dtype == 1) return D == 64 ? dkdv_impl_v1<u16, 64>(a, g, p, s) : dkdv_impl_v1<u16, 128>(a, g, p, s);
  return D == 64 ? dkdv_impl_v1<float, 64>(a, g, p, s) : dkdv_impl_v1<float, 128>(a, g, p, s);
}

}  // namespace dsa3d
