// Frame-sweeping dQ of 3D Deformable Slide Attention (MegaSlide-DiT, section
// "3D Deformable Slide Attention": the gradient of the windowed softmax attention
// with respect to the queries, dQ = scale * dS K with dS = P (dP - Delta),
// P = exp(scale Q K^T - lse), dP = dO V^T, Delta = rowsum(dO * O)), bf16.
//
// Same work decomposition as the forward (attn_fwd.hip): a workgroup sweeps the
// frames of one start blob column, every frame's key tile goes through an LDS ring
// once and serves the QS_SLOTS row tiles in flight, one per wave (a wave whose
// slot holds no tile this frame skips its MFMA work).
// A frame takes four ring steps (D = 128): V columns 0-63 and 64-127 (dP^T =
// V dO^T), then K columns 0-63 and 64-127 (S^T = K Q^T); at the last one P^T and
// dS^T follow and dQ^T += K^T dS^T reads both K steps transposed, so the ring keeps
// the previous step's tile (prefetch distance NBUF - 2).
//
// Delta comes from k_delta, one pass over O and dO.
#include "qs_common.hpp"

namespace dsa3d {

// Delta[h][n] = sum_d dO[n][h][d] O[n][h][d] (fp32), D / 8 lanes per row.  A wave
// takes 64 consecutive tokens of one head, DELTA_U row groups per trip with all their
// loads issued before the first use, so that enough bytes are in flight to stream O
// and dO at HBM rate and the results go out as whole lines of delta[h][.].
constexpr int DELTA_U = 4;
template <int D>
__global__ __launch_bounds__(256) void k_delta(const u16* __restrict__ o, const u16* __restrict__ dout,
                                               float* __restrict__ delta, int N, int H) {
  constexpr int LPR = D / 8, RPW = 64 / LPR;  // lanes per row, rows per wave and group
  const int lane = threadIdx.x & 63, sub = lane % LPR, rr = lane / LPR;
  const long long wv = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nchunk = (N + 63) / 64;
  if (wv >= (long long)nchunk * H) return;
  const int h = (int)(wv / nchunk), n0 = (int)(wv - (long long)h * nchunk) * 64;
  for (int g0 = 0; g0 < 64 / RPW; g0 += DELTA_U) {
    uint4 a[DELTA_U], b[DELTA_U];
#pragma unroll
    for (int u = 0; u < DELTA_U; ++u) {
      const int n = n0 + (g0 + u) * RPW + rr;
      if (n < N) {
        const size_t row = ((size_t)n * H + h) * D + sub * 8;
        a[u] = *reinterpret_cast<const uint4*>(o + row);
        b[u] = *reinterpret_cast<const uint4*>(dout + row);
      } else {
        a[u] = b[u] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int u = 0; u < DELTA_U; ++u) {
      const int n = n0 + (g0 + u) * RPW + rr;
      const uint32_t av[4] = {a[u].x, a[u].y, a[u].z, a[u].w}, bv[4] = {b[u].x, b[u].y, b[u].z, b[u].w};
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s += __uint_as_float(av[i] << 16) * __uint_as_float(bv[i] << 16);
        s += __uint_as_float(av[i] & 0xffff0000u) * __uint_as_float(bv[i] & 0xffff0000u);
      }
#pragma unroll
      for (int m = 1; m < LPR; m <<= 1) s += __shfl_xor(s, m, 64);
      if (n < N && sub == 0) delta[(size_t)h * N + n] = s;
    }
  }
}

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;

template <int D, int NBY, int NBX>
struct DqCfg {
  static constexpr int NB = NBY * NBX;
  static constexpr int NBPAD = (NB + 1) & ~1;
  static constexpr int NPAIR = NBPAD / 2;
  static constexpr int NPH = D / 64, NPH2 = 2 * NPH;
  static constexpr int TILE = NBPAD * 16 * 128;
  static constexpr int NLOADS = NBPAD * 2;      // 1 KB loads per phase tile (pad block too)
  static constexpr int NBUF = 4, PD = NBUF - 2;  // the previous K step stays readable
  static constexpr int NC = D / 32, NT = D / 16;
  static constexpr int RTILE = NPH * 2048;       // one staged row tile (Q or dO)
  static constexpr int SLOT = 2 * RTILE + 128;   // Q, dO, lse (64 B), Delta (64 B)
};

// Row-tile slots per wave (see attn_fwd.hip): one, so 8 waves run 2 per SIMD.
#ifndef DSA3D_DQ_NS
#define DSA3D_DQ_NS 1
#endif
constexpr int DQ_NS = DSA3D_DQ_NS;
constexpr int DQ_NW = QS_SLOTS / DQ_NS;

template <int D, int NBY, int NBX>
__global__ __launch_bounds__(64 * DQ_NW) void k_dq_qs(const u16* __restrict__ q, const u16* __restrict__ k,
                                                     const u16* __restrict__ v, const u16* __restrict__ dout,
                                                     const float* __restrict__ lse, const float* __restrict__ delta,
                                                     u16* __restrict__ dq, Geom g, Prep p, float sl2, float scale) {
  using C = DqCfg<D, NBY, NBX>;
  constexpr int NS = DQ_NS;
  __shared__ __attribute__((aligned(1024))) char ring[C::NBUF][C::TILE];
  __shared__ __attribute__((aligned(1024))) char stage[QS_SLOTS][C::SLOT];
  __shared__ QsPass T;

  const int nbc = g.nby * g.nbx, nw = qs_items(g);
  int L = xcd_remap(blockIdx.x, nw * g.nh);
  const int hl = L / nw, w = L - hl * nw, h = g.h0 + hl;
  const int bc = w % nbc;
  const int by = bc / g.nbx, bx = bc - by * g.nbx;
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, quad = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // tile loads per wave and step, the same for every wave (padding loads)
  constexpr int MY_LOADS = (C::NLOADS + DQ_NW - 1) / DQ_NW;
  __shared__ int s_sink[4];

  int roff[C::NC / C::NPH], toff[C::NT / C::NPH];
#pragma unroll
  for (int c = 0; c < C::NC / C::NPH; ++c) roff[c] = sw(r16, c * 64 + quad * 16);
#pragma unroll
  for (int t = 0; t < C::NT / C::NPH; ++t) toff[t] = sw(4 * quad + (r16 >> 2), (t * 16 + 4 * (r16 & 3)) * 2);

  Frag<u16> qf[NS][C::NC], dof[NS][C::NC];
  f32x4_t dqa[NS][C::NT];
  f32x4_t sacc[NS][C::NB], dpa[NS][C::NB];
  Frag<u16> dsf[NS][C::NPAIR];
  shortx4_t dsl[NS];  // dS^T of the unpaired last key block (odd NB), 4 keys per lane
  float ybias[NS][NBY], xbias[NS][NBX][4];
  float lse2[NS], dlt[NS];
  int qn[NS], fend[NS], rt[NS];  // rt: the row's slice (it sees frames rt .. rt + kt - 1)
#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int c = 0; c < C::NC; ++c) {
      zero_frag(qf[s][c]);
      zero_frag(dof[s][c]);
    }
#pragma unroll
    for (int t = 0; t < C::NT; ++t) dqa[s][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NBY; ++i) ybias[s][i] = 0.f;
#pragma unroll
    for (int j = 0; j < NBX; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) xbias[s][j][i] = 0.f;
    lse2[s] = 0.f;
    dlt[s] = 0.f;
    qn[s] = -1;
    fend[s] = -1;
    rt[s] = 0;
  }

  KeyTileLoadsW<D, NBX, C::NB, C::NBPAD, DQ_NW> kl;
  kl.init(g, h, by, bx, lane, wave);
  const size_t frame_el = (size_t)g.Hp * g.Wp * g.H * D;
  const int* sp = p.qs + p.qs_off[(g.ph > 1 ? hl : 0) * nw + w];  // per-head offsets: the head's lists
  const int npass = sp[0];
  sp += 1;
  for (int pass = 0; pass < npass; ++pass) {
    load_pass(T, sp, p, tid, 64 * DQ_NW);
    const int nf = __builtin_amdgcn_readfirstlane(T.hdr[0]);
    const int nsteps = nf * C::NPH2;
    // step x: V phases first, then K phases.  The rows, lse and Delta of tiles that
    // start at a frame go out just before its first tile loads.
    auto issue_step = [&](int x) {
      const int fi = x / C::NPH2, ph = x - fi * C::NPH2;
      const int f = __builtin_amdgcn_readfirstlane(T.frames[fi]);
      if (ph == 0) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int sl = NS * wave + s;
          const int t = __builtin_amdgcn_readfirstlane((int)T.act[fi][sl]);
          if (t >= 0) {
            issue_rows<D>(stage[sl], q, T.ids[t], g, h, lane);
            issue_rows<D>(stage[sl] + C::RTILE, dout, T.ids[t], g, h, lane);
            if (lane < 16) {
              const size_t n = T.ids[t][lane];
              dma4(lse + (size_t)h * g.N + n, stage[sl] + 2 * C::RTILE);
              dma4(delta + (size_t)h * g.N + n, stage[sl] + 2 * C::RTILE + 64);
            }
          }
        }
      }
      // this wave's tile loads (offsets inside a frame computed once)
      kl.issue(ring[x % C::NBUF], (ph < C::NPH ? v : k) + f * frame_el + (ph % C::NPH) * 64, lane, k, s_sink);
    };
    int issued = 0;
    for (; issued < C::PD && issued < nsteps; ++issued) issue_step(issued);
    wait_vmcnt(0);
    __syncthreads();

    // the frame and this wave's activating tile, carried from the read one frame
    // ahead below (one slot per wave)
    int f_cur = nf > 0 ? __builtin_amdgcn_readfirstlane(T.frames[0]) : 0;
    int t_cur = nf > 0 && NS == 1 ? __builtin_amdgcn_readfirstlane((int)T.act[0][wave]) : -1;
    // The dQ^T products of the last K step's own columns run one step late, in the
    // next frame's first (light) step, whose ring still holds that tile: pend says
    // they are due (with dS^T kept in dsf / dsl), pf is their frame.  A tile's dQ row
    // is written once they are done.
    bool pend = false;
    int pf = -1;
    // dQ^T += K^T dS^T over the columns of K column phase kp (the tile at kt_): per
    // key-block pair, its transposed reads for all column tiles together (from base
    // addresses fixed before the first read, block offsets in the instruction), then
    // its MFMAs; a single last block is a 16-deep product with half the reads
    auto dqt_products = [&](const char* kt_, int kp) {
      constexpr int NDT = C::NT / C::NPH;
      static_assert(NDT == 4, "four column tiles per phase");
      lds_char* vb[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) vb[dt] = (lds_char*)(kt_ + toff[dt]);
      __asm__ __volatile__("" : "+v"(vb[0]), "+v"(vb[1]), "+v"(vb[2]), "+v"(vb[3]));
#pragma unroll
      for (int c = 0; c < C::NPAIR; ++c) {
        shortx4_t lo[NDT], hi[NDT];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          lds_char* pa = vb[dt] + (2 * c) * 2048;
          lo[dt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t*)pa);
          if (2 * c + 1 < C::NB) hi[dt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t*)(pa + 2048));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int ot = kp * NDT + dt;
          if (2 * c + 1 < C::NB) {
            Frag<u16> a;
            const shortx4_t both[2] = {lo[dt], hi[dt]};
            __builtin_memcpy(&a.v, both, 16);
#pragma unroll
            for (int s = 0; s < NS; ++s) dqa[s][ot] = mma(a, dsf[s][c], dqa[s][ot]);
          } else {
#pragma unroll
            for (int s = 0; s < NS; ++s)
              dqa[s][ot] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lo[dt], dsl[s], dqa[s][ot], 0, 0, 0);
          }
        }
      }
    };
    auto flush = [&](const char* kt_) {
      if (pend) {
        dqt_products(kt_, C::NPH - 1);
        // ---- tiles whose last frame that was: write dQ = scale dQ^T^T
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          if (pf == fend[s]) {
            if (qn[s] >= 0) {
              u16* row = dq + ((size_t)qn[s] * g.H + h) * D;
#pragma unroll
              for (int t = 0; t < C::NT; ++t)
                store4(row + t * 16 + quad * 4, dqa[s][t][0] * scale, dqa[s][t][1] * scale, dqa[s][t][2] * scale,
                       dqa[s][t][3] * scale);
            }
            fend[s] = -1;
          }
        }
        pend = false;
      }
    };
    for (int fi = 0; fi < nf; ++fi) {
      const int f = f_cur;
      // what this frame's issues need, read once here rather than behind a wait in
      // each step: the next frame, and the rows of the tile that starts there in this
      // wave's slot (its Q / dO rows, lse and Delta go out PD steps before it)
      const bool has_next = fi + 1 < nf;
      const int fnext = has_next ? __builtin_amdgcn_readfirstlane(T.frames[fi + 1]) : 0;
      const int tnext = has_next && NS == 1 ? __builtin_amdgcn_readfirstlane((int)T.act[fi + 1][wave]) : -1;
      int ntok0 = 0, ntok1 = 0, ntokl = 0;
      if (tnext >= 0) {
        ntok0 = T.ids[tnext][lane >> 3];
        ntok1 = T.ids[tnext][8 + (lane >> 3)];
        ntokl = T.ids[tnext][lane & 15];
      }

      static_for<0, C::NPH2>([&](auto PHC) {
        constexpr int ph = decltype(PHC)::value;
        constexpr int kph = ph - C::NPH;  // K column phase (ph >= NPH)
        const int st = fi * C::NPH2 + ph;
        if (issued < nsteps) {
          if constexpr (NS == 1) {
            // issued == st + PD: its frame and phase are known here
            constexpr int phx = (ph + C::PD) % C::NPH2;
            constexpr bool in_next = ph + C::PD >= C::NPH2;
            static_assert(C::PD < 2 * C::NPH2, "an issue reaches at most one frame ahead");
            const int fx = in_next ? fnext : f;
            if constexpr (phx == 0) {
              if (tnext >= 0) {
                char* sg = stage[wave];
                issue_rows_tok<D>(sg, q, ntok0, ntok1, g, h, lane);
                issue_rows_tok<D>(sg + C::RTILE, dout, ntok0, ntok1, g, h, lane);
                if (lane < 16) {
                  dma4(lse + (size_t)h * g.N + ntokl, sg + 2 * C::RTILE);
                  dma4(delta + (size_t)h * g.N + ntokl, sg + 2 * C::RTILE + 64);
                }
              }
            }
            kl.issue(ring[issued % C::NBUF], (phx < C::NPH ? v : k) + fx * frame_el + (phx % C::NPH) * 64, lane, k,
                     s_sink);
          } else {
            issue_step(issued);
          }
          ++issued;
        }
        const char* tb = ring[st % C::NBUF];
        // opaque per step: keeps the compiler from precomputing every fragment
        // address of every ring slot outside the loop
#pragma unroll
        for (int c = 0; c < C::NC / C::NPH; ++c) __asm__ __volatile__("" : "+v"(roff[c]));
#pragma unroll
        for (int t = 0; t < C::NT / C::NPH; ++t) __asm__ __volatile__("" : "+v"(toff[t]));
        if constexpr (ph == 0) {
          // the previous frame's late dQ^T products (its last K tile is the previous
          // ring slot), then the tiles that start with this frame
          flush(ring[(st + C::NBUF - 1) % C::NBUF]);
    #pragma unroll
          for (int s = 0; s < NS; ++s) {
            const int sl = NS * wave + s;
            const int t = NS == 1 ? t_cur : __builtin_amdgcn_readfirstlane((int)T.act[fi][sl]);
            if (t >= 0) {
    #pragma unroll
              for (int c = 0; c < C::NC; ++c) {
                const int off = (c >> 1) * 2048 + sw(r16, (c & 1) * 64 + quad * 16);
                load_frag(qf[s][c], (const u16*)(stage[sl] + off));
                load_frag(dof[s][c], (const u16*)(stage[sl] + C::RTILE + off));
              }
              lse2[s] = reinterpret_cast<const float*>(stage[sl] + 2 * C::RTILE)[r16] * LOG2E;
              dlt[s] = reinterpret_cast<const float*>(stage[sl] + 2 * C::RTILE + 64)[r16];
              const int2 st = T.st[t][r16];
    #pragma unroll
              for (int i = 0; i < NBY; ++i)
                ybias[s][i] = (unsigned)(4 * by + 4 * i + quad - st.x) < (unsigned)g.ky ? 0.f : -INFINITY;
    #pragma unroll
              for (int j = 0; j < NBX; ++j)
    #pragma unroll
                for (int i = 0; i < 4; ++i)
                  xbias[s][j][i] = (unsigned)(4 * bx + 4 * j + i - st.y) < (unsigned)g.kx ? 0.f : -INFINITY;
              qn[s] = st.x >= 0 ? T.ids[t][r16] : -1;
              fend[s] = __builtin_amdgcn_readfirstlane(T.tlast[t]) + g.kt - 1;
              rt[s] = __builtin_amdgcn_readfirstlane(T.tau[t]) + T.dt[t][r16];
    #pragma unroll
              for (int tt = 0; tt < C::NT; ++tt) dqa[s][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
          }
        }
        // with one slot per wave, a wave whose slot holds no tile this frame skips its
        // MFMA work (a uniform branch) and leaves the SIMD to its partner
        const bool busy = NS > 1 || fend[0] >= f;
        if (busy) {
        // ---- dP^T += V dO^T (ph < NPH) or S^T += K Q^T (ph >= NPH) over this column phase
        if constexpr (ph == 0 || ph == C::NPH) {
#pragma unroll
          for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int b = 0; b < C::NB; ++b) {
              if constexpr (ph == 0)  // dP - Delta: the products accumulate onto -Delta
                dpa[s][b] = f32x4_t{-dlt[s], -dlt[s], -dlt[s], -dlt[s]};
              else
                sacc[s][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
        // V (or K) fragments in groups of KG blocks: the group's reads together (from
        // base addresses fixed before the first read, block offsets in the
        // instruction), then its MFMAs
        lds_char* kb[C::NC / C::NPH];
#pragma unroll
        for (int c = 0; c < C::NC / C::NPH; ++c) kb[c] = (lds_char*)(tb + roff[c]);
        static_assert(C::NC / C::NPH == 2, "two column groups per step");
        __asm__ __volatile__("" : "+v"(kb[0]), "+v"(kb[1]));
#pragma unroll
        for (int c = 0; c < C::NC / C::NPH; ++c) {
          constexpr int KG = 4;
#pragma unroll
          for (int b0 = 0; b0 < C::NB; b0 += KG) {
            Frag<u16> a[KG];
#pragma unroll
            for (int j = 0; j < KG; ++j)
              if (b0 + j < C::NB) a[j].v = *(const lds_bf16x8_t*)(kb[c] + (b0 + j) * 2048);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < KG; ++j) {
              if (b0 + j >= C::NB) continue;
              const int b = b0 + j;
#pragma unroll
              for (int s = 0; s < NS; ++s) {
                if constexpr (ph < C::NPH)
                  dpa[s][b] = mma(a[j], dof[s][ph * (C::NC / C::NPH) + c], dpa[s][b]);
                else
                  sacc[s][b] = mma(a[j], qf[s][kph * (C::NC / C::NPH) + c], sacc[s][b]);
              }
            }
          }
        }
        if constexpr (ph == C::NPH2 - 1) {
          // ---- P^T and dS^T on the window, as bf16 pairs of key blocks
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            // a row whose slice does not read this frame (a tile of several slices)
            // has P = 0 there; lse folds into the row bias (exact: biases are 0 or -inf)
            const float tb = (unsigned)(f - rt[s]) < (unsigned)g.kt ? 0.f : -INFINITY;
            float yb[NBY];
#pragma unroll
            for (int i = 0; i < NBY; ++i) yb[i] = (ybias[s][i] + tb) - lse2[s];
            auto ds_of = [&](int b, int i) {
              const float x = sacc[s][b][i] * sl2 + (yb[b / NBX] + xbias[s][b % NBX][i]);
              return __builtin_amdgcn_exp2f(x) * dpa[s][b][i];
            };
            static_for<0, C::NPAIR>([&](auto CC) {
              constexpr int c = decltype(CC)::value;
              if constexpr (2 * c + 1 < C::NB) {
                float d8[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  d8[i] = ds_of(2 * c, i);
                  d8[i + 4] = ds_of(2 * c + 1, i);
                }
                set_frag(dsf[s][c], d8);
              } else {
                const bf16x4_t d4 =
                    __builtin_convertvector((f32x4_t{ds_of(2 * c, 0), ds_of(2 * c, 1), ds_of(2 * c, 2), ds_of(2 * c, 3)}),
                                            bf16x4_t);
                __builtin_memcpy(&dsl[s], &d4, 8);
              }
            });
          }
          // ---- dQ^T += K^T dS^T over the earlier K steps' columns now (their tiles
          // leave the ring next step), over this step's own columns one step late
          pend = true;
          pf = f;
#pragma unroll
          for (int kp = 0; kp < C::NPH - 1; ++kp) dqt_products(ring[(st - (C::NPH - 1 - kp)) % C::NBUF], kp);
        }
        }  // busy
        if (issued - st - 2 == C::PD - 1)
          wait_vmcnt_c<MY_LOADS * (C::PD - 1)>();
        else
          wait_vmcnt(MY_LOADS * max(issued - st - 2, 0));
        lds_barrier();
      });
      f_cur = fnext;
      t_cur = tnext;
    }
    // the pass's last K tile is still in the ring (no loads follow)
    if (nf > 0) flush(ring[(nf * C::NPH2 - 1) % C::NBUF]);
  }
}

bool dq_qs_eligible(const Geom& g, int dtype, int D) { return fwd_qs_eligible(g, dtype, D); }

template <int D, int NBY, int NBX>
static hipError_t dq_qs_impl(const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s) {
  const long long total = (long long)qs_items(g) * g.nh;
  k_dq_qs<D, NBY, NBX><<<(unsigned)total, 64 * DQ_NW, 0, s>>>((const u16*)a.q, (const u16*)a.k, (const u16*)a.v,
                                                              (const u16*)a.dout, a.lse, p.delta, (u16*)a.out, g, p,
                                                              a.scale * LOG2E, a.scale);
  return hipGetLastError();
}

template <int D>
static hipError_t dq_qs_dispatch(const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s) {
  const int nby = (4 + g.ky - 1 + 3) / 4 <= 2 ? 2 : 3, nbx = (4 + g.kx - 1 + 3) / 4 <= 2 ? 2 : 3;
  if (nby == 2) return nbx == 2 ? dq_qs_impl<D, 2, 2>(a, g, p, s) : dq_qs_impl<D, 2, 3>(a, g, p, s);
  return nbx == 2 ? dq_qs_impl<D, 3, 2>(a, g, p, s) : dq_qs_impl<D, 3, 3>(a, g, p, s);
}

hipError_t launch_delta(int D, const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s) {
  const long long waves = (long long)((g.N + 63) / 64) * g.H;
  const unsigned blocks = (unsigned)((waves + 3) / 4);
  if (D == 64)
    k_delta<64><<<blocks, 256, 0, s>>>((const u16*)a.o, (const u16*)a.dout, p.delta, g.N, g.H);
  else
    k_delta<128><<<blocks, 256, 0, s>>>((const u16*)a.o, (const u16*)a.dout, p.delta, g.N, g.H);
  return hipGetLastError();
}

hipError_t launch_dq_qs(int D, const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s) {
  return D == 64 ? dq_qs_dispatch<64>(a, g, p, s) : dq_qs_dispatch<128>(a, g, p, s);
}

}  // namespace dsa3d
