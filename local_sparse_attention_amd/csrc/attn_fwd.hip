// Frame-sweeping forward of 3D Deformable Slide Attention (MegaSlide-DiT, section
// "3D Deformable Slide Attention", the attention of Eq. (1)) on gfx950, bf16.
//
// A workgroup owns one start blob column (by, bx) of one head and QS_TS slices of
// it, and sweeps the frames its row tiles read (the pass schedule built by
// qsched.hip).  Every frame's key tile -- the (4 + ky - 1) x (4 + kx - 1) keys
// anchored at (4 by, 4 bx), in NBY x NBX blocks of 4 x 4 -- is staged once into an
// LDS ring with direct global->LDS loads (issued by two loader waves) and read by
// all QS_SLOTS_FWD row tiles in flight (one per compute wave), which belong to the kt
// slices that read that frame.
//
// Per frame and busy slot (a wave whose slot holds no tile this frame skips it):
//   S^T = K Q^T        16x16x32 bf16 MFMA, K rows from LDS, Q^T held in registers
//   mask to the query's own window (additive 0 / -inf biases set at activation),
//   online softmax in the log2 domain, P kept as bf16 fragments
//   O^T += V^T P^T     V^T by transposed LDS reads (ds_read_b64_tr_b16)
// A slot's row tile is activated at its first frame (Q rows staged by direct
// loads issued with the frame's first tile loads) and written out after its last
// (the kt-th; later for a tile of several slices, whose rows each see only the kt
// frames of their own slice and no keys in the others).
#include "qs_common.hpp"

namespace dsa3d {

template <int D, int NBY, int NBX>
struct FwdCfg {
  static constexpr int NB = NBY * NBX;              // key blocks of a frame tile
  static constexpr int NPAIR = (NB + 1) / 2;        // 32-key pairs of the V pass (the last may be one block)
  static constexpr int NPH = D / 64;                // 128-byte column phases per K (or V) row
  static constexpr int NPH2 = 2 * NPH;              // ring steps per frame
  static constexpr int TILE = NB * 16 * 128;        // one phase tile
  static constexpr int NLOADS = NB * 2;             // 1 KB direct loads per phase tile
  static constexpr int NBUF = 5, PD = NBUF - 1;     // ring depth, steps loaded ahead
  static constexpr int NC = D / 32, NT = D / 16;
  static constexpr int QTILE = 16 * 128;            // one phase of a staged row tile
};

// Row-tile slots per compute wave: with one (the default), the QS_SLOTS_FWD = 10
// slots take 10 waves (with the two loaders, 3 per SIMD: the 168-register cap that 8
// compute waves and the loaders already had), so one wave's LDS and scalar work
// issues beside another's VALU and MFMA work; ten slots rather than eight leave fewer
// tiles waiting for a further pass over the frames (11% fewer frames swept at the
// 256-frame workload).  With two slots a wave, a K / V fragment read from LDS feeds
// the MFMAs of both, but five waves hide latency poorly (measured slower).
#ifndef DSA3D_FWD_NS
#define DSA3D_FWD_NS 1
#endif
constexpr int FWD_NS = DSA3D_FWD_NS;
constexpr int FWD_NW = QS_SLOTS_FWD / FWD_NS;  // compute waves
constexpr int FWD_LW = 2;                  // loader waves

template <int D, int NBY, int NBX>
__global__ __launch_bounds__(64 * (FWD_NW + FWD_LW)) void k_forward_qs(const u16* __restrict__ q, const u16* __restrict__ k,
                                                           const u16* __restrict__ v, u16* __restrict__ out,
                                                           float* __restrict__ lse, Geom g, Prep p, float sl2) {
  using C = FwdCfg<D, NBY, NBX>;
  constexpr int NS = FWD_NS;
  __shared__ __attribute__((aligned(1024))) char ring[C::NBUF][C::TILE];
  __shared__ __attribute__((aligned(1024))) char stage[QS_SLOTS_FWD][C::NPH * C::QTILE];
  __shared__ QsPass T;

  const int nbc = g.nby * g.nbx, nw = qs_items(g);
  int L = xcd_remap(blockIdx.x, nw * g.nh);
  const int hl = L / nw, w = L - hl * nw, h = g.h0 + hl;
  const int chunk = w / nbc, bc = w - chunk * nbc;
  const int by = bc / g.nbx, bx = bc - by * g.nbx;
  (void)chunk;
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, quad = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int NW = FWD_NW + FWD_LW;
  // FWD_LW loader waves issue every direct load (key tiles, Q rows) and wait for
  // them; the compute waves only meet them at the barrier that closes each step.
  // Tile loads per loader wave and step: the same for each, so the steady-state
  // wait is one immediate.
  static_assert(C::NLOADS % FWD_LW == 0, "tile loads split evenly over the loader waves");
  constexpr int MY_LOADS = C::NLOADS / FWD_LW;
  const bool loader = wave >= FWD_NW;
  const int lw = wave - FWD_NW;

  const int* sp = p.qs + p.qs_off[(g.ph > 1 ? hl : 0) * nw + w];  // per-head offsets: the head's lists
  const int npass = sp[0];
  sp += 1;
  if (loader) {
    for (int pass = 0; pass < npass; ++pass) {
      load_pass(T, sp, p, tid, 64 * NW);
      const int nf = __builtin_amdgcn_readfirstlane(T.hdr[0]);
      const int nsteps = nf * C::NPH2;
      static_for<0, FWD_LW>([&](auto LWC) {
        constexpr int LWI = decltype(LWC)::value;
        if (lw != LWI) return;
        KeyTileLoads<D, NBX, C::NB, C::NB, FWD_LW, LWI> kl;
        kl.init(g, h, by, bx, lane);
        const size_t frame_el = (size_t)g.Hp * g.Wp * g.H * D;
        // step x: phase x % NPH2 of frame index x / NPH2; K phases first, then V.  Q
        // rows of the tiles that start at a frame go out just before its first tile
        // loads, so the wait that covers those covers them too.
        auto issue_step = [&](int x) {
          const int fi = x / C::NPH2, ph = x - fi * C::NPH2;
          const int f = __builtin_amdgcn_readfirstlane(T.frames[fi]);
          if (ph == 0) {
#pragma unroll
            for (int sl = LWI; sl < QS_SLOTS_FWD; sl += FWD_LW) {
              const int t = __builtin_amdgcn_readfirstlane((int)T.act[fi][sl]);
              if (t >= 0) issue_rows<D>(stage[sl], q, T.ids[t], g, h, lane);
            }
          }
          kl.issue(ring[x % C::NBUF], (ph < C::NPH ? k : v) + f * frame_el + (ph % C::NPH) * 64, lane, k,
                   stage[0]);  // (no padding: the loads split evenly)
        };
        int issued = 0;
        for (; issued < C::PD && issued < nsteps; ++issued) issue_step(issued);
        wait_vmcnt(0);
        __syncthreads();
        for (int st = 0; st < nsteps; ++st) {
          if (issued < nsteps) {
            issue_step(issued);
            ++issued;
          }
          // step st + 1 (and the Q rows issued before it) must have landed; later
          // steps may stay in flight (Q rows only make the count stricter)
          if (issued - st - 2 == C::PD - 1)
            wait_vmcnt_c<MY_LOADS * (C::PD - 1)>();
          else
            wait_vmcnt(MY_LOADS * max(issued - st - 2, 0));
          lds_barrier();
        }
      });
    }
    return;
  }

  // per-lane LDS offsets of the fragments inside a phase tile (block 0)
  int roff[C::NC / C::NPH], toff[C::NT / C::NPH];
#pragma unroll
  for (int c = 0; c < C::NC / C::NPH; ++c) roff[c] = sw(r16, c * 64 + quad * 16);
#pragma unroll
  for (int t = 0; t < C::NT / C::NPH; ++t) toff[t] = sw(4 * quad + (r16 >> 2), (t * 16 + 4 * (r16 & 3)) * 2);

  // slot state (slots 2 wave, 2 wave + 1)
  Frag<u16> qf[NS][C::NC];
  f32x4_t oacc[NS][C::NT];
  float ybias[NS][NBY], xbias[NS][NBX][4];
  float m_run[NS], l_run[NS];
  int qn[NS], fend[NS], rt[NS];  // rt: the row's slice (it sees frames rt .. rt + kt - 1)
#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int c = 0; c < C::NC; ++c) zero_frag(qf[s][c]);
#pragma unroll
    for (int t = 0; t < C::NT; ++t) oacc[s][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NBY; ++i) ybias[s][i] = 0.f;
#pragma unroll
    for (int j = 0; j < NBX; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) xbias[s][j][i] = 0.f;
    m_run[s] = 0.f;
    l_run[s] = 0.f;
    qn[s] = -1;
    fend[s] = -1;
    rt[s] = 0;
  }

  for (int pass = 0; pass < npass; ++pass) {
    load_pass(T, sp, p, tid, 64 * NW);
    const int nf = __builtin_amdgcn_readfirstlane(T.hdr[0]);
    __syncthreads();  // the loader waves' pipeline fill
    for (int fi = 0; fi < nf; ++fi) {
      const int f = __builtin_amdgcn_readfirstlane(T.frames[fi]);
      // scores and P of this frame (not carried from one frame to the next)
      f32x4_t sacc[NS][C::NB];
      Frag<u16> pf[NS][C::NPAIR];
      shortx4_t pl[NS];  // P^T of the unpaired last key block (odd NB), 4 keys per lane
      // ---- activations: Q fragments, window biases, fresh softmax state
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int sl = NS * wave + s;
        const int t = __builtin_amdgcn_readfirstlane((int)T.act[fi][sl]);
        if (t >= 0) {
#pragma unroll
          for (int c = 0; c < C::NC; ++c)
            load_frag(qf[s][c], (const u16*)(stage[sl] + (c >> 1) * C::QTILE + sw(r16, (c & 1) * 64 + quad * 16)));
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
          m_run[s] = -INFINITY;  // the first rescale (alpha = 0) clears O and l
        }
      }

      static_for<0, C::NPH2>([&](auto PHC) {
        constexpr int ph = decltype(PHC)::value;
        const int st = fi * C::NPH2 + ph;
        const char* tb = ring[st % C::NBUF];
        typedef __attribute__((address_space(3))) char lds_char;
        typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;
        // opaque per step: keeps the compiler from precomputing every fragment
        // address of every ring slot outside the loop (more registers than a third
        // wave per SIMD leaves)
#pragma unroll
        for (int c = 0; c < C::NC / C::NPH; ++c) __asm__ __volatile__("" : "+v"(roff[c]));
#pragma unroll
        for (int t = 0; t < C::NT / C::NPH; ++t) __asm__ __volatile__("" : "+v"(toff[t]));
        // with one slot per wave, a wave whose slot holds no tile this frame skips its
        // MFMA and softmax work (a uniform branch) and leaves the SIMD to its partner
        const bool busy = NS > 1 || fend[0] >= f;
        if constexpr (ph < C::NPH) {
          if (busy) {
          // ---- S^T += K Q^T over this column phase
          if constexpr (ph == 0) {
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
              for (int b = 0; b < C::NB; ++b) sacc[s][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
          // K fragments in groups of KG blocks: the group's reads together (from fixed
          // base addresses, one per column group, set before the first read; block
          // offsets in the instruction), then its MFMAs
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
              for (int j = 0; j < KG; ++j)
                if (b0 + j < C::NB)
#pragma unroll
                  for (int s = 0; s < NS; ++s)
                    sacc[s][b0 + j] = mma(a[j], qf[s][ph * (C::NC / C::NPH) + c], sacc[s][b0 + j]);
            }
          }
          if constexpr (ph == C::NPH - 1) {
            // ---- window mask, online softmax (log2 domain), P as bf16 pairs
#pragma unroll
            for (int s = 0; s < NS; ++s) {
              // a row whose slice does not read this frame (a tile of several slices)
              // sees none of its keys.  Scores are taken relative to the current
              // reference max mref (0 before the row's first key), which folds into
              // the biases.
              const float tb = (unsigned)(f - rt[s]) < (unsigned)g.kt ? 0.f : -INFINITY;
              const float mref0 = m_run[s] == -INFINITY ? 0.f : m_run[s];
              float yb[NBY];
#pragma unroll
              for (int i = 0; i < NBY; ++i) yb[i] = ybias[s][i] + (tb - mref0);
              float cm = -INFINITY;
#pragma unroll
              for (int b = 0; b < C::NB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const float x = sacc[s][b][i] * sl2 + (yb[b / NBX] + xbias[s][b % NBX][i]);
                  sacc[s][b][i] = x;
                  cm = fmaxf(cm, x);
                }
              cm = quad_max_rs(cm);
              // The reference max moves only when a score exceeds it by more than
              // 2^8 (or on a row's first frame with keys, m = -inf): P <= 256
              // otherwise, and O and l need no rescale.  A row that has seen no key
              // yet keeps m = -inf (alpha = 0 clears its O and l until it does).
              if (__ballot(cm > (m_run[s] == -INFINITY ? -INFINITY : 8.f))) {
                const float mn = fmaxf(m_run[s], cm + mref0);
                const float mref = (mn == -INFINITY) ? 0.f : mn;
                const float alpha = __builtin_amdgcn_exp2f(m_run[s] - mref);
                l_run[s] *= alpha;
#pragma unroll
                for (int t = 0; t < C::NT; ++t) oacc[s][t] *= alpha;
                m_run[s] = mn;
                const float d = mref0 - mref;
#pragma unroll
                for (int b = 0; b < C::NB; ++b) sacc[s][b] += d;
              }
              float ps = 0.f;
              static_for<0, C::NPAIR>([&](auto CC) {
                constexpr int c = decltype(CC)::value;
                if constexpr (2 * c + 1 < C::NB) {
                  float pr[8];
#pragma unroll
                  for (int i = 0; i < 4; ++i) {
                    pr[i] = __builtin_amdgcn_exp2f(sacc[s][2 * c][i]);
                    pr[i + 4] = __builtin_amdgcn_exp2f(sacc[s][2 * c + 1][i]);
                    ps += pr[i] + pr[i + 4];
                  }
                  set_frag(pf[s][c], pr);
                } else {
                  f32x4_t e;
#pragma unroll
                  for (int i = 0; i < 4; ++i) {
                    e[i] = __builtin_amdgcn_exp2f(sacc[s][2 * c][i]);
                    ps += e[i];
                  }
                  const bf16x4_t p4 = __builtin_convertvector(e, bf16x4_t);
                  __builtin_memcpy(&pl[s], &p4, 8);
                }
              });
              ps = quad_sum_rs(ps);
              l_run[s] += ps;
            }
          }
          }
        } else {
          // ---- O^T += V^T P^T over this column phase
          constexpr int vph = ph - C::NPH;
          if (busy) {
          constexpr int NDT = C::NT / C::NPH;
          // one address per column tile, opaque, so that every read of the step takes
          // its block offset in the instruction and no address is rewritten between reads
          lds_char* vb[NDT];
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) vb[dt] = (lds_char*)(tb + toff[dt]);
          static_assert(NDT == 4, "four column tiles per step");
          __asm__ __volatile__("" : "+v"(vb[0]), "+v"(vb[1]), "+v"(vb[2]), "+v"(vb[3]));
#pragma unroll
          for (int c = 0; c < C::NPAIR; ++c) {
            constexpr int ot = vph * (C::NT / C::NPH);
            // the pair's transposed reads for all its column tiles first, then its MFMAs
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
              if (2 * c + 1 < C::NB) {
                Frag<u16> a;
                const shortx4_t both[2] = {lo[dt], hi[dt]};
                __builtin_memcpy(&a.v, both, 16);
#pragma unroll
                for (int s = 0; s < NS; ++s) oacc[s][ot + dt] = mma(a, pf[s][c], oacc[s][ot + dt]);
              } else {
                // a single last block: a 16-deep product
#pragma unroll
                for (int s = 0; s < NS; ++s)
                  oacc[s][ot + dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lo[dt], pl[s], oacc[s][ot + dt], 0, 0, 0);
              }
            }
          }
          }
          if constexpr (ph == C::NPH2 - 1) {
            // ---- tiles whose last frame this was: normalise and write
#pragma unroll
            for (int s = 0; s < NS; ++s) {
              if (f == fend[s]) {
                if (qn[s] >= 0) {
                  const float inv = 1.f / l_run[s];
                  u16* orow = out + ((size_t)qn[s] * g.H + h) * D;
#pragma unroll
                  for (int t = 0; t < C::NT; ++t)
                    store4(orow + t * 16 + quad * 4, oacc[s][t][0] * inv, oacc[s][t][1] * inv, oacc[s][t][2] * inv,
                           oacc[s][t][3] * inv);
                  if (quad == 0) lse[(size_t)h * g.N + qn[s]] = (m_run[s] + log2f(l_run[s])) * LN2;
                }
                fend[s] = -1;
              }
            }
          }
        }
        lds_barrier();
      });
    }
  }
}

// bf16 rows of 64 or 128, windows whose key tile spans at most 3 x 3 blocks,
// 3 <= kt <= 16 (a slot's next Q rows load while its current tile reads its last
// frames; a pass lists at most QS_TS + kt - 1 frames), and frames of under 4 GiB
// per tensor (32-bit load offsets inside a frame).
bool fwd_qs_eligible(const Geom& g, int dtype, int D) {
  return dtype == 1 && (D == 64 || D == 128) && qs_geometry(g) &&
         (unsigned long long)g.Hp * g.Wp * g.H * D * 2 < (1ull << 32);
}

template <int D, int NBY, int NBX>
static hipError_t fwd_qs_impl(const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s) {
  const long long total = (long long)qs_items(g) * g.nh;
  k_forward_qs<D, NBY, NBX><<<(unsigned)total, 64 * (FWD_NW + FWD_LW), 0, s>>>(
      (const u16*)a.q, (const u16*)a.k, (const u16*)a.v, (u16*)a.out, a.lse_out, g, p, a.scale * LOG2E);
  return hipGetLastError();
}

template <int D>
static hipError_t fwd_qs_dispatch(const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s) {
  const int nby = (4 + g.ky - 1 + 3) / 4 <= 2 ? 2 : 3, nbx = (4 + g.kx - 1 + 3) / 4 <= 2 ? 2 : 3;
  if (nby == 2) return nbx == 2 ? fwd_qs_impl<D, 2, 2>(a, g, p, s) : fwd_qs_impl<D, 2, 3>(a, g, p, s);
  return nbx == 2 ? fwd_qs_impl<D, 3, 2>(a, g, p, s) : fwd_qs_impl<D, 3, 3>(a, g, p, s);
}

hipError_t launch_forward_qs(int D, const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s) {
  return D == 64 ? fwd_qs_dispatch<64>(a, g, p, s) : fwd_qs_dispatch<128>(a, g, p, s);
}

}  // namespace dsa3d
