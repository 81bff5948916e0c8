// Key-centric dK / dV for 3D Deformable Slide Attention (MegaSlide-DiT, section
// "3D Deformable Slide Attention": the gradient of the windowed softmax attention,
// dV = P^T dO and dK = scale * dS^T Q with dS = P * (dP - rowsum(dO * O))).
//
// A workgroup owns one 4 x 4 key block column (kby, kbx) of one head and a run
// of frames, and holds the dK / dV of its keys in registers: wave pair s owns the
// frames t = s (mod kt), so while the queries of start slice tau stream past, the
// kt pairs hold exactly the kt frames tau .. tau+kt-1 those queries read.  A
// frame's sums are complete once slice t has gone by; its owner writes them and
// moves on to frame t + kt.  Every key gets its sums from one workgroup, in a
// fixed order: no atomics, and the result does not depend on timing.
//
// The queries of a slice that can reach the key block (start cells in the blob box
// of the column) are packed into items of KV_Q = 32 by a prep pass.  Items and,
// once per slice, the K / V rows of the frame that enters, stream through an LDS
// ring with direct global->LDS loads, PD entries ahead of the MFMAs, issued by
// loader waves of their own.
//
// Per item and wave (2 row tiles of 16 queries x the 16 keys of its frame), bf16
// MFMA 16x16x32:
//   S = Q K^T, dP = dO V^T          (per row tile, K / V fragments held in registers)
//   P = exp(S scale - lse) on the query's window, dS = P (dP - Delta)
//   dV^T += dO^T P, dK^T += Q^T dS  (32-query contraction, dO^T / Q^T by transposed
//                                    LDS reads, P / dS straight from the S layout)
#include "internal.hpp"
#include "tube.hpp"

namespace dsa3d {

typedef short shortx4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8_t;

// Blob rows (or columns) of start cells whose windows reach key block kb along an
// axis with window k, lattice length L: cells [4 kb - k + 1, 4 kb + 3] clipped.
__device__ __forceinline__ void blob_span(int kb, int k, int L, int& b0, int& b1) {
  const int lo = max(4 * kb - k + 1, 0), hi = min(4 * kb + 3, L - 1);
  b0 = lo >> 2;
  b1 = hi >> 2;
}

// ---- item lists -------------------------------------------------------------

// Items (KV_Q queries) per (head block, key block column, slice): into
// off[(hb * nkb + kb) * Lt + tau] (one head block unless the offsets are per head).
__device__ __forceinline__ void kvitem_count(const Geom& g, const int* __restrict__ cell_ptr, int* __restrict__ off,
                                             long long i) {
  const int nkbx = (g.Wp + 3) / 4, nkb = ((g.Hp + 3) / 4) * nkbx;
  if (i >= (long long)nkb * g.Lt * g.ph) return;
  const int hb = (int)(i / ((long long)nkb * g.Lt));
  const long long il = i - (long long)hb * nkb * g.Lt;
  const int kb = (int)(il / g.Lt), tau = (int)(il - (long long)kb * g.Lt);
  cell_ptr += (size_t)hb * g.keyspace;  // the head block's cells (their positions are global)
  const int kby = kb / nkbx, kbx = kb - kby * nkbx;
  int by0, by1, bx0, bx1;
  blob_span(kby, g.ky, g.Ly, by0, by1);
  blob_span(kbx, g.kx, g.Lx, bx0, bx1);
  int cnt = 0;
  for (int by = by0; by <= by1; ++by) {
    const int b0 = (tau * g.nby + by) * g.nbx + bx0, b1 = (tau * g.nby + by) * g.nbx + bx1;
    cnt += cell_ptr[(b1 + 1) * BLOB_CELLS] - cell_ptr[b0 * BLOB_CELLS];
  }
  off[i] = (cnt + KV_Q - 1) / KV_Q;
}

// Bit 4 i + j set: key (4 kby + i, 4 kbx + j) of the block lies in the window of
// the query whose window starts at (sy, sx).
__device__ __forceinline__ int block_mask(const Geom& g, int kby, int kbx, int sy, int sx) {
  int rows = 0, cols = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rows |= (unsigned)(4 * kby + i - sy) < (unsigned)g.ky ? 1 << i : 0;
    cols |= (unsigned)(4 * kbx + i - sx) < (unsigned)g.kx ? 1 << i : 0;
  }
  int m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) m |= (rows >> i & 1) ? cols << (4 * i) : 0;
  return m;
}

// One launch for two independent passes: blocks below cblocks count the items
// (kvitem_count), the others copy the (sy, sx) window starts of the bucketed
// queries in bucket order (nq of them), so that the item fill below reads them
// contiguously rather than gathering each query's start once per item that lists
// it (about nine times).
__global__ __launch_bounds__(256) void k_kvitem_count_starts(Geom g, const int* __restrict__ cell_ptr,
                                                             int* __restrict__ off, unsigned cblocks,
                                                             const int* __restrict__ perm,
                                                             const int4* __restrict__ starts, long long nq,
                                                             int2* __restrict__ sst) {
  if (blockIdx.x < cblocks) {
    kvitem_count(g, cell_ptr, off, (long long)blockIdx.x * 256 + threadIdx.x);
    return;
  }
  const long long i = (long long)(blockIdx.x - cblocks) * 256 + threadIdx.x;
  if (i >= nq) return;
  const int4 st = starts[perm[i]];
  sst[i] = make_int2(st.y, st.z);
}

// One wave per (key block column, slice): the queries of the blob box in sort
// order, then padding (query 0, no key of the block in its window) to whole items.
// Each query comes with the mask of the block's keys its window holds, so the
// dK / dV kernel tests a key with one bit extract instead of two range tests.
__global__ __launch_bounds__(256) void k_kvitem_fill(Geom g, const int* __restrict__ cell_ptr,
                                                     const int* __restrict__ perm, const int2* __restrict__ sst,
                                                     const int* __restrict__ off, int* __restrict__ ids,
                                                     int* __restrict__ kmask) {
  const int nkbx = (g.Wp + 3) / 4, nkb = ((g.Hp + 3) / 4) * nkbx;
  const long long i = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= (long long)nkb * g.Lt * g.ph) return;
  const int hb = (int)(i / ((long long)nkb * g.Lt));
  const long long il = i - (long long)hb * nkb * g.Lt;
  const int kb = (int)(il / g.Lt), tau = (int)(il - (long long)kb * g.Lt);
  cell_ptr += (size_t)hb * g.keyspace;
  const int tok0 = hb * g.N;  // sorted queries are numbered across head blocks
  const int kby = kb / nkbx, kbx = kb - kby * nkbx;
  int by0, by1, bx0, bx1;
  blob_span(kby, g.ky, g.Ly, by0, by1);
  blob_span(kbx, g.kx, g.Lx, bx0, bx1);
  const size_t base = (size_t)off[i] * KV_Q;
  const int total = (off[i + 1] - off[i]) * KV_Q;
  // The ranges of the blob rows first, their loads all in flight together, then one
  // pass of the lanes over the rows' queries in order: two dependent gathers per
  // wave instead of two per row.  A window up to 9 wide reaches at most three blob
  // rows (cells 4 kb - k + 1 .. 4 kb + 3); rows beyond that take the loop after.
  constexpr int MR = 3;
  int s0[MR], cnt[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    s0[r] = cnt[r] = 0;
    if (by0 + r <= by1) {
      const int row = tau * g.nby + by0 + r;
      s0[r] = cell_ptr[(row * g.nbx + bx0) * BLOB_CELLS];
      cnt[r] = cell_ptr[(row * g.nbx + bx1 + 1) * BLOB_CELLS] - s0[r];
    }
  }
  const int c01 = cnt[0] + cnt[1];
  int pos = c01 + cnt[2];
  for (int j = lane; j < pos; j += 64) {
    const int src = j < cnt[0] ? s0[0] + j : j < c01 ? s0[1] + (j - cnt[0]) : s0[2] + (j - c01);
    const int2 st = sst[src];
    ids[base + j] = perm[src] - tok0;
    kmask[base + j] = block_mask(g, kby, kbx, st.x, st.y);
  }
  for (int by = by0 + MR; by <= by1; ++by) {
    const int b0 = (tau * g.nby + by) * g.nbx + bx0, b1 = (tau * g.nby + by) * g.nbx + bx1;
    const int sr = cell_ptr[b0 * BLOB_CELLS], n = cell_ptr[(b1 + 1) * BLOB_CELLS] - sr;
    for (int j = lane; j < n; j += 64) {
      const int2 st = sst[sr + j];
      ids[base + pos + j] = perm[sr + j] - tok0;
      kmask[base + pos + j] = block_mask(g, kby, kbx, st.x, st.y);
    }
    pos += n;
  }
  for (int j = pos + lane; j < total; j += 64) {
    ids[base + j] = 0;
    kmask[base + j] = 0;
  }
}

// ---- the dK / dV kernel -----------------------------------------------------

template <int D, int KT>
struct DkdvCfg {
  static constexpr int NPH = D / 64;                 // 128-byte column phases of a bf16 row
  static constexpr int TILE = KV_Q * 128;            // one phase of an item's KV_Q rows
  static constexpr int META = 2 * NPH * TILE;        // item: key mask, lse, delta (4 B each) per query
  static constexpr int MASK = META, LSE = META + 4 * KV_Q, DELTA = META + 8 * KV_Q;
  static constexpr int SINK = META + 12 * KV_Q;      // 16 bytes nobody reads: target of the padding loads
  static constexpr int ENTRY = SINK + 16;
  static constexpr int NL = 2 * NPH * (TILE / 1024) + 3;  // direct loads per entry
  static constexpr int NBUF = D == 128 ? 7 : 8;   // ring entries (LDS: ring and P / dS)
  static constexpr int PD = NBUF - 2;                // entries in flight (the previous one stays readable)
  static constexpr int NIDS = PD + 2;                // token ring (loaded 2 PD + 1 entries ahead)
  static constexpr int NC = D / 32, NT = D / 16;
};

struct KvItems {
  const int* off;   // [nkb * Lt + 1]: items of (kb, tau) are off[kb Lt + tau] .. off[kb Lt + tau + 1]
  const int* ids;   // [items * KV_Q] query tokens
  const int* mask;  // [items * KV_Q] mask of the block's keys in the query's window
};

// Position in the entry stream of a workgroup: slice tau, entry j of the slice
// (j < 0: the K / V rows of frame tau + kt + j; j >= 0: item j of the slice).
struct Cursor {
  int tau, j, n, base;  // n items in the slice, the first is item `base`
};

// Frames per workgroup: at most DKDV_TS_MAX.  A long run along time keeps the
// columns that share queries in step with each other (L2 reuse) and spends few
// steps on the kt - 1 slices a chunk shares with the one before it.
constexpr int DKDV_TS_MAX = 256;
constexpr int DKDV_LW = 2;   // loader waves per workgroup

template <int D, int KT, int FPG>
__global__ __launch_bounds__(128 * ((KT + FPG - 1) / FPG) + 64 * DKDV_LW) void k_dkdv_tube(const u16* __restrict__ q, const u16* __restrict__ k,
                                                       const u16* __restrict__ v, const u16* __restrict__ dout,
                                                       const float* __restrict__ lse,
                                                       const float* __restrict__ delta, u16* __restrict__ dk,
                                                       u16* __restrict__ dv, Geom g, KvItems it, int ts,
                                                       float sl2, float scale) {
  using C = DkdvCfg<D, KT>;
  constexpr int kt = KT;
  // Frame slots s = 0 .. kt-1 (slot s holds the frames t = s (mod kt)) in groups of
  // FPG: wave pair p (waves 2 p, 2 p + 1) owns slots p FPG .. p FPG + FPG - 1 (the
  // last pair may own fewer), with K / V of their frames and the dK / dV columns
  // [hf D / 2, (hf + 1) D / 2) of their keys, hf = wave & 1.  For each item, wave hf
  // of a pair forms S, dP, P and dS of row tile hf for each of its slots (one read
  // of the Q / dO rows for all of them) and leaves P and dS in LDS; in the next step
  // both apply dV^T += dO^T P and dK^T += Q^T dS over all 32 queries to their half
  // of every slot (one transposed read of dO / Q for all of them).  The ring
  // therefore keeps the previous entry (prefetch distance NBUF - 2).
  // DKDV_LW more waves issue every global->LDS load (and wait for them): the
  // compute waves never wait on an LDS token read or on memory, only at the
  // barrier that closes each step.
  constexpr int NG = (KT + FPG - 1) / FPG;  // wave pairs
  constexpr int NWC = 2 * NG, NW = NWC + DKDV_LW;
  constexpr int NTH = C::NT / 2;  // d tiles per half
  __shared__ __attribute__((aligned(1024))) char ring[C::NBUF][C::ENTRY];
  __shared__ __attribute__((aligned(16))) char xch[2][KT][2][64 * 16];  // [step parity][frame slot][P, dS]

  const int nkbx = (g.Wp + 3) / 4, nkb = ((g.Hp + 3) / 4) * nkbx;
  const int nchunk = (g.F + ts - 1) / ts;
  int L = xcd_remap(blockIdx.x, nkb * nchunk * g.nh);
  const int hl = L / (nkb * nchunk);
  L -= hl * nkb * nchunk;
  const int h = g.h0 + hl;
  const int chunk = L / nkb, kb = L - chunk * nkb;
  const int kby = kb / nkbx, kbx = kb - kby * nkbx;
  const int t0 = chunk * ts, t1 = min(t0 + ts, g.F);  // frames written here
  const int tau_lo = max(t0 - kt + 1, 0), tau_hi = min(t1 - 1, g.Lt - 1);

  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, quad = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool loader = wave >= NWC;
  const int grp = wave >> 1, hf = wave & 1;  // (compute waves)
  const int lw = wave - NWC;                   // (loader waves)
  // every loader wave issues MY_LOADS loads per entry (the count is padded with
  // one-lane loads), so the steady-state wait is a single immediate
  constexpr int MY_LOADS = (C::NL + DKDV_LW - 1) / DKDV_LW;
  // Nothing in the loop below reads memory through the scalar unit: a scalar load
  // in flight makes every LDS wait a full lgkmcnt(0) wait, which would put its
  // latency in front of the MFMAs.  The slice boundaries of this workgroup go to
  // LDS once; item tokens arrive by direct loads into a small ring, 2 PD + 1
  // entries ahead of use.
  __shared__ int s_off[DKDV_TS_MAX + 8 + 1];
  __shared__ int s_ids[C::NIDS][KV_Q];
  const int hb = g.ph > 1 ? hl : 0;  // the head's item lists (per-head offsets)
  for (int i = tid; i <= tau_hi - tau_lo + 1; i += 64 * NW)
    s_off[i] = it.off[((size_t)hb * nkb + kb) * g.Lt + tau_lo + i];
  // The in-loop apply runs its MFMAs with P = dS = 0 when it has nothing to add,
  // so every ring byte it may read must hold a finite value from the start.
  for (int i = tid; i < C::NBUF * C::ENTRY / 16; i += 64 * NW)
    reinterpret_cast<uint4*>(&ring[0][0])[i] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();

  // this lane's key (key r16 of the block)
  const int key_y = 4 * kby + (r16 >> 2), key_x = 4 * kbx + (r16 & 3);

  auto slice_off = [&](int tau) { return __builtin_amdgcn_readfirstlane(s_off[tau - tau_lo]); };
  auto start_cursor = [&]() {
    Cursor c;
    c.tau = tau_lo;
    c.j = -kt;
    c.base = slice_off(tau_lo);
    c.n = slice_off(tau_lo + 1) - c.base;
    return c;
  };
  auto advance = [&](Cursor& c) {
    if (++c.j == c.n) {
      ++c.tau;
      if (c.tau <= tau_hi) {
        c.base += c.n;
        c.n = slice_off(c.tau + 1) - c.base;
      }
      c.j = -1;
    }
  };

  // tile offsets: Q / dO (item) or K / V (frame) of phase ph
  auto tile = [&](char* e, int tensor, int ph) { return e + (tensor * C::NPH + ph) * C::TILE; };

  // Three cursors over the same entry stream: token loads (pc, 2 PD + 1 ahead),
  // row loads (ic, PD ahead) and the MFMAs (cc).  Every wave runs PD + (entries)
  // steps, each closed by one barrier.
  Cursor cc = start_cursor();
  if (loader) {
    // Loader wave LWI issues loads LWI, LWI + DKDV_LW, ... of every entry; with the
    // index a compile-time constant each load is a handful of instructions.
    static_for<0, DKDV_LW>([&](auto LWC) {
      constexpr int LWI = decltype(LWC)::value;
      if (lw != LWI) return;
      // column of the 16-byte chunk this lane loads: rows 8 p + (lane >> 3) are
      // stored swizzled (chunk (lane & 7) ^ (row & 7)), the same for every part p
      const int lane_el = ((lane & 7) ^ (lane >> 3)) * 8;
      constexpr int PARTS = C::TILE / 1024;  // 1 KB parts of a tile: 8 rows of 128 B
      constexpr int NR = 2 * C::NPH * PARTS;  // row loads of an item
      static_assert(PARTS % DKDV_LW == 0, "loader waves split the parts evenly");
      auto issue = [&](const Cursor& c, int x, char* e) {
        if (c.j < 0) {
          // a frame: its 16 key rows fill the first 2 KB of each phase tile
          const int f = c.tau + kt + c.j;
          static_for<0, MY_LOADS>([&](auto JJ) {
            constexpr int j = LWI + DKDV_LW * decltype(JJ)::value;
            if constexpr (j < 4 * C::NPH) {
              constexpr int ti = j >> 1, hh = j & 1, tensor = ti / C::NPH, ph = ti % C::NPH;
              const int row = 8 * hh + (lane >> 3);
              const int y = 4 * kby + (row >> 2), x = 4 * kbx + (row & 3);
              const int tok = (y < g.Hp && x < g.Wp) ? (f * g.Hp + y) * g.Wp + x : 0;
              const u16* src = (tensor ? v : k) + ((size_t)tok * g.H + h) * D + ph * 64 + lane_el;
              dma16(src, e + ti * C::TILE + hh * 1024);
            } else {
              if (lane == 0) dma4(lse, e + C::SINK);  // keeps the per-entry load count uniform
            }
          });
        } else {
          const int item = c.base + c.j;
          const int* ids = s_ids[x % C::NIDS];
          // the tokens first: every direct load below clobbers memory for the
          // compiler, which would otherwise read (and wait for) each token again
          constexpr int NQ = PARTS / DKDV_LW;  // parts LWI + DKDV_LW qq
          size_t rowoff[NQ];
#pragma unroll
          for (int qq = 0; qq < NQ; ++qq)
            rowoff[qq] = ((size_t)ids[8 * (LWI + DKDV_LW * qq) + (lane >> 3)] * g.H + h) * D + lane_el;
          const size_t meta_off = (size_t)h * g.N + ids[lane & (KV_Q - 1)];
          static_for<0, MY_LOADS>([&](auto JJ) {
            constexpr int jj = decltype(JJ)::value, j = LWI + DKDV_LW * jj;
            if constexpr (j < NR) {
              constexpr int ti = j / PARTS, part = j % PARTS, tensor = ti / C::NPH, ph = ti % C::NPH;
              dma16((tensor ? dout : q) + rowoff[jj % NQ] + ph * 64, e + ti * C::TILE + part * 1024);
            } else if constexpr (j == NR) {
              if (lane < KV_Q / 4) dma16(it.mask + (size_t)item * KV_Q + 4 * lane, e + C::MASK);
            } else if constexpr (j < C::NL) {
              if (lane < KV_Q)
                dma4((j == NR + 1 ? lse : delta) + meta_off, e + (j == NR + 1 ? C::LSE : C::DELTA));
            } else {
              if (lane == 0) dma4(lse, e + C::SINK);  // padding of the load count
            }
          });
        }
      };
      // tokens of entry x (items only), by the last loader wave
      auto issue_ids = [&](const Cursor& c, int x) {
        if constexpr (LWI == DKDV_LW - 1)
          if (c.j >= 0 && lane < KV_Q) dma4(it.ids + (size_t)(c.base + c.j) * KV_Q + lane, s_ids[x % C::NIDS]);
      };

      Cursor pc = start_cursor(), ic = start_cursor();
      int npc = 0;
      for (; npc <= C::PD && pc.tau <= tau_hi; ++npc, advance(pc)) issue_ids(pc, npc);
      wait_vmcnt(0);
      __syncthreads();
      int issued = 0;
      auto issue_next = [&]() {
        if (ic.tau <= tau_hi) {
          issue(ic, issued, ring[issued % C::NBUF]);
          ++issued;
          advance(ic);
        }
        if (pc.tau <= tau_hi) {
          issue_ids(pc, npc);
          ++npc;
          advance(pc);
        }
      };
      // fill the pipeline: entries 0 .. PD - 1 (token loads only add to the count
      // of loads issued later, so the waits are exact or stricter)
      for (int st = -C::PD; st < 0; ++st) {
        issue_next();
        wait_vmcnt(MY_LOADS * max(issued - st - 2, 0));
        lds_barrier();
      }
      for (int st = 0; cc.tau <= tau_hi; ++st) {
        issue_next();
        // entry st + 1 must have landed; entries st + 2 .. issued - 1 may stay in flight
        if (issued - st - 2 == C::PD - 1)
          wait_vmcnt_c<MY_LOADS * (C::PD - 1)>();
        else
          wait_vmcnt(MY_LOADS * max(issued - st - 2, 0));
        lds_barrier();
        advance(cc);
      }
    });
    return;
  }

  __syncthreads();
  for (int st = -C::PD; st < 0; ++st) lds_barrier();

  // The compute loop, for a pair that owns NSG slots (a compile-time count).
  auto run = [&](auto NSGC) {
    constexpr int NSG = decltype(NSGC)::value;
    const int s0 = grp * FPG;  // first slot of this pair
    f32x4_t dka[NSG][NTH], dva[NSG][NTH];
#pragma unroll
    for (int i = 0; i < NSG; ++i)
#pragma unroll
      for (int t = 0; t < NTH; ++t) {
        dka[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        dva[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    int cur_f[NSG];
#pragma unroll
    for (int i = 0; i < NSG; ++i) cur_f[i] = -1;
    Frag<u16> kf[NSG][C::NC], vf[NSG][C::NC];  // K / V of each slot's frame (B fragments of S and dP)

    auto finalize = [&](int i) {
      const int f = cur_f[i];
      if (f >= t0 && f < t1 && key_y < g.Hp && key_x < g.Wp) {
        const size_t row = ((size_t)((f * g.Hp + key_y) * g.Wp + key_x) * g.H + h) * D + hf * (D / 2);
#pragma unroll
        for (int t = 0; t < NTH; ++t) {
          store4(dk + row + 16 * t + 4 * quad, dka[i][t][0] * scale, dka[i][t][1] * scale, dka[i][t][2] * scale,
                 dka[i][t][3] * scale);
          store4(dv + row + 16 * t + 4 * quad, dva[i][t][0], dva[i][t][1], dva[i][t][2], dva[i][t][3]);
        }
      }
    };

    // dV^T += dO^T P and dK^T += Q^T dS for this wave's half of every slot, with P /
    // dS of the item in ring entry e left by the pair's producers in xch[par].  (A
    // slot whose frame is outside [t0, t1) gets sums nobody writes.)
    auto apply = [&](char* e, int par) {
      Frag<u16> pb[NSG], db[NSG];
#pragma unroll
      for (int i = 0; i < NSG; ++i) {
        load_frag(pb[i], (const u16*)(xch[par][s0 + i][0] + lane * 16));
        load_frag(db[i], (const u16*)(xch[par][s0 + i][1] + lane * 16));
      }
      // A slots j < 4: rows 4 quad + j of row tile 0; j >= 4: the same rows of row tile 1
      const int trow = 4 * quad + (r16 >> 2);
#pragma unroll
      for (int tt = 0; tt < NTH; ++tt) {
        const int t = hf * NTH + tt;
        const int off = sw(trow, ((t & 3) * 16 + 4 * (r16 & 3)) * 2);
        Frag<u16> ao, aq;
        {
          const char* base = tile(e, 1, t >> 2) + off;
          const shortx4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t*)base);
          const shortx4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t*)(base + 16 * 128));
          const shortx4v both[2] = {lo, hi};
          __builtin_memcpy(&ao.v, both, 16);
        }
        {
          const char* base = tile(e, 0, t >> 2) + off;
          const shortx4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t*)base);
          const shortx4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t*)(base + 16 * 128));
          const shortx4v both[2] = {lo, hi};
          __builtin_memcpy(&aq.v, both, 16);
        }
#pragma unroll
        for (int i = 0; i < NSG; ++i) {
          dva[i][tt] = mma(ao, pb[i], dva[i][tt]);
          dka[i][tt] = mma(aq, db[i], dka[i][tt]);
        }
        __asm__ __volatile__("" ::: "memory");
      }
    };

    // S = Q K^T, dP = dO V^T of row tile hf against each slot's frame, then P and dS
    // of its queries 16 hf + 4 quad + i, which are slots 4 hf + i of the pair's B
    // fragments in xch[par] (8 of their 16 bytes per lane)
    auto produce = [&](char* e, int par) {
      const int q0 = 16 * hf + 4 * quad;
      // the queries' key masks, lse and Delta first: they do not depend on the products
      const float4 de = *reinterpret_cast<const float4*>(e + C::DELTA + q0 * 4);
      const int4 km = *reinterpret_cast<const int4*>(e + C::MASK + q0 * 4);
      const float4 ls = *reinterpret_cast<const float4*>(e + C::LSE + q0 * 4);
      // dP - Delta: the products accumulate onto -Delta of the lane's four queries
      const f32x4_t ndq = f32x4_t{-de.x, -de.y, -de.z, -de.w};
      f32x4_t sc[NSG], dp[NSG];
#pragma unroll
      for (int i = 0; i < NSG; ++i) {
        sc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        dp[i] = ndq;
      }
      // every Q and dO fragment of the row tile read together (two base addresses,
      // fixed before the first read; tensor and phase offsets in the instruction),
      // then the MFMAs
      lds_char* fb[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) fb[c] = (lds_char*)(e + sw(16 * hf + r16, c * 64 + quad * 16));
      __asm__ __volatile__("" : "+v"(fb[0]), "+v"(fb[1]));
      Frag<u16> aq[C::NC], ao[C::NC];
#pragma unroll
      for (int c = 0; c < C::NC; ++c) {
        aq[c].v = *(const lds_bf16x8_t*)(fb[c & 1] + (0 * C::NPH + (c >> 1)) * C::TILE);
        ao[c].v = *(const lds_bf16x8_t*)(fb[c & 1] + (1 * C::NPH + (c >> 1)) * C::TILE);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < C::NC; ++c) {
#pragma unroll
        for (int i = 0; i < NSG; ++i) sc[i] = mma(aq[c], kf[i][c], sc[i]);
#pragma unroll
        for (int i = 0; i < NSG; ++i) dp[i] = mma(ao[c], vf[i][c], dp[i]);
      }
      const int mk[4] = {km.x, km.y, km.z, km.w};
      const float lq[4] = {ls.x, ls.y, ls.z, ls.w};
      // per query: -lse in log2 units, and all ones if the lane's key is in its
      // window, else zero: P outside the window is +0 whatever exp2 gave (finite
      // scores, so no NaN can reach the mask)
      float nl[4];
      int keep[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        nl[j] = -lq[j] * LOG2E;
        keep[j] = __builtin_amdgcn_sbfe(mk[j], r16, 1);
      }
#pragma unroll
      for (int i = 0; i < NSG; ++i) {
        f32x4_t pe, ds;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pe[j] = __uint_as_float(__float_as_uint(__builtin_amdgcn_exp2f(sc[i][j] * sl2 + nl[j])) & keep[j]);
          ds[j] = pe[j] * dp[i][j];
        }
        // bf16 (round to nearest even), two values per conversion instruction
        *reinterpret_cast<bf16x4_t*>(xch[par][s0 + i][0] + lane * 16 + hf * 8) = __builtin_convertvector(pe, bf16x4_t);
        *reinterpret_cast<bf16x4_t*>(xch[par][s0 + i][1] + lane * 16 + hf * 8) = __builtin_convertvector(ds, bf16x4_t);
      }
    };

    // Slice by slice: the frames that enter (kt for the first slice, then one), then
    // the items.  The item loop changes only the accumulators, by MFMA, and the frame
    // steps sit outside it, which keeps the sums and the K / V fragments in fixed
    // registers while items stream past.
    int st = 0;     // entry
    int nprev = 0;  // items of the previous slice (its last one is still to apply)
    for (int tau = tau_lo; tau <= tau_hi; ++tau) {
      const int n = slice_off(tau + 1) - slice_off(tau);
      const int nf = tau == tau_lo ? kt : 1;
      for (int jf = 0; jf < nf; ++jf, ++st) {
        // ---- the previous slice's last item, then a frame enters: the pair that
        // owns its slot writes the frame the slot leaves and takes K / V
        if (jf == 0 && nprev > 0) apply(ring[(st - 1) % C::NBUF], (st - 1) & 1);
        const int f = tau + kt - nf + jf;
        const int sf = f % kt;
        static_for<0, NSG>([&](auto IC) {
          constexpr int i = decltype(IC)::value;
          if (sf == s0 + i) {
            if (cur_f[i] >= 0) {
              finalize(i);
#pragma unroll
              for (int t = 0; t < NTH; ++t) {
                dka[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                dva[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
              }
            }
            // the frame's K and V rows (first 2 KB of each phase tile of the entry)
            // as MFMA B fragments: key r16, head-dim slots 32 c + 8 quad .. + 7
            char* e = ring[st % C::NBUF];
#pragma unroll
            for (int c = 0; c < C::NC; ++c) {
              const int koff = sw(r16, (c & 1) * 64 + quad * 16);
              load_frag(kf[i][c], (const u16*)(tile(e, 0, c >> 1) + koff));
              load_frag(vf[i][c], (const u16*)(tile(e, 1, c >> 1) + koff));
            }
            cur_f[i] = f;
          }
        });
        lds_barrier();
      }
      // ---- the items: each wave of a pair forms P and dS of one row tile; in the next
      // step both apply them
      if (n > 0) {
        produce(ring[st % C::NBUF], st & 1);
        lds_barrier();
        ++st;
        for (int j = 1; j < n; ++j, ++st) {
          apply(ring[(st + C::NBUF - 1) % C::NBUF], (st - 1) & 1);
          produce(ring[st % C::NBUF], st & 1);
          lds_barrier();
        }
      }
      nprev = n;
    }
    // the last item (its ring slot is not reused any more)
    if (nprev > 0) apply(ring[(st - 1) % C::NBUF], (st - 1) & 1);
#pragma unroll
    for (int i = 0; i < NSG; ++i) finalize(i);
  };
  constexpr int LAST = KT - (NG - 1) * FPG;  // slots of the last pair
  if (LAST != FPG && grp == NG - 1)
    run(std::integral_constant<int, LAST>{});
  else
    run(std::integral_constant<int, FPG>{});
}

bool dkdv_tube_eligible(const Geom& g, int dtype, int D) {
  (void)D;
  return dtype == 1 && kv_items_geometry(g);
}

hipError_t launch_kv_items(const Geom& g, const Prep& p, hipStream_t s) {
  const long long n = (long long)kv_item_columns(g) * g.Lt * g.ph, nq = (long long)g.N * g.ph;
  const unsigned cblocks = (unsigned)((n + 255) / 256);
  k_kvitem_count_starts<<<cblocks + (unsigned)((nq + 255) / 256), 256, 0, s>>>(g, p.cell_ptr, p.kv_off, cblocks,
                                                                                p.perm, p.starts, nq, p.sorted_st);
  if (launch_scan_excl(reinterpret_cast<uint32_t*>(p.kv_off), (int)(n + 1), s, p.scan_part) != hipSuccess)
    return hipGetLastError();
  k_kvitem_fill<<<(unsigned)((n + 3) / 4), 256, 0, s>>>(g, p.cell_ptr, p.perm, p.sorted_st, p.kv_off, p.kv_ids,
                                                        p.kv_mask);
  return hipGetLastError();
}

// Frame slots per wave pair: two where the registers allow it (kt = 3, 5: the
// workgroup has 2 ceil(kt / 2) + 2 waves, at most two per SIMD, so a wave may hold
// the K / V fragments and dK / dV sums of two frames), one for kt = 7 (sixteen
// waves, four per SIMD, 128 registers a wave) and kt = 1.
#ifndef DSA3D_DKDV_FPG3
#define DSA3D_DKDV_FPG3 2
#endif
#ifndef DSA3D_DKDV_FPG5
#define DSA3D_DKDV_FPG5 2
#endif
template <int KT>
constexpr int dkdv_fpg() {
  return KT == 3 ? DSA3D_DKDV_FPG3 : KT == 5 ? DSA3D_DKDV_FPG5 : 1;
}

template <int D, int KT>
static hipError_t dkdv_impl(const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s) {
  constexpr int FPG = dkdv_fpg<KT>();
  constexpr int NG = (KT + FPG - 1) / FPG;
  const int nkb = kv_item_columns(g);
  // the longest chunk that still leaves at least 512 workgroups (two per compute unit)
  int ts = min(g.F, DKDV_TS_MAX);
  while (ts > 8 && (long long)nkb * g.nh * ((g.F + ts - 1) / ts) < 512) ts = (ts + 1) / 2;
  const int nchunk = (g.F + ts - 1) / ts;
  const long long total = (long long)nkb * nchunk * g.nh;
  KvItems it{p.kv_off, p.kv_ids, p.kv_mask};
  k_dkdv_tube<D, KT, FPG><<<(unsigned)total, 128 * NG + 64 * DKDV_LW, 0, s>>>(
      (const u16*)a.q, (const u16*)a.k, (const u16*)a.v, (const u16*)a.dout, a.lse, p.delta, (u16*)a.dk, (u16*)a.dv, g,
      it, ts, a.scale * LOG2E, a.scale);
  return hipGetLastError();
}

hipError_t launch_dkdv_tube(int D, const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s) {
  switch (g.kt) {
#define DSA3D_DKDV_KT(n) \
  case n:                \
    return D == 64 ? dkdv_impl<64, n>(a, g, p, s) : dkdv_impl<128, n>(a, g, p, s);
    DSA3D_DKDV_KT(1) DSA3D_DKDV_KT(3) DSA3D_DKDV_KT(5) DSA3D_DKDV_KT(7)
#undef DSA3D_DKDV_KT
    default:
      return hipErrorInvalidValue;  // kv_items_geometry() admits odd kt <= 8 only
  }
}

}  // namespace dsa3d
