// Query-side work lists shared by the frame-sweeping forward and dQ kernels
// (built once per call: one set used by every head when the offsets are shared, or
// one set per head, head-major, for per-head offsets).  Work item w of the lists is
// item w mod qs_items of head block w / qs_items.
//
// Row tiles: a work item is one start blob column (by, bx) and QS_TS consecutive
// slices (1 x 4 x 4 start cells of the lattice of the 3D Deformable Slide
// Attention section).  Each slice's blob contributes its full groups of 16
// queries as tiles of their own; the leftover group of a slice (fewer than 16
// queries) joins the open leftover tile of an earlier slice of the item when the
// queries fit in 16 and that tile's first slice is less than QS_SPAN slices back,
// else it opens a new one.  A tile of slices tau0 .. tlast reads the frames
// tau0 .. tlast + kt - 1; each row sees only the kt frames of its own slice
// (tq_dt = its slice - tau0), the kernels mask the others.  Descriptor (QT_INTS
// ints): tau0, tlast, then per part (first index into perm, count, slice - tau0),
// unused parts with count 0.  Tiles are listed in order of tau0.  tq_ids / tq_st
// hold each tile's query tokens and window starts (sy, sx), padded to 16 with
// token 0 and a start no key matches.
//
// Schedules: a work item's row tiles get one of nslots slots for the frames they
// read; greedy, in tile order, a tile takes the slot that has been free the longest
// (a slot is free again once its tile has read its last frame).  Tiles that find
// no free slot at their first frame wait for a further pass over the frames.
// Each pass lists the frames it sweeps (the union of its tiles' frame ranges, in
// order) and its tiles as (tile, tau0, slot, index of frame tau0 in the list).
#include "internal.hpp"

namespace dsa3d {

// Row tiles of work item w (see above): writes their descriptors to out (if not
// null) and returns their count, which is at most the item's group count.  A
// blob's queries are perm[beg .. beg + cnt) (from cell_ptr); its groups are the
// runs of GROUP_Q from beg, the last one possibly short.
__device__ int item_tiles(const Geom& g, const int* __restrict__ cell_ptr, int w, int* out) {
  const int nbc = g.nby * g.nbx, nw = qs_items(g);
  const int hb = w / nw;
  w -= hb * nw;
  cell_ptr += (size_t)hb * g.keyspace;  // the head block's cells (their positions are global)
  const int chunk = w / nbc, bc = w - chunk * nbc;
  const int by = bc / g.nbx, bx = bc - by * g.nbx;
  const int c0 = chunk * QS_TS, ns = min(QS_TS, g.Lt - c0);
  auto put = [&](int t, int tau, int begin, int cnt) {
    int* d = out + (size_t)t * QT_INTS;
    d[0] = tau;
    d[1] = tau;
    d[2] = begin;
    d[3] = cnt;
    d[4] = 0;
    for (int q = 1; q < QS_SPAN; ++q) d[3 + 3 * q] = 0;
  };
  // every slice's bounds first (loads of slices past ns repeat the last one), so
  // that the loads are in flight together rather than one slice at a time
  int cb[QS_TS], ce[QS_TS];
#pragma unroll
  for (int i = 0; i < QS_TS; ++i) {
    const int b = ((c0 + min(i, ns - 1)) * g.nby + by) * g.nbx + bx;
    cb[i] = cell_ptr[b * BLOB_CELLS];
    ce[i] = cell_ptr[(b + 1) * BLOB_CELLS];
  }
  int n = 0, open = -1, acc = 0, s0 = 0, np = 0;
  for (int i = 0; i < ns; ++i) {
    const int tau = c0 + i;
    const int beg = cb[i], cnt = ce[i] - beg;
    const int nfull = cnt / GROUP_Q, rest = cnt - nfull * GROUP_Q;
    for (int k = 0; k < nfull; ++k, ++n)
      if (out) put(n, tau, beg + k * GROUP_Q, GROUP_Q);
    if (rest == 0) continue;
    const int rbeg = beg + nfull * GROUP_Q;
    if (open >= 0 && acc + rest <= GROUP_Q && tau - s0 < QS_SPAN) {
      if (out) {
        int* d = out + (size_t)open * QT_INTS;
        d[1] = tau;
        d[2 + 3 * np] = rbeg;
        d[3 + 3 * np] = rest;
        d[4 + 3 * np] = tau - s0;
      }
      ++np;
      acc += rest;
    } else {
      if (out) put(n, tau, rbeg, rest);
      open = n++;
      s0 = tau;
      acc = rest;
      np = 1;
    }
  }
  return n;
}

// Row tile counts of the work items (blocks from tblock0 on), and, in the blocks
// before, the group counts of the blobs (up to GROUP_Q queries each, goff[nblobs] =
// 0), both for an exclusive scan.
__global__ __launch_bounds__(64) void k_qtile_count(Geom g, const int* __restrict__ cell_ptr, int nw,
                                                    int* __restrict__ qt_off, int tblock0, int nblobs,
                                                    int* __restrict__ goff) {
  if ((int)blockIdx.x < tblock0) {
    const int b = blockIdx.x * 64 + threadIdx.x;
    if (b > nblobs) return;
    const int cnt = b == nblobs ? 0 : cell_ptr[(b + 1) * BLOB_CELLS] - cell_ptr[b * BLOB_CELLS];
    goff[b] = (cnt + GROUP_Q - 1) / GROUP_Q;
    return;
  }
  const int w = (blockIdx.x - tblock0) * 64 + threadIdx.x;
  if (w < nw) qt_off[w] = item_tiles(g, cell_ptr, w, nullptr);
  if (w == nw) qt_off[w] = 0;
}

// Two fills in one launch, both after the scans of the blob group counts (goff) and
// of the row tile counts (qt_off): blocks below gblocks write the groups of 256 blobs
// each (and the group count), the others the row tiles of 256 work items each.
__global__ __launch_bounds__(256) void k_groups_qtiles(Geom g, const int* __restrict__ cell_ptr,
                                                       const int* __restrict__ goff, int nblobs, int2* __restrict__ groups,
                                                       int* __restrict__ ngroups, int gblocks, int nw,
                                                       const int* __restrict__ qt_off, int* __restrict__ qt) {
  if ((int)blockIdx.x < gblocks) {
    const int b = blockIdx.x * 256 + threadIdx.x;
    if (b == 0) *ngroups = goff[nblobs];
    if (b >= nblobs) return;
    const int beg = cell_ptr[b * BLOB_CELLS];
    const int cnt = cell_ptr[(b + 1) * BLOB_CELLS] - beg;
    const int g0 = goff[b], ng = goff[b + 1] - g0;
    for (int i = 0; i < ng; ++i) groups[g0 + i] = make_int2(beg + i * GROUP_Q, min(GROUP_Q, cnt - i * GROUP_Q));
    return;
  }
  const int w = (blockIdx.x - gblocks) * 256 + threadIdx.x;
  if (w < nw) item_tiles(g, cell_ptr, w, qt + (size_t)qt_off[w] * QT_INTS);
}

// Rows of the tiles: 16 lanes per tile, row j from the part that holds it.  The
// sorted queries are numbered across head blocks; a row keeps its token (mod N).
__global__ __launch_bounds__(256) void k_tile_fill(const int* __restrict__ perm, const int4* __restrict__ starts,
                                                   const int* __restrict__ qt, const int* __restrict__ ntiles, int N,
                                                   int* __restrict__ tq_ids, int2* __restrict__ tq_st,
                                                   signed char* __restrict__ tq_dt) {
  const int t = blockIdx.x * 16 + (threadIdx.x >> 4), j = threadIdx.x & 15;
  if (t >= *ntiles) return;
  const int* d = qt + (size_t)t * QT_INTS;
  int id = 0, dt = 0, r = j;
  int2 st = make_int2(-(1 << 29), -(1 << 29));
  for (int q = 0; q < QS_SPAN; ++q) {
    const int cnt = d[3 + 3 * q];
    if (r >= 0 && r < cnt) {
      id = perm[d[2 + 3 * q] + r];
      const int4 s = starts[id];
      st = make_int2(s.y, s.z);
      dt = d[4 + 3 * q];
    }
    r -= cnt;
  }
  tq_ids[(size_t)t * 16 + j] = id % N;
  tq_st[(size_t)t * 16 + j] = st;
  tq_dt[(size_t)t * 16 + j] = (signed char)dt;
}

// Runs the greedy schedule of work item w, whose ntiles tiles (global indices t0 ..,
// in order of first slice) have first / last slices tiles.tau0(i) / tiles.tlast(i),
// and writes it to out; returns its size in ints.  work: 4 QS_MAXT ints of scratch
// (LDS in the kernel), written by all nlanes lanes alike and copied out by lane
// lane of nlanes; tiles.uni(x) marks a value as the same in every lane, so that a
// whole wave runs the pass on the scalar unit.
template <typename Tiles>
__device__ int build_schedule(const Geom& g, int w, int t0, int ntiles, const Tiles& tiles, int* out, int* work,
                              int lane, int nlanes, int nslots) {
  const int nbc = g.nby * g.nbx;
  const int chunk = (w % qs_items(g)) / nbc;
  const int c0 = chunk * QS_TS, ns = min(QS_TS, g.Lt - c0);
  // cur[i] .. lim[i]: the tiles (of the item) whose first slice is c0 + i that are
  // still to be scheduled.  Both arrays are cleared in a loop of their own with a
  // constant bound and written only at indices below ns: a guarded clear folded into
  // a loop that runs to ns became an indexed register write at index ns, one past
  // the array.
  int cur[QS_TS], lim[QS_TS];
  for (int i = 0; i < QS_TS; ++i) cur[i] = lim[i] = 0;
  for (int i = 0, t = 0; i < ns; ++i) {
    cur[i] = t;
    while (t < ntiles && tiles.tau0(t) < c0 + i + 1) ++t;
    lim[i] = t;
  }
  int size = 1, npass = 0;
  for (;;) {
    int free_at[QS_SLOTS_MAX];
    for (int s = 0; s < QS_SLOTS_MAX; ++s) free_at[s] = s < nslots ? -(1 << 29) : (1 << 30);
    int nf = 0, nt = 0, fmax = -1;
    int* hdr = out ? out + size : nullptr;
    int* frames = hdr ? hdr + 2 : nullptr;
    // tiles are written after the frames, whose count is known only at the end,
    // so collect them first into a bounded list: (tile, slice, slot, frame index)
    int* tl4 = work;
    for (int i = 0; i < ns && nt < QS_MAXT; ++i) {
      const int tau = c0 + i;
      while (cur[i] < lim[i] && nt < QS_MAXT) {
        int best = -1;
        for (int s = 0; s < QS_SLOTS_MAX; ++s)
          if (free_at[s] <= tau && (best < 0 || free_at[s] < free_at[best])) best = s;
        if (best < 0) break;
        const int ti = cur[i];
        const int tlast = tiles.tlast(ti);
        const int fi = tau > fmax ? nf : nf - 1 - (fmax - tau);
        for (int f = max(tau, fmax + 1); f < tlast + g.kt; ++f) {
          if (frames) frames[nf] = f;
          ++nf;
        }
        fmax = max(fmax, tlast + g.kt - 1);
        tl4[4 * nt + 0] = t0 + ti;
        tl4[4 * nt + 1] = tau;
        tl4[4 * nt + 2] = best;
        tl4[4 * nt + 3] = fi;
        ++nt;
        free_at[best] = tlast + g.kt;
        ++cur[i];
      }
    }
    if (nt == 0) break;
    if (hdr) {
      hdr[0] = nf;
      hdr[1] = nt;
      int* tl = frames + nf;
      for (int t = lane; t < 4 * nt; t += nlanes) tl[t] = tl4[t];
    }
    size += 2 + nf + 4 * nt;
    ++npass;
  }
  if (out) out[0] = npass;
  return size;
}

// The same schedule for an item of at most 128 tiles, held in registers: tile t's
// first / last slice in lane t mod 64 of ta / tb [t / 64] (read back with readlane),
// the slots' first free frames in lanes 0 .. nslots - 1 of one register (the choice of slot by a
// DPP minimum), the tiles already scheduled in two 64-bit masks, a pass's frames (fewer than 64:
// QS_TS + kt - 1) and tile entries (at most QS_MAXT = 64) collected one per lane
// (lane i keeps the i-th) and stored at the pass's end by one vector store each.  Tiles are
// visited in order; once a tile finds no free slot, the rest of its slice waits for
// the next pass, as above.
static_assert(QS_MAXT <= 64 && QS_TS + 16 - 1 < 64, "one lane per frame and per tile entry");
static_assert(QS_SLOTS_MAX <= 16, "the slots' free frames sit in lanes 0-15 (one row for DPP)");
__device__ int build_schedule_regs(const Geom& g, int t0, int ntiles, int ta0, int tb0, int ta1, int tb1, int* out,
                                   int lane, int nslots) {
  constexpr int NOSLOT = 0x7fffffff;  // above every frame number
  uint64_t done0 = 0, done1 = 0;
  int size = 1, npass = 0;
  for (;;) {
    // slot s's first free frame in lane s (lanes past the slots: NOSLOT)
    int fa = lane < nslots ? -(1 << 29) : NOSLOT;
    int nf = 0, nt = 0, fmax = -1, blocked = -(1 << 30);
    int fr = 0, e0 = 0, e1 = 0, e2 = 0, e3 = 0;
    for (int t = 0; t < ntiles && nt < QS_MAXT; ++t) {
      const bool hi = t >= 64;
      const int bit = t & 63;
      if (((hi ? done1 : done0) >> bit) & 1) continue;
      const int tau = __builtin_amdgcn_readlane(hi ? ta1 : ta0, bit);
      if (tau == blocked) continue;
      // the free slot that has been free the longest (the lowest such slot on a tie):
      // the minimum over lanes 0-15 by DPP (within quads, across the two quads of each
      // half row, then across the two half rows), then the first lane that holds it
      const int cand = fa <= tau ? fa : NOSLOT;
      int m = cand;
      m = min(m, __builtin_amdgcn_update_dpp(NOSLOT, m, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
      m = min(m, __builtin_amdgcn_update_dpp(NOSLOT, m, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
      m = min(m, __builtin_amdgcn_update_dpp(NOSLOT, m, 0x141, 0xF, 0xF, false));  // row_half_mirror
      m = min(m, __builtin_amdgcn_update_dpp(NOSLOT, m, 0x140, 0xF, 0xF, false));  // row_mirror
      const int mn = __builtin_amdgcn_readlane(m, 0);
      if (mn == NOSLOT) {
        blocked = tau;
        continue;
      }
      const int best = __builtin_ctzll(__ballot(lane < nslots && cand == mn));
      const int tlast = __builtin_amdgcn_readlane(hi ? tb1 : tb0, bit);
      const int fi = tau > fmax ? nf : nf - 1 - (fmax - tau);
      for (int f = max(tau, fmax + 1); f < tlast + g.kt; ++f, ++nf) fr = lane == nf ? f : fr;
      fmax = max(fmax, tlast + g.kt - 1);
      const bool mine = lane == nt;
      e0 = mine ? t0 + t : e0;
      e1 = mine ? tau : e1;
      e2 = mine ? best : e2;
      e3 = mine ? fi : e3;
      ++nt;
      fa = lane == best ? tlast + g.kt : fa;
      if (hi) done1 |= 1ull << bit;
      else done0 |= 1ull << bit;
    }
    if (nt == 0) break;
    if (out) {
      int* hdr = out + size;
      if (lane == 0) {
        hdr[0] = nf;
        hdr[1] = nt;
      }
      if (lane < nf) hdr[2 + lane] = fr;
      if (lane < nt) {
        int* te = hdr + 2 + nf + 4 * lane;
        te[0] = e0;
        te[1] = e1;
        te[2] = e2;
        te[3] = e3;
      }
    }
    size += 2 + nf + 4 * nt;
    ++npass;
  }
  if (out && lane == 0) out[0] = npass;
  return size;
}

// Tile slices of a work item read from the descriptors in global memory, or from
// a copy in LDS.
struct TilesGlobal {
  const int* qt;  // descriptors of the item's first tile
  __device__ int tau0(int i) const { return qt[(size_t)i * QT_INTS]; }
  __device__ int tlast(int i) const { return qt[(size_t)i * QT_INTS + 1]; }
  __device__ int uni(int x) const { return __builtin_amdgcn_readfirstlane(x); }
};
struct TilesLds {
  const int2* c;  // (tau0, tlast) per tile
  __device__ int tau0(int i) const { return __builtin_amdgcn_readfirstlane(c[i].x); }
  __device__ int tlast(int i) const { return __builtin_amdgcn_readfirstlane(c[i].y); }
  __device__ int uni(int x) const { return __builtin_amdgcn_readfirstlane(x); }
};

// Room for the schedule of work item w: every pass schedules at least one tile and
// holds 2 + (frames <= QS_TS + kt - 1) + 4 per tile ints, so 1 + tiles (QS_TS + kt
// + 5) bounds it; the exclusive sum of these over the items before w is
// w + qt_off[w] (QS_TS + kt + 5), which needs no scan of its own (and stays within
// qs_ints(): tiles <= groups).
__device__ __forceinline__ int sched_offset(const Geom& g, const int* qt_off, int w) {
  return w + qt_off[w] * (QS_TS + g.kt + 5);
}

// One wave per work item: the wave copies the item's tile slices to LDS (when they
// fit), then runs the greedy pass on them with every value uniform (scalar
// instructions; the stores carry one value for all lanes).  Lane 0 also writes the
// item's schedule offset (and wave nw its end).
constexpr int SCHED_WAVES = 4, SCHED_CACHE = 1024;
__global__ __launch_bounds__(64 * SCHED_WAVES) void k_sched_fill(Geom g, const int* __restrict__ qt,
                                                                 const int* __restrict__ qt_off, int nw,
                                                                 int* __restrict__ off, int* __restrict__ sched,
                                                                 int nslots) {
  __shared__ int2 cache[SCHED_WAVES][SCHED_CACHE];
  __shared__ int work[SCHED_WAVES][4 * QS_MAXT];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int w = blockIdx.x * SCHED_WAVES + wv;
  const bool live = w < nw;
  if (w <= nw && lane == 0) off[w] = sched_offset(g, qt_off, w);
  const int t0 = live ? qt_off[w] : 0, ntiles = live ? qt_off[w + 1] - t0 : 0;
  const bool regs = ntiles <= 128, cached = !regs && ntiles <= SCHED_CACHE;
  int ta0 = 0, tb0 = 0, ta1 = 0, tb1 = 0;
  if (regs) {
    const int* d0 = qt + (size_t)(t0 + min(lane, max(ntiles - 1, 0))) * QT_INTS;
    const int* d1 = qt + (size_t)(t0 + min(lane + 64, max(ntiles - 1, 0))) * QT_INTS;
    if (ntiles > 0) {
      ta0 = d0[0];
      tb0 = d0[1];
      ta1 = d1[0];
      tb1 = d1[1];
    }
  }
  if (cached)
    for (int i = lane; i < ntiles; i += 64)
      cache[wv][i] = make_int2(qt[(size_t)(t0 + i) * QT_INTS], qt[(size_t)(t0 + i) * QT_INTS + 1]);
  __syncthreads();
  if (live) {
    int* out = sched + sched_offset(g, qt_off, w);
    if (regs)
      build_schedule_regs(g, t0, ntiles, ta0, tb0, ta1, tb1, out, lane, nslots);
    else if (cached)
      build_schedule(g, w, t0, ntiles, TilesLds{cache[wv]}, out, work[wv], lane, 64, nslots);
    else
      build_schedule(g, w, t0, ntiles, TilesGlobal{qt + (size_t)t0 * QT_INTS}, out, work[wv], lane, 64, nslots);
  }
}

hipError_t launch_qtile_count(const Geom& g, const Prep& p, hipStream_t s, bool blob_groups) {
  const int nw = qs_items(g) * g.ph, nblobs = g.nblobs * g.ph;
  const int tblock0 = blob_groups ? (nblobs + 1 + 63) / 64 : 0;
  k_qtile_count<<<(unsigned)(tblock0 + (nw + 1 + 63) / 64), 64, 0, s>>>(g, p.cell_ptr, nw, p.qt_off, tblock0, nblobs,
                                                                         p.goff);
  return hipGetLastError();
}

hipError_t launch_groups_qtiles(const Geom& g, const Prep& p, bool groups, bool qtiles, hipStream_t s) {
  const int nblobs = g.nblobs * g.ph, nw = qtiles ? qs_items(g) * g.ph : 0;
  const int gblocks = groups ? (nblobs + 255) / 256 + (nblobs == 0) : 0;
  const unsigned nb = (unsigned)(gblocks + (nw + 255) / 256);
  if (nb == 0) return hipSuccess;
  k_groups_qtiles<<<nb, 256, 0, s>>>(g, p.cell_ptr, p.goff, nblobs, p.groups, p.ngroups, gblocks, nw, p.qt_off, p.qt);
  return hipGetLastError();
}

hipError_t launch_sched_fill(const Geom& g, const Prep& p, int nslots, hipStream_t s) {
  const int nw = qs_items(g) * g.ph;
  k_sched_fill<<<(unsigned)((nw + 1 + SCHED_WAVES - 1) / SCHED_WAVES), 64 * SCHED_WAVES, 0, s>>>(g, p.qt, p.qt_off, nw,
                                                                                              p.qs_off, p.qs, nslots);
  return hipGetLastError();
}

hipError_t launch_qsched_rows(const Geom& g, const Prep& p, int nslots, hipStream_t s) {
  const int nw = qs_items(g) * g.ph;
  k_tile_fill<<<(unsigned)((p.max_groups + 15) / 16), 256, 0, s>>>(p.perm, p.starts, p.qt, p.qt_off + nw, g.N,
                                                                   p.tq_ids, p.tq_st, p.tq_dt);
  return launch_sched_fill(g, p, nslots, s);
}

hipError_t launch_qsched(const Geom& g, const Prep& p, int nslots, hipStream_t s) {
  hipError_t e = launch_qtile_count(g, p, s);
  if (e != hipSuccess) return e;
  e = launch_scan_excl(reinterpret_cast<uint32_t*>(p.qt_off), qs_items(g) * g.ph + 1, s, p.scan_part);
  if (e != hipSuccess) return e;
  if ((e = launch_groups_qtiles(g, p, false, true, s)) != hipSuccess) return e;
  return launch_qsched_rows(g, p, nslots, s);
}

}  // namespace dsa3d
