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
// Schedules: a work item's row tiles get one of QS_SLOTS slots for the frames they
// read; greedy, in tile order, a tile takes the slot that has been free the longest
// (a slot is free again once its tile has read its last frame).  Tiles that find
// no free slot at their first frame wait for a further pass over the frames.
// Each pass lists the frames it sweeps (the union of its tiles' frame ranges, in
// order) and its tiles as (tile, tau0, slot, index of frame tau0 in the list).
#include "internal.hpp"

namespace dsa3d {

// Row tiles of work item w (see above): writes their descriptors to out (if not
// null) and returns their count, which is at most the item's group count.
__device__ int item_tiles(const Geom& g, const int* __restrict__ goff, const int2* __restrict__ groups, int w,
                          int* out) {
  const int nbc = g.nby * g.nbx, nw = qs_items(g);
  const int hb = w / nw;
  w -= hb * nw;
  goff += (size_t)hb * g.nblobs;  // the head block's blobs (their group indices are global)
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
  int n = 0, open = -1, acc = 0, s0 = 0, np = 0;
  for (int i = 0; i < ns; ++i) {
    const int tau = c0 + i, b = (tau * g.nby + by) * g.nbx + bx;
    const int gb = goff[b], ng = goff[b + 1] - gb;
    if (ng == 0) continue;
    const int2 last = groups[gb + ng - 1];
    const int nfull = last.y == GROUP_Q ? ng : ng - 1;
    for (int k = 0; k < nfull; ++k, ++n)
      if (out) put(n, tau, groups[gb + k].x, GROUP_Q);
    if (last.y == GROUP_Q) continue;
    if (open >= 0 && acc + last.y <= GROUP_Q && tau - s0 < QS_SPAN) {
      if (out) {
        int* d = out + (size_t)open * QT_INTS;
        d[1] = tau;
        d[2 + 3 * np] = last.x;
        d[3 + 3 * np] = last.y;
        d[4 + 3 * np] = tau - s0;
      }
      ++np;
      acc += last.y;
    } else {
      if (out) put(n, tau, last.x, last.y);
      open = n++;
      s0 = tau;
      acc = last.y;
      np = 1;
    }
  }
  return n;
}

__global__ __launch_bounds__(64) void k_qtile_count(Geom g, const int* __restrict__ goff,
                                                    const int2* __restrict__ groups, int nw, int* __restrict__ qt_off) {
  const int w = blockIdx.x * 64 + threadIdx.x;
  if (w < nw) qt_off[w] = item_tiles(g, goff, groups, w, nullptr);
  if (w == nw) qt_off[w] = 0;
}

__global__ __launch_bounds__(64) void k_qtile_fill(Geom g, const int* __restrict__ goff,
                                                   const int2* __restrict__ groups, int nw,
                                                   const int* __restrict__ qt_off, int* __restrict__ qt) {
  const int w = blockIdx.x * 64 + threadIdx.x;
  if (w < nw) item_tiles(g, goff, groups, w, qt + (size_t)qt_off[w] * QT_INTS);
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
                              int lane, int nlanes) {
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
    int free_at[QS_SLOTS];
    for (int s = 0; s < QS_SLOTS; ++s) free_at[s] = -(1 << 29);
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
        for (int s = 0; s < QS_SLOTS; ++s)
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
// + 5) bounds it (the sum over items stays within qs_ints(): tiles <= groups).
__global__ __launch_bounds__(64) void k_sched_count(Geom g, const int* __restrict__ qt_off, int nw,
                                                    int* __restrict__ off) {
  const int w = blockIdx.x * 64 + threadIdx.x;
  if (w >= nw) return;
  off[w] = 1 + (qt_off[w + 1] - qt_off[w]) * (QS_TS + g.kt + 5);
}

// One wave per work item: the wave copies the item's tile slices to LDS (when they
// fit), then runs the greedy pass on them with every value uniform (scalar
// instructions; the stores carry one value for all lanes).
constexpr int SCHED_WAVES = 4, SCHED_CACHE = 1024;
__global__ __launch_bounds__(64 * SCHED_WAVES) void k_sched_fill(Geom g, const int* __restrict__ qt,
                                                                 const int* __restrict__ qt_off, int nw,
                                                                 const int* __restrict__ off, int* __restrict__ sched) {
  __shared__ int2 cache[SCHED_WAVES][SCHED_CACHE];
  __shared__ int work[SCHED_WAVES][4 * QS_MAXT];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int w = blockIdx.x * SCHED_WAVES + wv;
  const bool live = w < nw;
  const int t0 = live ? qt_off[w] : 0, ntiles = live ? qt_off[w + 1] - t0 : 0;
  const bool cached = ntiles <= SCHED_CACHE;
  if (cached)
    for (int i = lane; i < ntiles; i += 64)
      cache[wv][i] = make_int2(qt[(size_t)(t0 + i) * QT_INTS], qt[(size_t)(t0 + i) * QT_INTS + 1]);
  __syncthreads();
  if (live) {
    if (cached)
      build_schedule(g, w, t0, ntiles, TilesLds{cache[wv]}, sched + off[w], work[wv], lane, 64);
    else
      build_schedule(g, w, t0, ntiles, TilesGlobal{qt + (size_t)t0 * QT_INTS}, sched + off[w], work[wv], lane,
                     64);
  }
}

hipError_t launch_qsched(const Geom& g, const Prep& p, hipStream_t s) {
  const int nw = qs_items(g) * g.ph;
  const unsigned wb = (unsigned)((nw + 1 + 63) / 64);
  k_qtile_count<<<wb, 64, 0, s>>>(g, p.goff, p.groups, nw, p.qt_off);
  if (launch_scan_excl(reinterpret_cast<uint32_t*>(p.qt_off), nw + 1, s, p.scan_part) != hipSuccess)
    return hipGetLastError();
  k_qtile_fill<<<wb, 64, 0, s>>>(g, p.goff, p.groups, nw, p.qt_off, p.qt);
  k_tile_fill<<<(unsigned)((p.max_groups + 15) / 16), 256, 0, s>>>(p.perm, p.starts, p.qt, p.qt_off + nw, g.N,
                                                                   p.tq_ids, p.tq_st, p.tq_dt);
  k_sched_count<<<wb, 64, 0, s>>>(g, p.qt_off, nw, p.qs_off);
  if (launch_scan_excl(reinterpret_cast<uint32_t*>(p.qs_off), nw + 1, s, p.scan_part) != hipSuccess)
    return hipGetLastError();
  k_sched_fill<<<(unsigned)((nw + SCHED_WAVES - 1) / SCHED_WAVES), 64 * SCHED_WAVES, 0, s>>>(g, p.qt, p.qt_off, nw,
                                                                                          p.qs_off, p.qs);
  return hipGetLastError();
}

}  // namespace dsa3d
