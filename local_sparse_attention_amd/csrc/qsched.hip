// Query-side work lists shared by the frame-sweeping forward and dQ kernels
// (head-independent: built once per call, used by every head).
//
// Row tiles: the queries of one start blob slice (1 x 4 x 4 start cells of the
// lattice of the 3D Deformable Slide Attention section) in groups of 16, as listed
// by groups / goff.  tq_ids / tq_st hold each tile's query tokens and window
// starts (sy, sx), padded to 16 with token 0 and a start no key matches.
//
// Schedules: a workgroup owns one start blob column (by, bx) and QS_TS consecutive
// slices.  Its row tiles get one of QS_SLOTS slots for the kt frames they read;
// greedy, in slice order, a tile takes the slot that has been free the longest
// (a slot is free again once its tile has read its last frame).  Tiles that find
// no free slot at their first frame wait for a further pass over the frames.
// Each pass lists the frames it sweeps (the union of its tiles' frame ranges, in
// order) and its tiles as (tile, slice, slot, index of the slice's frame in the list).
#include "internal.hpp"

namespace dsa3d {

__global__ __launch_bounds__(256) void k_tile_fill(const int* __restrict__ perm, const int4* __restrict__ starts,
                                                   const int2* __restrict__ groups, const int* __restrict__ ngroups,
                                                   int* __restrict__ tq_ids, int2* __restrict__ tq_st) {
  const int g = blockIdx.x * 16 + (threadIdx.x >> 4), j = threadIdx.x & 15;
  if (g >= *ngroups) return;
  const int2 gr = groups[g];
  int id = 0;
  int2 st = make_int2(-(1 << 29), -(1 << 29));
  if (j < gr.y) {
    id = perm[gr.x + j];
    const int4 s = starts[id];
    st = make_int2(s.y, s.z);
  }
  tq_ids[(size_t)g * 16 + j] = id;
  tq_st[(size_t)g * 16 + j] = st;
}

// Runs the greedy schedule of work item w (blob column, chunk) and writes it to out;
// returns its size in ints.
__device__ int build_schedule(const Geom& g, const int* __restrict__ goff, int w, int* out) {
  const int nbc = g.nby * g.nbx;
  const int chunk = w / nbc, bc = w - chunk * nbc;
  const int by = bc / g.nbx, bx = bc - by * g.nbx;
  const int c0 = chunk * QS_TS, ns = min(QS_TS, g.Lt - c0);
  int done[QS_TS];
  for (int i = 0; i < QS_TS; ++i) done[i] = 0;
  auto blob_of = [&](int tau) { return (tau * g.nby + by) * g.nbx + bx; };
  int size = 1, npass = 0;
  for (;;) {
    int free_at[QS_SLOTS];
    for (int s = 0; s < QS_SLOTS; ++s) free_at[s] = -(1 << 29);
    // first pass over the slices: count frames and tiles; second: write
    int nf = 0, nt = 0, fmax = -1;
    int* hdr = out ? out + size : nullptr;
    int* frames = hdr ? hdr + 2 : nullptr;
    // tiles are written after the frames, whose count is known only at the end,
    // so collect them first into a bounded local list
    int tg[QS_MAXT], tt[QS_MAXT], tslot[QS_MAXT], tfi[QS_MAXT];
    for (int i = 0; i < ns && nt < QS_MAXT; ++i) {
      const int tau = c0 + i, b = blob_of(tau);
      const int first = goff[b], ntl = goff[b + 1] - first;
      while (done[i] < ntl && nt < QS_MAXT) {
        int best = -1;
        for (int s = 0; s < QS_SLOTS; ++s)
          if (free_at[s] <= tau && (best < 0 || free_at[s] < free_at[best])) best = s;
        if (best < 0) break;
        int fi;
        if (tau > fmax) {
          fi = nf;
        } else {
          fi = nf - 1 - (fmax - tau);
        }
        for (int f = max(tau, fmax + 1); f < tau + g.kt; ++f) {
          if (frames) frames[nf] = f;
          ++nf;
        }
        fmax = max(fmax, tau + g.kt - 1);
        tg[nt] = first + done[i];
        tt[nt] = tau;
        tslot[nt] = best;
        tfi[nt] = fi;
        ++nt;
        free_at[best] = tau + g.kt;
        ++done[i];
      }
    }
    if (nt == 0) break;
    if (hdr) {
      hdr[0] = nf;
      hdr[1] = nt;
      int* tl = frames + nf;
      for (int t = 0; t < nt; ++t) {
        tl[4 * t + 0] = tg[t];
        tl[4 * t + 1] = tt[t];
        tl[4 * t + 2] = tslot[t];
        tl[4 * t + 3] = tfi[t];
      }
    }
    size += 2 + nf + 4 * nt;
    ++npass;
  }
  if (out) out[0] = npass;
  return size;
}

// Room for the schedule of work item w: every pass schedules at least one tile and
// holds 2 + (frames <= QS_TS + kt - 1) + 4 per tile ints, so 1 + tiles (QS_TS + kt
// + 5) bounds it (the sum over items stays within qs_ints()).
__global__ __launch_bounds__(64) void k_sched_count(Geom g, const int* __restrict__ goff, int nw, int* __restrict__ off) {
  const int w = blockIdx.x * 64 + threadIdx.x;
  if (w >= nw) return;
  const int nbc = g.nby * g.nbx;
  const int chunk = w / nbc, bc = w - chunk * nbc;
  const int by = bc / g.nbx, bx = bc - by * g.nbx;
  const int c0 = chunk * QS_TS, ns = min(QS_TS, g.Lt - c0);
  int tiles = 0;
  for (int i = 0; i < ns; ++i) {
    const int b = ((c0 + i) * g.nby + by) * g.nbx + bx;
    tiles += goff[b + 1] - goff[b];
  }
  off[w] = 1 + tiles * (QS_TS + g.kt + 5);
}

__global__ __launch_bounds__(64) void k_sched_fill(Geom g, const int* __restrict__ goff, int nw,
                                                   const int* __restrict__ off, int* __restrict__ sched) {
  const int w = blockIdx.x * 64 + threadIdx.x;
  if (w < nw) build_schedule(g, goff, w, sched + off[w]);
}

hipError_t launch_qsched(const Geom& g, const Prep& p, hipStream_t s) {
  k_tile_fill<<<(unsigned)((p.max_groups + 15) / 16), 256, 0, s>>>(p.perm, p.starts, p.groups, p.ngroups, p.tq_ids,
                                                                   p.tq_st);
  const int nw = qs_items(g);
  k_sched_count<<<(unsigned)((nw + 63) / 64), 64, 0, s>>>(g, p.goff, nw, p.qs_off);
  if (launch_scan_excl(reinterpret_cast<uint32_t*>(p.qs_off), nw + 1, s) != hipSuccess) return hipGetLastError();
  k_sched_fill<<<(unsigned)((nw + 63) / 64), 64, 0, s>>>(g, p.goff, nw, p.qs_off, p.qs);
  return hipGetLastError();
}

}  // namespace dsa3d
