// Pieces shared by the query-side frame-sweeping kernels (forward, dQ): the pass
// tables a workgroup keeps in LDS and the direct loads of key tiles.
#pragma once

#include "internal.hpp"
#include "tube.hpp"

namespace dsa3d {

// One pass of a work item's schedule (see qsched.hip), in LDS.
struct QsPass {
  int ids[QS_MAXT][16];             // query tokens of each tile of the pass
  int2 st[QS_MAXT][16];             // their window starts (sy, sx)
  signed char dt[QS_MAXT][16];      // their slices minus the tile's first slice
  int tau[QS_MAXT];                 // first slice of each tile
  int tlast[QS_MAXT];               // last slice of each tile
  short act[QS_TS + 16][QS_SLOTS_MAX];  // tile activated at (frame index, slot), or -1
  int frames[QS_TS + 16];           // frames swept by the pass
  int hdr[2];                       // frame count, tile count
};

// Reads the pass at sp into T (all threads of the workgroup; ends with a barrier)
// and advances sp past it.
__device__ __forceinline__ void load_pass(QsPass& T, const int*& sp, const Prep& p, int tid, int nthreads) {
  if (tid == 0) {
    T.hdr[0] = sp[0];
    T.hdr[1] = sp[1];
  }
  for (int i = tid; i < (QS_TS + 16) * QS_SLOTS_MAX; i += nthreads) (&T.act[0][0])[i] = -1;
  __syncthreads();
  const int nf = T.hdr[0], nt = T.hdr[1];
  for (int i = tid; i < nf; i += nthreads) T.frames[i] = sp[2 + i];
  const int* tl = sp + 2 + nf;
  for (int i = tid; i < nt * 16; i += nthreads) {
    const int t = i >> 4, j = i & 15;
    const int gi = tl[4 * t];
    T.ids[t][j] = p.tq_ids[(size_t)gi * 16 + j];
    T.st[t][j] = p.tq_st[(size_t)gi * 16 + j];
    T.dt[t][j] = p.tq_dt[(size_t)gi * 16 + j];
    if (j == 0) {
      T.tau[t] = tl[4 * t + 1];
      T.tlast[t] = p.qt[(size_t)gi * QT_INTS + 1];
      T.act[tl[4 * t + 3]][tl[4 * t + 2]] = (short)t;
    }
  }
  sp += 2 + nf + 4 * nt;
  __syncthreads();
}

// Lane constants of the key tile loads below.  Load j, lane l covers row
// 8 j + (l >> 3) of the tile: key (2 (j & 1) + (l >> 5), (l >> 3) & 3) of block
// j >> 1, 16-byte chunk (l & 7) ^ ((l >> 3) & 7) of the swizzled row.
struct KeyLane {
  int ly, lx;           // key offset inside the block's half (rows), column
  uint32_t off, off0;   // element offset of the lane's key inside a frame; of token (0, 0)
};
template <int D>
__device__ __forceinline__ KeyLane key_lane(const Geom& g, int h, int lane) {
  KeyLane kl;
  kl.ly = lane >> 5;
  kl.lx = (lane >> 3) & 3;
  kl.off0 = (uint32_t)(h * D + ((lane & 7) ^ ((lane >> 3) & 7)) * 8);
  kl.off = (uint32_t)((kl.ly * g.Wp + kl.lx) * g.H * D) + kl.off0;
  return kl;
}

// Direct loads of column phase ph (64 bf16 columns) of the key tile of frame f
// anchored at start blob (by, bx): NBLK blocks of 4 x 4 keys, NBX per tile row, 16
// rows of 128 bytes each in the swizzled layout; this wave's share (PER loads) of
// the 2 NLB 1 KB loads.  NLB >= NBLK: the extra blocks, like rows outside the grid,
// read the frame's token (0, 0), finite values that the window mask or a zero
// weight ignores.  Only the in-grid test and one add depend on the lane.
template <int D, int NBX, int NBLK, int NLB, int NW>
__device__ __forceinline__ void issue_key_tile(char* dst, const u16* src, const Geom& g, const KeyLane& kl, int by,
                                               int bx, int f, int ph, int wave) {
  static_assert((2 * NLB) % NW == 0, "loads must split evenly over the waves");
  const u16* base = src + (size_t)f * g.Hp * g.Wp * g.H * D + ph * 64;
#pragma unroll
  for (int jj = 0; jj < 2 * NLB / NW; ++jj) {
    int j = wave + NW * jj;
    // opaque to the optimiser: the per-load values below do not depend on the frame,
    // and hoisting all of them out of the frame loop costs more registers than the
    // few instructions it saves
    __asm__ __volatile__("" : "+s"(j));
    const int b = j >> 1;
    const int bi = b / NBX, bj = b - bi * NBX;
    const int y0 = 4 * by + 4 * bi + 2 * (j & 1), x0 = 4 * bx + 4 * bj;
    const bool in = b < NBLK && kl.ly < g.Hp - y0 && kl.lx < g.Wp - x0;
    const uint32_t off = in ? (uint32_t)((y0 * g.Wp + x0) * g.H * D) + kl.off : kl.off0;
    dma16(base + off, dst + j * 1024);
  }
}

// The same loads as issue_key_tile, as a loop over this wave's loads with the
// address computed per lane (kernels whose registers are too tight to keep the
// unrolled version's values live).
template <int D, int NBX, int NBLK, int NLB, int NW>
__device__ __forceinline__ void issue_key_tile_loop(char* dst, const u16* src, const Geom& g, int by, int bx, int h,
                                                    int f, int ph, int wave, int lane) {
  for (int j = wave; j < 2 * NLB; j += NW) {
    const int row = 8 * j + (lane >> 3), b = row >> 4, kk = row & 15;
    const int bi = b / NBX, bj = b - bi * NBX;
    const int y = 4 * by + 4 * bi + (kk >> 2), x = 4 * bx + 4 * bj + (kk & 3);
    const int tok = (b < NBLK && y < g.Hp && x < g.Wp) ? (f * g.Hp + y) * g.Wp + x : f * g.Hp * g.Wp;
    const int ch = (lane & 7) ^ (row & 7);
    dma16(src + ((size_t)tok * g.H + h) * D + ph * 64 + ch * 8, dst + j * 1024);
  }
}

// Loads WI, WI + NW, WI + 2 NW, ... of the 2 NLB 1 KB loads of one column phase
// of the key tile of frame f (layout as in issue_key_tile), for the wave that is
// number WI (a compile-time constant: each load is then a few instructions) of NW
// issuing waves.  Every such wave issues ceil(2 NLB / NW) loads; the missing ones
// are one-lane loads of pad_src into sink, so all waves count the same.  src
// points at the tensor's element (token 0, head h, column phase ph, the lane's
// 16-byte chunk (l & 7) ^ ((l >> 3) & 7)).
template <int D, int NBX, int NBLK, int NLB, int NW, int WI>
__device__ __forceinline__ void issue_key_tile_w(char* dst, const u16* src, const Geom& g, int by, int bx, int f,
                                                 int lane, const void* pad_src, void* sink) {
  const int ly = lane >> 5, lx = (lane >> 3) & 3;
  const int fbase = f * g.Hp * g.Wp;
  static_for<0, (2 * NLB + NW - 1) / NW>([&](auto JJ) {
    constexpr int j = WI + NW * decltype(JJ)::value;
    if constexpr (j < 2 * NLB) {
      constexpr int b = j >> 1, bi = b / NBX, bj = b % NBX;
      const int y = 4 * by + 4 * bi + 2 * (j & 1) + ly, x = 4 * bx + 4 * bj + lx;
      const int tok = (b < NBLK && y < g.Hp && x < g.Wp) ? fbase + y * g.Wp + x : fbase;
      dma16(src + (size_t)tok * g.H * D, dst + j * 1024);
    } else {
      if (lane == 0) dma4(pad_src, sink);
    }
  });
}

// The loads WI, WI + NW, ... of issue_key_tile_w with their frame-independent
// part precomputed: off[i] is the lane's byte offset, inside one frame of the
// [N][H][D] tensor and from column 0 of head h, of load WI + NW i (0 for loads
// beyond the tile).  issue() then costs no vector instructions per load.  Needs
// Hp Wp H D 2 < 2^32 (byte offsets inside a frame fit 32 bits).
template <int D, int NBX, int NBLK, int NLB, int NW, int WI>
struct KeyTileLoads {
  static constexpr int N = (2 * NLB + NW - 1) / NW;
  uint32_t off[N];
  __device__ __forceinline__ void init(const Geom& g, int h, int by, int bx, int lane) {
    const int ly = lane >> 5, lx = (lane >> 3) & 3;
    const uint32_t lane_b = (uint32_t)(h * D + (((lane & 7) ^ ((lane >> 3) & 7)) * 8)) * 2u;
    static_for<0, N>([&](auto JJ) {
      constexpr int i = decltype(JJ)::value, j = WI + NW * i;
      if constexpr (j < 2 * NLB) {
        constexpr int b = j >> 1, bi = b / NBX, bj = b % NBX;
        const int y = 4 * by + 4 * bi + 2 * (j & 1) + ly, x = 4 * bx + 4 * bj + lx;
        const bool in = b < NBLK && y < g.Hp && x < g.Wp;
        off[i] = (in ? (uint32_t)(y * g.Wp + x) * (uint32_t)(g.H * D) * 2u : 0u) + lane_b;
      } else {
        off[i] = 0u;
      }
    });
  }
  // frame_base: the tensor's element (token (f, 0, 0), head 0, column phase start)
  __device__ __forceinline__ void issue(char* dst, const u16* frame_base, int lane, const void* pad_src,
                                        void* sink) const {
    static_for<0, N>([&](auto JJ) {
      constexpr int i = decltype(JJ)::value, j = WI + NW * i;
      if constexpr (j < 2 * NLB) {
        dma16_s(frame_base, off[i], dst + j * 1024);
      } else {
        if (lane == 0) dma4(pad_src, sink);
      }
    });
  }
};

// KeyTileLoads for issuing wave wi (wave-uniform, known at run time): load
// wi + NW i, i < N.  The missing loads of the last round are one-lane loads of
// pad_src into sink, so every wave counts the same.
template <int D, int NBX, int NBLK, int NLB, int NW>
struct KeyTileLoadsW {
  static constexpr int N = (2 * NLB + NW - 1) / NW;
  uint32_t off[N];
  int wi;
  __device__ __forceinline__ void init(const Geom& g, int h, int by, int bx, int lane, int wave) {
    wi = wave;
    const int ly = lane >> 5, lx = (lane >> 3) & 3;
    const uint32_t lane_b = (uint32_t)(h * D + (((lane & 7) ^ ((lane >> 3) & 7)) * 8)) * 2u;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int j = wi + NW * i, b = j >> 1, bi = b / NBX, bj = b - bi * NBX;
      const int y = 4 * by + 4 * bi + 2 * (j & 1) + ly, x = 4 * bx + 4 * bj + lx;
      const bool in = j < 2 * NLB && b < NBLK && y < g.Hp && x < g.Wp;
      off[i] = (in ? (uint32_t)(y * g.Wp + x) * (uint32_t)(g.H * D) * 2u : 0u) + lane_b;
    }
  }
  __device__ __forceinline__ void issue(char* dst, const u16* frame_base, int lane, const void* pad_src,
                                        void* sink) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int j = wi + NW * i;
      if (j < 2 * NLB)
        dma16_s(frame_base, off[i], dst + j * 1024);
      else if (lane == 0)
        dma4(pad_src, sink);
    }
  }
};

// The lane's element offset inside a row for issue_key_tile_w and issue_rows.
__device__ __forceinline__ int lane_chunk_el(int lane) { return ((lane & 7) ^ ((lane >> 3) & 7)) * 8; }

// Direct loads of the 16 rows (tokens ids[0..15]) of a [N][H][D] bf16 tensor into a
// staged row tile: NPH phases of 16 x 128 bytes, swizzled like the key tiles.
// tok0 / tok1: the tokens of rows lane >> 3 and 8 + (lane >> 3).
template <int D>
__device__ __forceinline__ void issue_rows_tok(char* dst, const u16* src, int tok0, int tok1, const Geom& g, int h,
                                               int lane) {
  const u16* r0 = src + ((size_t)tok0 * g.H + h) * D + lane_chunk_el(lane);
  const u16* r1 = src + ((size_t)tok1 * g.H + h) * D + lane_chunk_el(lane);
#pragma unroll
  for (int j = 0; j < 2 * (D / 64); ++j) {
    const int ph = j >> 1, hh = j & 1;
    dma16((hh ? r1 : r0) + ph * 64, dst + ph * 2048 + hh * 1024);
  }
}
template <int D>
__device__ __forceinline__ void issue_rows(char* dst, const u16* src, const int* ids, const Geom& g, int h, int lane) {
  // both tokens first: every direct load clobbers memory for the compiler, which
  // would otherwise read (and wait for) the token again before each load
  issue_rows_tok<D>(dst, src, ids[lane >> 3], ids[8 + (lane >> 3)], g, h, lane);
}

}  // namespace dsa3d
