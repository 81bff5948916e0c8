// "Tube" forward kernel for 3D Deformable Slide Attention (MegaSlide-DiT, section
// "3D Deformable Slide Attention", Eq. (1) attention term) on gfx950.
//
// One workgroup owns one 1 x 4 x 4 start blob position (by, bx) of the start
// lattice and one head, and sweeps the frames of the grid.  The queries whose
// window starts at (tau, 4by..4by+3, 4bx..4bx+3) form the blob's slice tau; all of
// them read frames tau .. tau+kt-1, and inside a frame only the (4+ky-1) x (4+kx-1)
// key tile anchored at (4by, 4bx).  The workgroup has kt waves; wave w owns the
// slices tau = w (mod kt), so at frame f the kt slices f-kt+1 .. f are in flight
// at once, one per wave, and all of them read the same key tile.  A frame tile is
// staged into LDS once per blob (not once per slice and query group): K first and
// V second, in 128-byte column phases, with direct global->LDS loads
// (global_load_lds_dwordx4) double-buffered against the MFMAs.
//
// Per wave and frame: S^T = K Q^T on 16x16x32 bf16 MFMA (4x4 key blocks x 16
// queries), mask to the query's own window, online softmax, O^T += V^T P^T with
// V^T read by ds_read_b64_tr_b16.  A wave holds up to 32 queries of its slice;
// slices with more are finished in further sweeps ("passes") that only visit the
// frames those slices need.
//
// LDS tile layout: rows of 128 bytes (one key, one column phase), key blocks of 16
// rows; the 16-byte chunk c of row r sits at chunk position c ^ (r & 7), which
// spreads the row-wise and the transposed fragment reads over the banks.
#include "internal.hpp"
#include "tube.hpp"

namespace dsa3d {


template <typename T, int D>
struct TubeCfg {
  static constexpr int EV = 16 / (int)sizeof(T);   // elements per 16-byte chunk
  static constexpr int PW = 128 / (int)sizeof(T);  // phase width (elements): 128 bytes of a row
  static constexpr int NPH = D / PW;               // column phases per K (or V) pass
  static constexpr int NBMAX = 9;                  // key blocks (4x4 keys) per frame tile
  static constexpr int NBPAD = 10;                 // rounded up to whole 32-key pairs
  static constexpr int ROWS = NBPAD * 16;          // rows per phase tile
  static constexpr int TILE_BYTES = ROWS * 128;
  static constexpr int NCP = PW / 32;              // 32-deep contraction steps per phase
  static constexpr int NTP = PW / 16;              // 16-wide d tiles per phase
  static constexpr int NC = D / 32, NT = D / 16;
  static constexpr int RT = 2;                     // 16-query row tiles per wave
  static constexpr int QCAP = RT * 16;
  static constexpr int NPAIR = NBPAD / 2;
  static constexpr int NLOADS = NBMAX * 16 * 128 / 1024;  // 1 KB direct loads per phase tile (pad rows stay 0)
  static constexpr int NBUF = 7;                   // ring of phase tiles in LDS
  static constexpr int PD = NBUF - 1;              // prefetch distance (steps)
};

constexpr int TUBE_TS = 32;      // start slices per workgroup
constexpr int TUBE_MAX_TS = 64;


// Row-wise fragment: 8 elements of row `row` starting at element `e0` (16 or 32 bytes).
__device__ __forceinline__ void lds_frag_row(Frag<u16>& f, const char* tile, int row, int e0) {
  const uint4 u = *reinterpret_cast<const uint4*>(tile + sw(row, e0 * 2));
  __builtin_memcpy(&f.v, &u, 16);
}
__device__ __forceinline__ void lds_frag_row(Frag<float>& f, const char* tile, int row, int e0) {
  const float4 a = *reinterpret_cast<const float4*>(tile + sw(row, e0 * 4));
  const float4 b = *reinterpret_cast<const float4*>(tile + sw(row, e0 * 4 + 16));
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

// Transposed fragment: slot j < 4 is row r_lo + j, slot j >= 4 is row r_hi + j - 4,
// all at column c0 + (lane & 15).  bf16: two ds_read_b64_tr_b16; within a 16-lane
// group, lane i returns element (i & 3) of the 8 bytes loaded by lane 4j + (i >> 2),
// so each lane points at row r + (i >> 2), columns c0 + 4 (i & 3) .. +3.
__device__ __forceinline__ void lds_frag_tr(Frag<u16>& f, const char* tile, int r_lo, int r_hi, int c0, int lane) {
  const int i = lane & 15;
  const int byte = (c0 + 4 * (i & 3)) * 2;
  const char* pa = tile + sw(r_lo + (i >> 2), byte);
  const char* pb = tile + sw(r_hi + (i >> 2), byte);
  const shortx4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t*)pa);
  const shortx4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t*)pb);
  const shortx4_t both[2] = {a, b};
  __builtin_memcpy(&f.v, both, 16);
}
__device__ __forceinline__ void lds_frag_tr(Frag<float>& f, const char* tile, int r_lo, int r_hi, int c0, int lane) {
  const int byte = (c0 + (lane & 15)) * 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f.v[j] = *reinterpret_cast<const float*>(tile + sw(r_lo + j, byte));
    f.v[j + 4] = *reinterpret_cast<const float*>(tile + sw(r_hi + j, byte));
  }
}

// Per-lane byte offsets inside a swizzled phase tile, independent of the key block:
// a block is 16 rows (2048 bytes), so block b adds b * 2048 and keeps (row & 7).
// Row-wise fragment of chunk step c: row r16 of the block, elements c*32 + quad*8.
template <typename T>
__device__ __forceinline__ int row_frag_off(int c, int lane, int half) {
  const int r16 = lane & 15, quad = lane >> 4;
  const int byte = (c * 32 + quad * 8) * (int)sizeof(T) + 16 * half;
  return sw(r16, byte);
}
// Transposed bf16 fragment of d tile dt (rows 4*quad + (i >> 2) of a block).
__device__ __forceinline__ int tr_frag_off(int dt, int lane) {
  const int i = lane & 15, quad = lane >> 4;
  return sw(4 * quad + (i >> 2), (dt * 16 + 4 * (i & 3)) * 2);
}

__device__ __forceinline__ void lds_row(Frag<u16>& f, const char* blk, const int* off) {
  const uint4 u = *reinterpret_cast<const uint4*>(blk + off[0]);
  __builtin_memcpy(&f.v, &u, 16);
}
__device__ __forceinline__ void lds_row(Frag<float>& f, const char* blk, const int* off) {
  const float4 a = *reinterpret_cast<const float4*>(blk + off[0]);
  const float4 b = *reinterpret_cast<const float4*>(blk + off[1]);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
// pair = blocks (2c, 2c+1) starting at `pair`; slots j < 4 come from the first block
__device__ __forceinline__ void lds_tr(Frag<u16>& f, const char* pair, const int* toff, int dt, int lane) {
  const shortx4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t*)(pair + toff[dt]));
  const shortx4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t*)(pair + 2048 + toff[dt]));
  const shortx4_t both[2] = {a, b};
  __builtin_memcpy(&f.v, both, 16);
}
__device__ __forceinline__ void lds_tr(Frag<float>& f, const char* pair, const int*, int dt, int lane) {
  lds_frag_tr(f, pair, 4 * (lane >> 4), 16 + 4 * (lane >> 4), dt * 16, lane);
}

struct TubeGeo {
  int by, bx;   // start blob position
  int nbx_t;    // key blocks per tile row
  int nb;       // key blocks in the tile
};


// Token of tile row `row` at frame f, or -1 outside the grid / past the tile.
__device__ __forceinline__ int tile_token(const Geom& g, const TubeGeo& tg, int f, int row) {
  const int b = row >> 4, kk = row & 15;
  if (b >= tg.nb) return -1;
  const int bi = b / tg.nbx_t, bj = b - bi * tg.nbx_t;
  const int y = 4 * tg.by + 4 * bi + (kk >> 2), x = 4 * tg.bx + 4 * bj + (kk & 3);
  if (y >= g.Hp || x >= g.Wp) return -1;
  return (f * g.Hp + y) * g.Wp + x;
}

// Issue the direct loads of one phase tile: columns [col, col + PW) of the keys
// of frame f.  Rows outside the grid are left as they are (every row of both
// buffers is zeroed once; masked keys meet zero softmax weights).
template <typename T, int D>
__device__ __forceinline__ void issue_tile(char* dst, const T* __restrict__ src, const Geom& g, const TubeGeo& tg,
                                           int f, int col, int h, int wave, int nwaves, int lane) {
  using C = TubeCfg<T, D>;
  for (int j = wave; j < C::NLOADS; j += nwaves) {
    const int row = 8 * j + (lane >> 3);
    const int chunk = (lane & 7) ^ (row & 7);  // logical chunk landing at this lane's slot
    // every lane loads, so each wave issues the same number of loads every step (the
    // ring's vmcnt waits count on it); rows outside the grid read token 0 instead,
    // finite values that the mask gives zero weight
    const int tok = max(tile_token(g, tg, f, row), 0);
    const T* gp = src + ((size_t)tok * g.H + h) * D + col + chunk * C::EV;
    dma16(gp, dst + j * 1024);
  }
}



__device__ __forceinline__ void wait_direct_loads() { __asm__ __volatile__("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup schedule of a chunk of start slices: every row tile (16 queries of
// one slice of the start blob) gets a slot (wave, register set) for the kt frames
// its slice reads; a slot takes its next row tile once the previous one is done
// and G more frames have passed (its Q rows are loaded into the slot's LDS area
// ahead of time, while the previous row tile may still be reading it).  Row tiles
// that find no free slot at their slice's first frame wait for the next pass.
// Built by one thread; tiny.
constexpr int FT_NW = 4;        // waves per workgroup (one per SIMD)
#ifndef DSA3D_FT_NS
#define DSA3D_FT_NS 3
#endif
constexpr int FT_NS = DSA3D_FT_NS;  // row-tile slots per wave
constexpr int FT_SLOTS = FT_NW * FT_NS;
constexpr int FT_MAXQ = 24;     // queued row tiles per slot and pass

template <typename T, int D, int NBX>
__global__ __launch_bounds__(256) void k_forward_ft(const T* __restrict__ q, const T* __restrict__ k,
                                                    const T* __restrict__ v, T* __restrict__ out,
                                                    float* __restrict__ lse, Geom g, Prep p, float sl2, int TS) {
  using C = TubeCfg<T, D>;
  constexpr int NPH2 = 2 * C::NPH;
  // fp32 runs one slot per wave: with several, a conditional MFMA block that a wave
  // skips can leave an accumulator read closer to its MFMA than the hardware allows
  // (seen as wrong fp32 results; kept out of the code rather than worked around)
  constexpr int NW = FT_NW, NS = sizeof(T) == 4 ? 1 : FT_NS;
  constexpr int QROW = D * (int)sizeof(T);   // bytes of one query row
  constexpr int QCH = QROW / 16;             // 16-byte chunks per query row
  constexpr int QROWS_PER_LOAD = 1024 / QROW;
  constexpr int NBUF = 5, PD = NBUF - 1;
  constexpr int GAP = (PD + NPH2 - 1) / NPH2;  // frames between row tiles on one slot
  __shared__ __attribute__((aligned(1024))) char tile[NBUF][C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char qlds[FT_SLOTS][16 * QROW];
  __shared__ int s_beg[TUBE_MAX_TS], s_cnt[TUBE_MAX_TS], s_done[TUBE_MAX_TS];
  __shared__ short s_qtau[FT_SLOTS][FT_MAXQ], s_qr[FT_SLOTS][FT_MAXQ];
  __shared__ int s_qlen[FT_SLOTS];
  __shared__ short s_frames[TUBE_MAX_TS + 48];
  __shared__ int s_nf, s_left;

  const int nblob2 = g.nby * g.nbx;
  const int nchunk = (g.Lt + TS - 1) / TS;
  int logical = xcd_remap(blockIdx.x + gridDim.x * blockIdx.y, nblob2 * nchunk * g.H);
  const int h = logical / (nblob2 * nchunk);
  logical -= h * nblob2 * nchunk;
  const int tchunk = logical / nblob2, blob2 = logical - tchunk * nblob2;
  TubeGeo tg;
  tg.by = blob2 / g.nbx;
  tg.bx = blob2 - tg.by * g.nbx;
  tg.nbx_t = NBX;
  tg.nb = ((4 + g.ky - 1 + 3) / 4) * NBX;
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, quad = lane >> 4;
  // wave index in a scalar register: everything derived from it (slots, their
  // activity) is wave-uniform, so the MFMA guards are scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kt = g.kt;
  const int tau0 = tchunk * TS, ns = min(TS, g.Lt - tau0);

  for (int i = tid; i < NBUF * C::TILE_BYTES / 16; i += NW * 64)
    reinterpret_cast<uint4*>(&tile[0][0])[i] = uint4{0u, 0u, 0u, 0u};
  for (int i = tid; i < ns; i += NW * 64) {
    const int blob = ((tau0 + i) * g.nby + tg.by) * g.nbx + tg.bx;
    s_beg[i] = p.cell_ptr[blob * BLOB_CELLS];
    s_cnt[i] = p.cell_ptr[(blob + 1) * BLOB_CELLS] - s_beg[i];
    s_done[i] = 0;
  }
  __syncthreads();

  const int ybase = 4 * tg.by + quad, xbase = 4 * tg.bx;
  int roff[C::NCP][2], toff[C::NTP];
#pragma unroll
  for (int c = 0; c < C::NCP; ++c) {
    roff[c][0] = row_frag_off<T>(c, lane, 0);
    roff[c][1] = row_frag_off<T>(c, lane, 1);
  }
#pragma unroll
  for (int dt = 0; dt < C::NTP; ++dt) toff[dt] = tr_frag_off(dt, lane);
  // B fragment of Q for chunk step cc of the query row in qlds: row r16, 16-byte
  // chunk c stored at chunk position c ^ r16 (mod QCH) of its QROW-byte row
  auto q_frag = [&](Frag<T>& f, int slot, int cc) {
    const char* base = qlds[slot] + r16 * QROW;
    const int ch0 = (cc * 32 + quad * 8) * (int)sizeof(T) / 16;
    if constexpr (sizeof(T) == 2) {
      const uint4 u = *reinterpret_cast<const uint4*>(base + ((ch0 ^ r16) % QCH) * 16);
      __builtin_memcpy(&f.v, &u, 16);
    } else {
      const float4 a = *reinterpret_cast<const float4*>(base + ((ch0 ^ r16) % QCH) * 16);
      const float4 b = *reinterpret_cast<const float4*>(base + (((ch0 + 1) ^ r16) % QCH) * 16);
      f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
      f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    }
  };
  // Token ids of row tile (slice i, tile r): 16 scalar loads (rows past the slice
  // repeat its first query); the slice's start-cell boundaries likewise.
  // (LDS values that are the same in every lane go through readfirstlane so the
  // compiler addresses with them on the scalar unit: scalar loads keep the vector
  // memory counter for the direct loads alone)
  auto tile_ids = [&](int i, int r, int* ids) {
    cint_ptr pp = (cint_ptr)p.perm + __builtin_amdgcn_readfirstlane(s_beg[i]) + r * 16;
    const int last = __builtin_amdgcn_readfirstlane(s_cnt[i]) - r * 16 - 1;
#pragma unroll
    for (int j = 0; j < 16; ++j) ids[j] = pp[j <= last ? j : 0];
  };
  // Direct loads of the 16 Q rows of (slice i, tile r) into slot sl's LDS area
  // (QROWS_PER_LOAD rows per 1 KB load): each lane fetches the logical chunk that
  // lands at its slot of the swizzled row.
  auto issue_q = [&](int sl, int i, int r) {
    int ids[16];
    tile_ids(i, r, ids);
#pragma unroll
    for (int j = 0; j < 16 / QROWS_PER_LOAD; ++j) {
      const int row = j * QROWS_PER_LOAD + lane / QCH, pc = lane % QCH;
      int id = ids[0];
#pragma unroll
      for (int m = 1; m < 16; ++m) id = (row == m) ? ids[m] : id;
      const int chunk = (pc ^ row) % QCH;
      const T* gp = q + ((size_t)id * g.H + h) * D + chunk * (16 / (int)sizeof(T));
      dma16(gp, qlds[sl] + j * 1024);
    }
  };

  f32x4_t oacc[NS][C::NT];
  f32x4_t sacc[NS][C::NBMAX];  // S^T, then (after the K phases) P
  float m_run[NS], l_run[NS];
  int qsy[NS], qsx[NS], qn[NS];
  bool qv[NS];

  for (;;) {
    // ---- schedule this pass (thread 0)
    if (tid == 0) {
      int free_at[FT_SLOTS];
      for (int sl = 0; sl < NW * NS; ++sl) {
        free_at[sl] = -(1 << 29);
        s_qlen[sl] = 0;
      }
      int left = 0, nf = 0, fmax = -1;
      for (int i = 0; i < ns; ++i) {
        const int tau = tau0 + i, ntiles = (s_cnt[i] + 15) >> 4;
        while (s_done[i] < ntiles) {
          int best = -1;
          for (int sl = 0; sl < NW * NS; ++sl)
            if (free_at[sl] <= tau && s_qlen[sl] < FT_MAXQ && (best < 0 || free_at[sl] < free_at[best])) best = sl;
          if (best < 0) break;
          s_qtau[best][s_qlen[best]] = (short)i;
          s_qr[best][s_qlen[best]] = (short)s_done[i];
          ++s_qlen[best];
          free_at[best] = tau + kt + GAP;
          ++s_done[i];
          // the slice's frames, plus GAP frames before it so that a slot's Q loads
          // always come PD steps after its previous row tile's last read
          for (int f = max(max(tau - GAP, 0), fmax + 1); f < tau + kt; ++f) s_frames[nf++] = (short)f;
          fmax = max(fmax, tau + kt - 1);
        }
        left += ntiles - s_done[i];
      }
      s_nf = nf;
      s_left = left;
    }
    __syncthreads();
    const int nf = __builtin_amdgcn_readfirstlane(s_nf);
    if (nf == 0) break;

    int qhead[NS], qnext[NS];  // entry in flight / next entry whose Q rows are not requested yet
    bool act[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      qhead[s] = 0;
      qnext[s] = 0;
      act[s] = false;
    }

    const int nsteps = nf * NPH2;
    const int my_loads = (C::NLOADS - wave + NW - 1) / NW;
    // request the Q rows of this wave's row tiles that start at frame fq (issued just
    // before the tile loads of that frame's first step, so the same wait covers them)
    auto issue_q_for_frame = [&](int fq) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int sl = wave * NS + s;
        const int qlen = __builtin_amdgcn_readfirstlane(s_qlen[sl]);
        if (qnext[s] < qlen) {
          const int qi = __builtin_amdgcn_readfirstlane(s_qtau[sl][qnext[s]]);
          if (tau0 + qi == fq) {
            issue_q(sl, qi, __builtin_amdgcn_readfirstlane(s_qr[sl][qnext[s]]));
            ++qnext[s];
          }
        }
      }
    };
    auto issue_step = [&](int st) {
      const int ph = st % NPH2;
      const int fs = __builtin_amdgcn_readfirstlane(s_frames[st / NPH2]);
      if (ph == 0) issue_q_for_frame(fs);
      issue_tile<T, D>(tile[st % NBUF], ph < C::NPH ? k : v, g, tg, fs, (ph % C::NPH) * C::PW, h, wave, NW, lane);
    };
    for (int st = 0; st < PD && st < nsteps; ++st) issue_step(st);
    wait_vmcnt(0);
    __syncthreads();

    for (int fi = 0; fi < nf; ++fi) {
      const int f = __builtin_amdgcn_readfirstlane(s_frames[fi]);
      // ---- slots whose next row tile starts at this frame (its Q rows have landed)
      int nact = 0;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int sl = wave * NS + s;
        const int qlen = __builtin_amdgcn_readfirstlane(s_qlen[sl]);
        const int hi_ = qhead[s] < qlen ? __builtin_amdgcn_readfirstlane(s_qtau[sl][qhead[s]]) : -(1 << 29);
        if (!act[s] && tau0 + hi_ == f) {
          const int i = hi_, r = __builtin_amdgcn_readfirstlane(s_qr[sl][qhead[s]]);
          int ids[16];
          tile_ids(i, r, ids);
          int id = ids[0];
#pragma unroll
          for (int m = 1; m < 16; ++m) id = (r16 == m) ? ids[m] : id;
          qn[s] = id;
          qv[s] = r * 16 + r16 < __builtin_amdgcn_readfirstlane(s_cnt[i]);
          // start cell of this lane's query: the slice's queries are sorted by cell
          const int blob = (f * g.nby + tg.by) * g.nbx + tg.bx;
          const int pos = __builtin_amdgcn_readfirstlane(s_beg[i]) + r * 16 + r16;
          int cell = 0;
          cint_ptr cp = (cint_ptr)p.cell_ptr + blob * BLOB_CELLS;
#pragma unroll
          for (int c = 1; c < BLOB_CELLS; ++c) cell = (cp[c] <= pos) ? c : cell;
          qsy[s] = qv[s] ? 4 * tg.by + (cell >> 2) : -(1 << 29);
          qsx[s] = 4 * tg.bx + (cell & 3);
#pragma unroll
          for (int t = 0; t < C::NT; ++t) oacc[s][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          m_run[s] = -INFINITY;
          l_run[s] = 0.f;
          act[s] = true;
        }
        nact += act[s];
      }

      static_for<0, NPH2>([&](auto PHC) {
        constexpr int ph = decltype(PHC)::value;
        const int st = fi * NPH2 + ph;
        if (st + PD < nsteps) issue_step(st + PD);
        const char* tb = tile[st % NBUF];
        if (nact > 0) {
          if constexpr (ph < C::NPH) {
            // ---- S^T += K Q^T over this column phase, one K fragment for every active slot
            if constexpr (ph == 0) {
#pragma unroll
              for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int b = 0; b < C::NBMAX; ++b) sacc[s][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int c = 0; c < C::NCP; ++c) {
              Frag<T> qb[NS];
#pragma unroll
              for (int s = 0; s < NS; ++s)
                if (act[s]) q_frag(qb[s], wave * NS + s, ph * C::NCP + c);
#pragma unroll
              for (int b = 0; b < C::NBMAX; ++b) {
                if (b < tg.nb) {
                  Frag<T> a;
                  lds_row(a, tb + b * 2048, roff[c]);
#pragma unroll
                  for (int s = 0; s < NS; ++s)
                    if (act[s]) sacc[s][b] = mma(a, qb[s], sacc[s][b]);
                }
              }
            }
            if constexpr (ph == C::NPH - 1) {
              // ---- mask to each query's window, online softmax, P kept in sacc
#pragma unroll
              for (int s = 0; s < NS; ++s) {
                if (!act[s]) continue;
                float cm = -INFINITY;
#pragma unroll
                for (int b = 0; b < C::NBMAX; ++b) {
                  const bool yok = b < tg.nb && (unsigned)(ybase + 4 * (b / NBX) - qsy[s]) < (unsigned)g.ky;
#pragma unroll
                  for (int i = 0; i < 4; ++i) {
                    const bool ok = yok && (unsigned)(xbase + 4 * (b % NBX) + i - qsx[s]) < (unsigned)g.kx;
                    const float x = ok ? sacc[s][b][i] * sl2 : -INFINITY;
                    sacc[s][b][i] = x;
                    cm = fmaxf(cm, x);
                  }
                }
                cm = quad_max(cm);
                const float mn = fmaxf(m_run[s], cm);
                const float mref = (mn == -INFINITY) ? 0.f : mn;
                const float alpha = __builtin_amdgcn_exp2f(m_run[s] - mref);
                float ps = 0.f;
#pragma unroll
                for (int b = 0; b < C::NBMAX; ++b)
#pragma unroll
                  for (int i = 0; i < 4; ++i) {
                    sacc[s][b][i] = __builtin_amdgcn_exp2f(sacc[s][b][i] - mref);
                    ps += sacc[s][b][i];
                  }
                ps = quad_sum(ps);
                l_run[s] = l_run[s] * alpha + ps;
                m_run[s] = mn;
#pragma unroll
                for (int t = 0; t < C::NT; ++t) oacc[s][t] *= alpha;
              }
            }
          } else {
            // ---- O^T += V^T P^T over this column phase
            constexpr int vph = ph - C::NPH;
            const int npair = (tg.nb + 1) >> 1;
#pragma unroll
            for (int c = 0; c < C::NPAIR; ++c) {
              if (c < npair) {
                Frag<T> pf[NS];  // P of key blocks 2c, 2c+1 (slot j < 4: block 2c)
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                  float pr[8];
#pragma unroll
                  for (int i = 0; i < 4; ++i) {
                    pr[i] = sacc[s][2 * c][i];
                    pr[i + 4] = (2 * c + 1 < C::NBMAX) ? sacc[s][2 * c + 1][i] : 0.f;
                  }
                  set_frag(pf[s], pr);
                }
#pragma unroll
                for (int dt = 0; dt < C::NTP; ++dt) {
                  Frag<T> a;
                  lds_tr(a, tb + (2 * c) * 2048, toff, dt, lane);
#pragma unroll
                  for (int s = 0; s < NS; ++s)
                    if (act[s]) oacc[s][vph * C::NTP + dt] = mma(a, pf[s], oacc[s][vph * C::NTP + dt]);
                }
              }
            }
            if constexpr (ph == NPH2 - 1) {
              // ---- slots whose slice ends at this frame: normalise, write, advance.
              // (The stores join the vmcnt count; the waits below only ever allow the
              // ring's later loads outstanding, so stores in flight make them stricter.)
#pragma unroll
              for (int s = 0; s < NS; ++s) {
                const int sl = wave * NS + s;
                if (act[s] && f == tau0 + __builtin_amdgcn_readfirstlane(s_qtau[sl][qhead[s]]) + kt - 1) {
                  if (qv[s]) {
                    const float inv = 1.f / l_run[s];
                    T* orow = out + ((size_t)qn[s] * g.H + h) * D;
#pragma unroll
                    for (int t = 0; t < C::NT; ++t)
                      store4(orow + t * 16 + quad * 4, oacc[s][t][0] * inv, oacc[s][t][1] * inv,
                             oacc[s][t][2] * inv, oacc[s][t][3] * inv);
                    if (quad == 0) lse[(size_t)h * g.N + qn[s]] = (m_run[s] + log2f(l_run[s])) * LN2;
                  }
                  act[s] = false;
                  ++qhead[s];
                }
              }
            }
          }
        }
        // step st + 1 (tile and any Q rows requested with it) must have landed; the
        // loads of steps st + 2 .. st + PD may stay in flight
        wait_vmcnt(my_loads * max(min(PD, nsteps - 1 - st) - 1, 0));
        lds_barrier();
      });
    }
    if (__builtin_amdgcn_readfirstlane(s_left) == 0) break;
    __syncthreads();
  }
}

// The frame-tiled kernels take windows whose key tile is at most 3 x 3 blocks of
// 4 x 4 keys, rows of at most 256 bytes (the query rows of all slots live in LDS)
// and kt <= 32 (a pass lists at most TUBE_TS + kt frames).
bool tube_eligible(const Geom& g, int dtype, int D) {
  return g.ky <= 9 && g.kx <= 9 && g.kt <= 32 && D * (dtype == 1 ? 2 : 4) <= 256;
}

template <typename T, int D>
static hipError_t fwd_tube_impl(const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s) {
  const int TS = TUBE_TS;
  const long long total = (long long)g.nby * g.nbx * ((g.Lt + TS - 1) / TS) * g.H;
  dim3 grid((unsigned)total, 1);
  const int nbx = (4 + g.kx - 1 + 3) / 4;
  if (nbx <= 2)
    k_forward_ft<T, D, 2><<<grid, 256, 0, s>>>((const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse_out, g,
                                               p, a.scale * LOG2E, TS);
  else
    k_forward_ft<T, D, 3><<<grid, 256, 0, s>>>((const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse_out, g,
                                               p, a.scale * LOG2E, TS);
  return hipGetLastError();
}

hipError_t launch_forward_tube(int dtype, int D, const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s) {
  if (dtype == 1) return D == 64 ? fwd_tube_impl<u16, 64>(a, g, p, s) : fwd_tube_impl<u16, 128>(a, g, p, s);
  return fwd_tube_impl<float, 64>(a, g, p, s);  // fp32 rows of 128 elements take the per-group kernels
}

}  // namespace dsa3d
