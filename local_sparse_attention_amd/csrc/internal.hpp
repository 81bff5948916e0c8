// Host-side declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"

namespace dsa3d {

// Scratch carved from the caller's workspace (see workspace_layout()).
struct Prep {
  int4* starts;        // [N] (st, sy, sx, 0)
  uint32_t* keys[2];   // [N] sort keys (ping-pong)
  int* vals[2];        // [N] query ids (ping-pong)
  uint32_t* ghist;     // [256 * radix_blocks]
  int* cell_ptr;       // [keyspace + 1]: queries of start cell c are perm[cell_ptr[c] .. cell_ptr[c+1])
  int* goff;           // [nblobs + 1]: groups of blob b are groups[goff[b] .. goff[b+1])
  int2* groups;        // [max_groups]: (first index into perm, query count <= 16)
  int* ngroups;        // [1]
  float* delta;        // [H][N] (backward only)
  // key-centric dK/dV item lists (backward, kv_items_geometry() only)
  int* kv_off;         // [nkb * Lt + 1]: items of key block column kb, slice tau
  int* kv_ids;         // [max_kv_items * KV_Q] query tokens, KV_Q per item
  int2* kv_st;         // [max_kv_items * KV_Q] (sy, sx) window starts
  // query-side frame-sweeping kernels (qs_geometry() only)
  int* qt_off;         // [qs_items + 1]: row tiles of work item w are qt[qt_off[w] .. qt_off[w+1])
  int* qt;             // [max_groups * QT_INTS] row tile descriptors (see qsched.hip)
  int* tq_ids;         // [max_groups * 16] row tile query tokens
  int2* tq_st;         // [max_groups * 16] row tile (sy, sx) window starts
  signed char* tq_dt;  // [max_groups * 16] row's slice minus the tile's first slice
  int* qs_off;         // [qs_items + 1] schedule of work item w at qs + qs_off[w]
  int* qs;             // schedules (see qsched.hip)
  int* perm;           // = the vals buffer the sort ends in
  int radix_blocks;
  int radix_passes;
  int max_groups;
};

constexpr int RADIX_TILE = 4096;

Geom make_geom(int F, int Hp, int Wp, int H, int kt, int ky, int kx);
size_t workspace_layout(const Geom& g, bool backward, char* base, Prep* p);

hipError_t launch_window_starts(const int32_t* off, const Geom& g, int32_t* starts3, hipStream_t s);
hipError_t launch_prep(const int32_t* off, const Geom& g, Prep& p, hipStream_t s);
// In-place exclusive scan of n uint32 values (one workgroup).
hipError_t launch_scan_excl(uint32_t* data, int n, hipStream_t s);

// Key-centric dK/dV: windows whose key blocks reach at most 3 x 3 start blobs
// (ky, kx <= 9) and kt <= 8 (one wave per frame in flight).
inline bool kv_items_geometry(const Geom& g) { return g.kt <= 8 && g.ky <= 9 && g.kx <= 9; }
inline int kv_item_columns(const Geom& g) { return ((g.Hp + 3) / 4) * ((g.Wp + 3) / 4); }
// Items are KV_Q queries of one slice whose start blob can reach the column: every
// query counts for at most 3 x 3 columns.
constexpr int KV_Q = 32;
inline size_t max_kv_items(const Geom& g) {
  return ((size_t)9 * g.N + KV_Q - 1) / KV_Q + (size_t)kv_item_columns(g) * g.Lt + 1;
}

// Query-side schedules: a work item is one start blob column and QS_TS slices;
// QS_SLOTS row tiles in flight, at most QS_MAXT per pass.  A row tile holds the
// queries of one slice, or the leftover queries (fewer than 16 each) of up to
// QS_SPAN consecutive slices; its descriptor is QT_INTS ints.
constexpr int QS_TS = 32, QS_SLOTS = 8, QS_MAXT = 64, QS_SPAN = 3;
constexpr int QT_INTS = 2 + 3 * QS_SPAN;
__host__ __device__ inline bool qs_geometry(const Geom& g) { return g.kt >= 3 && g.kt <= 16 && g.ky <= 9 && g.kx <= 9; }
__host__ __device__ inline int qs_items(const Geom& g) { return g.nby * g.nbx * ((g.Lt + QS_TS - 1) / QS_TS); }
// A pass holds 2 + (frames <= QS_TS + kt - 1) + 4 ints per tile and schedules at
// least one tile; every item has a pass count.
inline size_t qs_ints(const Geom& g, int max_groups) {
  return (size_t)qs_items(g) + (size_t)max_groups * (QS_TS + g.kt + 5);
}
hipError_t launch_qsched(const Geom& g, const Prep& p, hipStream_t s);

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;      // backward: forward output
  const void* dout;   // backward
  const float* lse;   // backward input
  void* out;          // forward: O ; backward: dq
  void* dk;
  void* dv;
  float* lse_out;     // forward output
  float scale;
};

// Per-group kernels: any geometry.
hipError_t launch_forward_v1(int dtype, int D, const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s);
// Query-side frame-sweeping forward (bf16, qs_geometry()): needs launch_qsched().
bool fwd_qs_eligible(const Geom& g, int dtype, int D);
hipError_t launch_forward_qs(int D, const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s);
// Query-side dQ (same eligibility and schedule) and the Delta pass it needs.
bool dq_qs_eligible(const Geom& g, int dtype, int D);
hipError_t launch_delta(int D, const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s);
hipError_t launch_dq_qs(int D, const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s);

// v1 backward pieces: dQ (also writes p.delta) and dK/dV.
hipError_t launch_backward_dq_v1(int dtype, int D, const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s);
hipError_t launch_backward_dkdv_v1(int dtype, int D, const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s);
// Key-centric pipelined dK/dV (bf16): item lists, then the kernel (needs p.delta).
bool dkdv_tube_eligible(const Geom& g, int dtype, int D);
hipError_t launch_kv_items(const Geom& g, const Prep& p, hipStream_t s);
hipError_t launch_dkdv_tube(int D, const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s);

}  // namespace dsa3d
