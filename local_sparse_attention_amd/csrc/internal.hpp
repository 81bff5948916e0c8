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
  int* kv_mask;        // [max_kv_items * KV_Q] mask of the key block in each query's window
  int2* sorted_st;     // [N * ph] (sy, sx) of the window starts in bucket order
  // query-side frame-sweeping kernels (qs_geometry() only)
  int* qt_off;         // [qs_items + 1]: row tiles of work item w are qt[qt_off[w] .. qt_off[w+1])
  int* qt;             // [max_groups * QT_INTS] row tile descriptors (see qsched.hip)
  int* tq_ids;         // [max_groups * 16] row tile query tokens
  int2* tq_st;         // [max_groups * 16] row tile (sy, sx) window starts
  signed char* tq_dt;  // [max_groups * 16] row's slice minus the tile's first slice
  int* qs_off;         // [qs_items + 1] schedule of work item w at qs + qs_off[w]
  int* qs;             // schedules (see qsched.hip)
  int* perm;           // = the vals buffer the sort ends in
  uint32_t* scan_part; // chunk totals of the multi-workgroup scans (scan_part_words(n) each)
  int radix_blocks;    // per head block of the bucketing
  int radix_passes;
  int max_groups;
};

constexpr int RADIX_TILE = 1024;
constexpr int RADIX_RAW_NBS = 64;  // segments of at most this many radix blocks scatter from raw counts
constexpr int SCAN_CHUNK_N = 16384;  // values one scan workgroup takes at a time
inline size_t scan_part_words(size_t n) { return (n + SCAN_CHUNK_N - 1) / SCAN_CHUNK_N + 1; }

Geom make_geom(int F, int Hp, int Wp, int H, int kt, int ky, int kx);
size_t workspace_layout(const Geom& g, bool backward, char* base, Prep* p);

hipError_t launch_window_starts(const int32_t* off, const Geom& g, int32_t* starts3, hipStream_t s);
// The bucketing (window starts, sort, cell_ptr, groups) and, with qs, the query-side
// work lists of the frame-sweeping kernels (launch_qsched() in one pass with it).
hipError_t launch_prep(const int32_t* off, const Geom& g, Prep& p, bool qs, int nslots, hipStream_t s);
// In-place exclusive scan of n uint32 values: one workgroup, or, given part
// (scan_part_words(n) words of scratch) and more than a few chunks, a scan per chunk
// on its own workgroup, a scan of the chunk totals and an add.
hipError_t launch_scan_excl(uint32_t* data, int n, hipStream_t s, uint32_t* part = nullptr);
// Two such scans; one launch of two workgroups when both fit one workgroup each.
hipError_t launch_scan_excl2(uint32_t* a, int na, uint32_t* b, int nb, hipStream_t s, uint32_t* part = nullptr);
// Stable LSD radix sort of nseg segments of seglen (key, value) pairs each, every
// segment on its own (segment i stays at i * seglen ..), 8 bits a pass from bit 0,
// values starting as the item index: ping-pong buffers, ghist holds
// 256 * nseg * ceil(seglen / RADIX_TILE) words.  Returns the buffer index (0 or 1)
// that holds the result, -1 on a launch error.  first_hist_done: ghist already holds
// the first pass's raw counts (k_radix_hist's layout), which the caller may only
// leave for segments of at most RADIX_RAW_NBS blocks.
int radix_sort(uint32_t* keys[2], int* vals[2], uint32_t* ghist, int seglen, int nseg, int passes, hipStream_t s,
               uint32_t* part = nullptr, bool first_hist_done = false);
// cell_ptr[i * keyspace + c] = number of sorted keys before the first key >= c of
// segment i (segments of seglen sorted keys), for i * keyspace + c = 0 .. nseg * keyspace.
// Keys must be below keyspace, except in the last segment, where keys equal to keyspace
// (a sentinel) sort after every cell and are counted by no cell.
hipError_t launch_cell_ptr(const uint32_t* sorted_keys, int seglen, int nseg, int keyspace, int* cell_ptr,
                           hipStream_t s);

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
// The forward holds QS_SLOTS_FWD row tiles in flight (its schedules are built for that many
// slots), dQ QS_SLOTS; pass tables are sized for the larger.
constexpr int QS_SLOTS_FWD = 10, QS_SLOTS_MAX = 10;
constexpr int QT_INTS = 2 + 3 * QS_SPAN;
__host__ __device__ inline bool qs_geometry(const Geom& g) { return g.kt >= 3 && g.kt <= 16 && g.ky <= 9 && g.kx <= 9; }
__host__ __device__ inline int qs_items(const Geom& g) { return g.nby * g.nbx * ((g.Lt + QS_TS - 1) / QS_TS); }
// A pass holds 2 + (frames <= QS_TS + kt - 1) + 4 ints per tile and schedules at
// least one tile; every item has a pass count.
inline size_t qs_ints(const Geom& g, int max_groups) {
  return (size_t)qs_items(g) + (size_t)max_groups * (QS_TS + g.kt + 5);
}
// The work lists after a bucketing: row tile counts (qt_off), then (after their scan)
// the groups and / or row tiles, then the tile rows and the schedules.
// (with blob_groups also the blob group counts into goff, see k_blob_ngroups)
hipError_t launch_qtile_count(const Geom& g, const Prep& p, hipStream_t s, bool blob_groups = false);
hipError_t launch_groups_qtiles(const Geom& g, const Prep& p, bool groups, bool qtiles, hipStream_t s);
hipError_t launch_qsched_rows(const Geom& g, const Prep& p, int nslots, hipStream_t s);
hipError_t launch_sched_fill(const Geom& g, const Prep& p, int nslots, hipStream_t s);
// All of it for a bucketing built earlier.
hipError_t launch_qsched(const Geom& g, const Prep& p, int nslots, hipStream_t s);

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

// Host-side argument checks of the forward (everything but the workspace) and its
// launch sequence once the arguments are known to be valid (api.hip).
int check_forward_args(const void* q, const void* k, const void* v, const int32_t* offsets, int F, int Hp, int Wp,
                       int heads, int head_dim, int kt, int ky, int kx, float scale, int dtype, const void* out,
                       const float* lse);
int run_forward(const void* q, const void* k, const void* v, const int32_t* offsets, const Geom& g, int head_dim,
                float scale, int dtype, void* out, float* lse, char* workspace, hipStream_t stream, unsigned flags,
                const hipEvent_t* events);

int check_backward_args(const void* q, const void* k, const void* v, const int32_t* offsets, const void* out,
                        const float* lse, const void* dout, int F, int Hp, int Wp, int heads, int head_dim, int kt,
                        int ky, int kx, float scale, int dtype, const void* dq, const void* dk, const void* dv);
// delta_ready: Delta of every head is already in the workspace (per-head calls)
int run_backward(const void* q, const void* k, const void* v, const int32_t* offsets, const void* out,
                 const float* lse, const void* dout, const Geom& g, int head_dim, float scale, int dtype, void* dq,
                 void* dk, void* dv, char* workspace, hipStream_t stream, unsigned flags, const hipEvent_t* events,
                 bool delta_ready);

}  // namespace dsa3d
