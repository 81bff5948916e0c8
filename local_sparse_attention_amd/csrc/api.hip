// C ABI entry points (include/dsa3d.h): argument checks, workspace carving and the
// launch sequence on the caller's stream.  Everything here runs on the host.
#include <math.h>
#include <stdlib.h>

#include "dsa3d.h"
#include "internal.hpp"

using namespace dsa3d;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool odd_in(int k, int G) { return k >= 1 && (k & 1) == 1 && k <= G; }

int check_geom(int F, int Hp, int Wp, int heads, int kt, int ky, int kx) {
  if (F < 1 || Hp < 1 || Wp < 1 || heads < 1 || heads > 65535) return DSA3D_ERR_GRID;
  const long long N = (long long)F * Hp * Wp;
  if (N >= (1LL << 30)) return DSA3D_ERR_GRID;
  if (!odd_in(kt, F) || !odd_in(ky, Hp) || !odd_in(kx, Wp)) return DSA3D_ERR_WINDOW;
  // start cells are numbered blob by blob (1 x 4 x 4 cells each) in 32-bit sort keys
  const long long blobs = (long long)(F - kt + 1) * ((Hp - ky + 1 + 3) / 4) * ((Wp - kx + 1 + 3) / 4);
  if (blobs * 16 >= (1LL << 31)) return DSA3D_ERR_GRID;
  return DSA3D_OK;
}

int check_common(int F, int Hp, int Wp, int heads, int head_dim, int kt, int ky, int kx, float scale, int dtype) {
  if (dtype != DSA3D_F32 && dtype != DSA3D_BF16) return DSA3D_ERR_DTYPE;
  if (head_dim != 64 && head_dim != 128) return DSA3D_ERR_HEAD_DIM;
  const int gs = check_geom(F, Hp, Wp, heads, kt, ky, kx);
  if (gs != DSA3D_OK) return gs;
  if (!isfinite(scale)) return DSA3D_ERR_SCALE;
  return DSA3D_OK;
}

// Per-head offsets in one set of launches: the bucketing of every head at once
// (g.ph = heads: sort keys head-major, every list one block per head) when the
// frame-sweeping kernels apply and the head-major counts stay inside int32.
bool heads_batchable(const Geom& g) {
  return g.H > 1 && qs_geometry(g) && kv_items_geometry(g) && (long long)g.N * g.H < (1LL << 31) &&
         (long long)g.keyspace * g.H < (1LL << 31);
}

}  // namespace

namespace dsa3d {

int check_forward_args(const void* q, const void* k, const void* v, const int32_t* offsets, int F, int Hp, int Wp,
                       int heads, int head_dim, int kt, int ky, int kx, float scale, int dtype, const void* out,
                       const float* lse) {
  if (!q || !k || !v || !offsets || !out || !lse) return DSA3D_ERR_NULL;
  const int st = check_common(F, Hp, Wp, heads, head_dim, kt, ky, kx, scale, dtype);
  if (st != DSA3D_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(offsets) & 3u))
    return DSA3D_ERR_ALIGN;
  return DSA3D_OK;
}

int run_forward(const void* q, const void* k, const void* v, const int32_t* offsets, const Geom& g, int head_dim,
                float scale, int dtype, void* out, float* lse, char* workspace, hipStream_t stream, unsigned flags,
                const hipEvent_t* events) {
  Prep p;
  workspace_layout(g, false, workspace, &p);
  if (events) (void)hipEventRecord(events[0], stream);
  const bool qs = !(flags & DSA3D_FLAG_GENERIC_KERNELS) && fwd_qs_eligible(g, dtype, head_dim);
  if (launch_prep(offsets, g, p, qs, QS_SLOTS_FWD, stream) != hipSuccess) return DSA3D_ERR_LAUNCH;
  if (events) (void)hipEventRecord(events[1], stream);
  AttnArgs a = {};
  a.q = q; a.k = k; a.v = v;
  a.out = out; a.lse_out = lse;
  a.scale = scale;
  const hipError_t e = qs ? launch_forward_qs(head_dim, a, g, p, stream)
                          : launch_forward_v1(dtype, head_dim, a, g, p, stream);
  if (events) (void)hipEventRecord(events[2], stream);
  return e == hipSuccess ? DSA3D_OK : DSA3D_ERR_LAUNCH;
}

int check_backward_args(const void* q, const void* k, const void* v, const int32_t* offsets, const void* out,
                        const float* lse, const void* dout, int F, int Hp, int Wp, int heads, int head_dim, int kt,
                        int ky, int kx, float scale, int dtype, const void* dq, const void* dk, const void* dv) {
  if (!q || !k || !v || !offsets || !out || !lse || !dout || !dq || !dk || !dv) return DSA3D_ERR_NULL;
  const int st = check_common(F, Hp, Wp, heads, head_dim, kt, ky, kx, scale, dtype);
  if (st != DSA3D_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || (reinterpret_cast<uintptr_t>(lse) & 3u) ||
      (reinterpret_cast<uintptr_t>(offsets) & 3u))
    return DSA3D_ERR_ALIGN;
  return DSA3D_OK;
}

static AttnArgs backward_args(const void* q, const void* k, const void* v, const void* out, const float* lse,
                              const void* dout, float scale, void* dq, void* dk, void* dv) {
  AttnArgs a = {};
  a.q = q; a.k = k; a.v = v;
  a.o = out; a.dout = dout; a.lse = lse;
  a.out = dq; a.dk = dk; a.dv = dv;
  a.scale = scale;
  return a;
}

int run_backward(const void* q, const void* k, const void* v, const int32_t* offsets, const void* out,
                 const float* lse, const void* dout, const Geom& g, int head_dim, float scale, int dtype, void* dq,
                 void* dk, void* dv, char* workspace, hipStream_t stream, unsigned flags, const hipEvent_t* events,
                 bool delta_ready) {
  Prep p;
  workspace_layout(g, true, workspace, &p);
  // with DSA3D_FLAG_REUSE_PREP the workspace holds what run_forward built for the same
  // offsets and geometry: the window starts and buckets always, the query-side schedules
  // when the frame-sweeping forward ran
  const bool reuse = (flags & DSA3D_FLAG_REUSE_PREP) != 0;
  if (events) (void)hipEventRecord(events[0], stream);
  const bool kv_tube = !(flags & DSA3D_FLAG_GENERIC_KERNELS) && dkdv_tube_eligible(g, dtype, head_dim);
  const bool qs = !(flags & DSA3D_FLAG_GENERIC_KERNELS) && dq_qs_eligible(g, dtype, head_dim);
  const bool sched_built = reuse && fwd_qs_eligible(g, dtype, head_dim);
  if (!reuse && launch_prep(offsets, g, p, qs, QS_SLOTS, stream) != hipSuccess) return DSA3D_ERR_LAUNCH;
  if (kv_tube && launch_kv_items(g, p, stream) != hipSuccess) return DSA3D_ERR_LAUNCH;
  // dQ holds fewer row tiles in flight than the forward: with the forward's tiles in the
  // workspace only the pass schedules are built again, for dQ's slots
  if (qs && reuse && !sched_built && launch_qsched(g, p, QS_SLOTS, stream) != hipSuccess) return DSA3D_ERR_LAUNCH;
  if (qs && sched_built && launch_sched_fill(g, p, QS_SLOTS, stream) != hipSuccess) return DSA3D_ERR_LAUNCH;
  const AttnArgs a = backward_args(q, k, v, out, lse, dout, scale, dq, dk, dv);
  // Delta = rowsum(dO * O) of every head for both kernels (the per-group dQ kernel makes
  // its own head's)
  if (qs && !delta_ready && launch_delta(head_dim, a, g, p, stream) != hipSuccess) return DSA3D_ERR_LAUNCH;
  if (events) (void)hipEventRecord(events[1], stream);
  if (qs ? launch_dq_qs(head_dim, a, g, p, stream) != hipSuccess
         : launch_backward_dq_v1(dtype, head_dim, a, g, p, stream) != hipSuccess)
    return DSA3D_ERR_LAUNCH;
  if (events) (void)hipEventRecord(events[2], stream);
  const hipError_t e = kv_tube ? launch_dkdv_tube(head_dim, a, g, p, stream)
                               : launch_backward_dkdv_v1(dtype, head_dim, a, g, p, stream);
  if (events) (void)hipEventRecord(events[3], stream);
  return e == hipSuccess ? DSA3D_OK : DSA3D_ERR_LAUNCH;
}

}  // namespace dsa3d

extern "C" {

size_t dsa3d_workspace_bytes(int F, int Hp, int Wp, int heads, int kt, int ky, int kx, int backward) {
  if (check_geom(F, Hp, Wp, heads, kt, ky, kx) != DSA3D_OK) return 0;
  const Geom g = make_geom(F, Hp, Wp, heads, kt, ky, kx);
  return workspace_layout(g, backward != 0, nullptr, nullptr);
}

size_t dsa3d_workspace_bytes_heads(int F, int Hp, int Wp, int heads, int kt, int ky, int kx, int backward) {
  if (check_geom(F, Hp, Wp, heads, kt, ky, kx) != DSA3D_OK) return 0;
  Geom g = make_geom(F, Hp, Wp, heads, kt, ky, kx);
  if (heads_batchable(g)) g.ph = heads;
  return workspace_layout(g, backward != 0, nullptr, nullptr);
}

int dsa3d_window_starts(const int32_t* offsets, int F, int Hp, int Wp, int kt, int ky, int kx, int32_t* starts,
                        hipStream_t stream) {
  if (!offsets || !starts) return DSA3D_ERR_NULL;
  const int gs = check_geom(F, Hp, Wp, 1, kt, ky, kx);
  if (gs != DSA3D_OK) return gs;
  if ((reinterpret_cast<uintptr_t>(offsets) & 3u) || (reinterpret_cast<uintptr_t>(starts) & 3u))
    return DSA3D_ERR_ALIGN;
  const Geom g = make_geom(F, Hp, Wp, 1, kt, ky, kx);
  return launch_window_starts(offsets, g, starts, stream) == hipSuccess ? DSA3D_OK : DSA3D_ERR_LAUNCH;
}

int dsa3d_forward_ex(const void* q, const void* k, const void* v, const int32_t* offsets, int F, int Hp, int Wp,
                     int heads, int head_dim, int kt, int ky, int kx, float scale, int dtype, void* out, float* lse,
                     void* workspace, size_t workspace_bytes, hipStream_t stream, unsigned flags,
                     const hipEvent_t* events) {
  if (!workspace) return DSA3D_ERR_NULL;
  const int st = check_forward_args(q, k, v, offsets, F, Hp, Wp, heads, head_dim, kt, ky, kx, scale, dtype, out, lse);
  if (st != DSA3D_OK) return st;
  if (flags & ~(unsigned)DSA3D_FLAG_GENERIC_KERNELS) return DSA3D_ERR_FLAGS;
  if (!aligned16(workspace)) return DSA3D_ERR_ALIGN;
  const Geom g = make_geom(F, Hp, Wp, heads, kt, ky, kx);
  if (workspace_bytes < workspace_layout(g, false, nullptr, nullptr)) return DSA3D_ERR_WORKSPACE;
  return run_forward(q, k, v, offsets, g, head_dim, scale, dtype, out, lse, static_cast<char*>(workspace), stream,
                     flags, events);
}

int dsa3d_forward(const void* q, const void* k, const void* v, const int32_t* offsets, int F, int Hp, int Wp,
                  int heads, int head_dim, int kt, int ky, int kx, float scale, int dtype, void* out, float* lse,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return dsa3d_forward_ex(q, k, v, offsets, F, Hp, Wp, heads, head_dim, kt, ky, kx, scale, dtype, out, lse, workspace,
                          workspace_bytes, stream, 0u, nullptr);
}

int dsa3d_backward_ex(const void* q, const void* k, const void* v, const int32_t* offsets, const void* out,
                      const float* lse, const void* dout, int F, int Hp, int Wp, int heads, int head_dim, int kt,
                      int ky, int kx, float scale, int dtype, void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes, hipStream_t stream, unsigned flags,
                      const hipEvent_t* events) {
  if (!workspace) return DSA3D_ERR_NULL;
  const int st = check_backward_args(q, k, v, offsets, out, lse, dout, F, Hp, Wp, heads, head_dim, kt, ky, kx, scale,
                                     dtype, dq, dk, dv);
  if (st != DSA3D_OK) return st;
  if (flags & ~(unsigned)(DSA3D_FLAG_GENERIC_KERNELS | DSA3D_FLAG_REUSE_PREP)) return DSA3D_ERR_FLAGS;
  if (!aligned16(workspace)) return DSA3D_ERR_ALIGN;
  const Geom g = make_geom(F, Hp, Wp, heads, kt, ky, kx);
  if (workspace_bytes < workspace_layout(g, true, nullptr, nullptr)) return DSA3D_ERR_WORKSPACE;
  return run_backward(q, k, v, offsets, out, lse, dout, g, head_dim, scale, dtype, dq, dk, dv,
                      static_cast<char*>(workspace), stream, flags, events, false);
}

int dsa3d_backward(const void* q, const void* k, const void* v, const int32_t* offsets, const void* out,
                   const float* lse, const void* dout, int F, int Hp, int Wp, int heads, int head_dim, int kt,
                   int ky, int kx, float scale, int dtype, void* dq, void* dk, void* dv, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  return dsa3d_backward_ex(q, k, v, offsets, out, lse, dout, F, Hp, Wp, heads, head_dim, kt, ky, kx, scale, dtype, dq,
                           dk, dv, workspace, workspace_bytes, stream, 0u, nullptr);
}

int dsa3d_forward_heads(const void* q, const void* k, const void* v, const int32_t* offsets, int F, int Hp, int Wp,
                        int heads, int head_dim, int kt, int ky, int kx, float scale, int dtype, void* out, float* lse,
                        void* workspace, size_t workspace_bytes, hipStream_t stream, unsigned flags) {
  if (!workspace) return DSA3D_ERR_NULL;
  const int st = check_forward_args(q, k, v, offsets, F, Hp, Wp, heads, head_dim, kt, ky, kx, scale, dtype, out, lse);
  if (st != DSA3D_OK) return st;
  if (flags & ~(unsigned)DSA3D_FLAG_GENERIC_KERNELS) return DSA3D_ERR_FLAGS;
  if (!aligned16(workspace)) return DSA3D_ERR_ALIGN;
  Geom g = make_geom(F, Hp, Wp, heads, kt, ky, kx);
  if (workspace_bytes < workspace_layout(g, false, nullptr, nullptr)) return DSA3D_ERR_WORKSPACE;
  // every head at once when the workspace holds the bucketing of all heads
  Geom gb = g;
  gb.ph = heads;
  if (!(flags & DSA3D_FLAG_GENERIC_KERNELS) && heads_batchable(g) && fwd_qs_eligible(g, dtype, head_dim) &&
      workspace_bytes >= workspace_layout(gb, false, nullptr, nullptr))
    return run_forward(q, k, v, offsets, gb, head_dim, scale, dtype, out, lse, static_cast<char*>(workspace), stream,
                       flags, nullptr);
  // else one head at a time: its own window starts, buckets and work lists (the
  // workspace is reused in stream order), then the attention kernels on that head only
  for (int h = 0; h < heads; ++h) {
    g.h0 = h;
    g.nh = 1;
    const int r = run_forward(q, k, v, offsets + (size_t)3 * g.N * h, g, head_dim, scale, dtype, out, lse,
                              static_cast<char*>(workspace), stream, flags, nullptr);
    if (r != DSA3D_OK) return r;
  }
  return DSA3D_OK;
}

int dsa3d_backward_heads(const void* q, const void* k, const void* v, const int32_t* offsets, const void* out,
                         const float* lse, const void* dout, int F, int Hp, int Wp, int heads, int head_dim, int kt,
                         int ky, int kx, float scale, int dtype, void* dq, void* dk, void* dv, void* workspace,
                         size_t workspace_bytes, hipStream_t stream, unsigned flags) {
  if (!workspace) return DSA3D_ERR_NULL;
  const int st = check_backward_args(q, k, v, offsets, out, lse, dout, F, Hp, Wp, heads, head_dim, kt, ky, kx, scale,
                                     dtype, dq, dk, dv);
  if (st != DSA3D_OK) return st;
  if (flags & ~(unsigned)(DSA3D_FLAG_GENERIC_KERNELS | DSA3D_FLAG_REUSE_PREP)) return DSA3D_ERR_FLAGS;
  if (!aligned16(workspace)) return DSA3D_ERR_ALIGN;
  Geom g = make_geom(F, Hp, Wp, heads, kt, ky, kx);
  if (workspace_bytes < workspace_layout(g, true, nullptr, nullptr)) return DSA3D_ERR_WORKSPACE;
  Geom gb = g;
  gb.ph = heads;
  if (!(flags & DSA3D_FLAG_GENERIC_KERNELS) && heads_batchable(g) && dq_qs_eligible(g, dtype, head_dim) &&
      dkdv_tube_eligible(g, dtype, head_dim) && workspace_bytes >= workspace_layout(gb, true, nullptr, nullptr)) {
    // the forward took its batched route with this workspace too when its kernels are
    // the frame-sweeping ones; otherwise it left one head's buckets only
    const unsigned fl = fwd_qs_eligible(g, dtype, head_dim) ? flags : flags & ~(unsigned)DSA3D_FLAG_REUSE_PREP;
    return run_backward(q, k, v, offsets, out, lse, dout, gb, head_dim, scale, dtype, dq, dk, dv,
                        static_cast<char*>(workspace), stream, fl, nullptr, false);
  }
  flags &= ~(unsigned)DSA3D_FLAG_REUSE_PREP;  // one head after the other: each head's buckets are rebuilt
  // Delta of every head once (it does not depend on the offsets)
  const bool qs = !(flags & DSA3D_FLAG_GENERIC_KERNELS) && dq_qs_eligible(g, dtype, head_dim);
  if (qs) {
    Prep p;
    workspace_layout(g, true, static_cast<char*>(workspace), &p);
    const AttnArgs a = backward_args(q, k, v, out, lse, dout, scale, dq, dk, dv);
    if (launch_delta(head_dim, a, g, p, stream) != hipSuccess) return DSA3D_ERR_LAUNCH;
  }
  for (int h = 0; h < heads; ++h) {
    g.h0 = h;
    g.nh = 1;
    const int r = run_backward(q, k, v, offsets + (size_t)3 * g.N * h, out, lse, dout, g, head_dim, scale, dtype, dq,
                               dk, dv, static_cast<char*>(workspace), stream, flags, nullptr, true);
    if (r != DSA3D_OK) return r;
  }
  return DSA3D_OK;
}

const char* dsa3d_status_string(int status) {
  switch (status) {
    case DSA3D_OK: return "ok";
    case DSA3D_ERR_NULL: return "a required pointer is null";
    case DSA3D_ERR_DTYPE: return "dtype must be DSA3D_F32 (0) or DSA3D_BF16 (1)";
    case DSA3D_ERR_HEAD_DIM: return "head_dim must be 64 or 128";
    case DSA3D_ERR_GRID: return "grid must be >= 1 per axis with N < 2^30 (and < 2^27 blobs of start cells), and 1 <= heads <= 65535";
    case DSA3D_ERR_WINDOW: return "each window dimension must be odd, >= 1 and not larger than the grid";
    case DSA3D_ERR_ALIGN: return "tensors and workspace must be 16-byte aligned (lse, offsets 4-byte)";
    case DSA3D_ERR_WORKSPACE: return "workspace is smaller than dsa3d_workspace_bytes()";
    case DSA3D_ERR_LAUNCH: return "a kernel launch failed";
    case DSA3D_ERR_SCALE: return "scale must be finite";
    case DSA3D_ERR_FLAGS: return "unknown bits in flags";
    case DSA3D_ERR_MODE: return "mode must be DSA3D_SAMPLE_BOX (0) or DSA3D_SAMPLE_FREE (1)";
    case DSA3D_ERR_LAYOUT: return "offset strides must be >= 0 and not overlap (box mode: stride_sample 0)";
    case DSA3D_ERR_SCRATCH: return "the geometry needs more scratch than the static array holds (DSA3D_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
