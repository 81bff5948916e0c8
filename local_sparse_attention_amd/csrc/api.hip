// C ABI entry points (include/dsa3d.h): argument checks, workspace carving and the
// launch sequence on the caller's stream.  Everything here runs on the host.
#include <math.h>
#include <stdlib.h>

#include "dsa3d.h"
#include "internal.hpp"

using namespace dsa3d;

namespace {

// Set DSA3D_GENERIC_KERNELS=1 to run the per-group kernels for every geometry
// (used by the tests to cover both kernel families on the same inputs).
bool generic_only() {
  const char* e = getenv("DSA3D_GENERIC_KERNELS");
  return e && e[0] == '1';
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool odd_in(int k, int G) { return k >= 1 && (k & 1) == 1 && k <= G; }

int check_geom(int F, int Hp, int Wp, int heads, int kt, int ky, int kx) {
  if (F < 1 || Hp < 1 || Wp < 1 || heads < 1 || heads > 65535) return DSA3D_ERR_GRID;
  const long long N = (long long)F * Hp * Wp;
  if (N >= (1LL << 30)) return DSA3D_ERR_GRID;
  if (!odd_in(kt, F) || !odd_in(ky, Hp) || !odd_in(kx, Wp)) return DSA3D_ERR_WINDOW;
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

}  // namespace

extern "C" {

size_t dsa3d_workspace_bytes(int F, int Hp, int Wp, int heads, int kt, int ky, int kx, int backward) {
  if (check_geom(F, Hp, Wp, heads, kt, ky, kx) != DSA3D_OK) return 0;
  const Geom g = make_geom(F, Hp, Wp, heads, kt, ky, kx);
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

int dsa3d_forward_timed(const void* q, const void* k, const void* v, const int32_t* offsets, int F, int Hp, int Wp,
                        int heads, int head_dim, int kt, int ky, int kx, float scale, int dtype, void* out,
                        float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream,
                        const hipEvent_t* events) {
  if (!q || !k || !v || !offsets || !out || !lse || !workspace) return DSA3D_ERR_NULL;
  const int st = check_common(F, Hp, Wp, heads, head_dim, kt, ky, kx, scale, dtype);
  if (st != DSA3D_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(offsets) & 3u))
    return DSA3D_ERR_ALIGN;
  const Geom g = make_geom(F, Hp, Wp, heads, kt, ky, kx);
  if (workspace_bytes < workspace_layout(g, false, nullptr, nullptr)) return DSA3D_ERR_WORKSPACE;
  Prep p;
  workspace_layout(g, false, static_cast<char*>(workspace), &p);
  if (events) hipEventRecord(events[0], stream);
  if (launch_prep(offsets, g, p, stream) != hipSuccess) return DSA3D_ERR_LAUNCH;
  const bool qs = !generic_only() && fwd_qs_eligible(g, dtype, head_dim);
  if (qs && launch_qsched(g, p, stream) != hipSuccess) return DSA3D_ERR_LAUNCH;
  if (events) hipEventRecord(events[1], stream);
  AttnArgs a = {};
  a.q = q; a.k = k; a.v = v;
  a.out = out; a.lse_out = lse;
  a.scale = scale;
  const hipError_t e = qs ? launch_forward_qs(head_dim, a, g, p, stream)
                          : launch_forward_v1(dtype, head_dim, a, g, p, stream);
  if (events) hipEventRecord(events[2], stream);
  return e == hipSuccess ? DSA3D_OK : DSA3D_ERR_LAUNCH;
}

int dsa3d_forward(const void* q, const void* k, const void* v, const int32_t* offsets, int F, int Hp, int Wp,
                  int heads, int head_dim, int kt, int ky, int kx, float scale, int dtype, void* out, float* lse,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return dsa3d_forward_timed(q, k, v, offsets, F, Hp, Wp, heads, head_dim, kt, ky, kx, scale, dtype, out, lse,
                             workspace, workspace_bytes, stream, nullptr);
}

int dsa3d_backward_timed(const void* q, const void* k, const void* v, const int32_t* offsets, const void* out,
                         const float* lse, const void* dout, int F, int Hp, int Wp, int heads, int head_dim,
                         int kt, int ky, int kx, float scale, int dtype, void* dq, void* dk, void* dv,
                         void* workspace, size_t workspace_bytes, hipStream_t stream, const hipEvent_t* events) {
  if (!q || !k || !v || !offsets || !out || !lse || !dout || !dq || !dk || !dv || !workspace) return DSA3D_ERR_NULL;
  const int st = check_common(F, Hp, Wp, heads, head_dim, kt, ky, kx, scale, dtype);
  if (st != DSA3D_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || !aligned16(workspace) || (reinterpret_cast<uintptr_t>(lse) & 3u) ||
      (reinterpret_cast<uintptr_t>(offsets) & 3u))
    return DSA3D_ERR_ALIGN;
  const Geom g = make_geom(F, Hp, Wp, heads, kt, ky, kx);
  if (workspace_bytes < workspace_layout(g, true, nullptr, nullptr)) return DSA3D_ERR_WORKSPACE;
  Prep p;
  workspace_layout(g, true, static_cast<char*>(workspace), &p);
  if (events) hipEventRecord(events[0], stream);
  if (launch_prep(offsets, g, p, stream) != hipSuccess) return DSA3D_ERR_LAUNCH;
  const bool kv_tube = !generic_only() && dkdv_tube_eligible(g, dtype, head_dim);
  const bool qs = !generic_only() && dq_qs_eligible(g, dtype, head_dim);
  if (kv_tube && launch_kv_items(g, p, stream) != hipSuccess) return DSA3D_ERR_LAUNCH;
  if (qs && launch_qsched(g, p, stream) != hipSuccess) return DSA3D_ERR_LAUNCH;
  AttnArgs a = {};
  a.q = q; a.k = k; a.v = v;
  a.o = out; a.dout = dout; a.lse = lse;
  a.out = dq; a.dk = dk; a.dv = dv;
  a.scale = scale;
  // Delta = rowsum(dO * O) for both kernels (the per-group dQ kernel makes its own)
  if (qs && launch_delta(head_dim, a, g, p, stream) != hipSuccess) return DSA3D_ERR_LAUNCH;
  if (events) hipEventRecord(events[1], stream);
  if (qs ? launch_dq_qs(head_dim, a, g, p, stream) != hipSuccess
         : launch_backward_dq_v1(dtype, head_dim, a, g, p, stream) != hipSuccess)
    return DSA3D_ERR_LAUNCH;
  if (events) hipEventRecord(events[2], stream);
  const hipError_t e = kv_tube ? launch_dkdv_tube(head_dim, a, g, p, stream)
                               : launch_backward_dkdv_v1(dtype, head_dim, a, g, p, stream);
  if (events) hipEventRecord(events[3], stream);
  return e == hipSuccess ? DSA3D_OK : DSA3D_ERR_LAUNCH;
}

int dsa3d_backward(const void* q, const void* k, const void* v, const int32_t* offsets, const void* out,
                   const float* lse, const void* dout, int F, int Hp, int Wp, int heads, int head_dim, int kt,
                   int ky, int kx, float scale, int dtype, void* dq, void* dk, void* dv, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  return dsa3d_backward_timed(q, k, v, offsets, out, lse, dout, F, Hp, Wp, heads, head_dim, kt, ky, kx, scale, dtype,
                              dq, dk, dv, workspace, workspace_bytes, stream, nullptr);
}

const char* dsa3d_status_string(int status) {
  switch (status) {
    case DSA3D_OK: return "ok";
    case DSA3D_ERR_NULL: return "a required pointer is null";
    case DSA3D_ERR_DTYPE: return "dtype must be DSA3D_F32 (0) or DSA3D_BF16 (1)";
    case DSA3D_ERR_HEAD_DIM: return "head_dim must be 64 or 128";
    case DSA3D_ERR_GRID: return "grid must be >= 1 per axis with N < 2^30, and 1 <= heads <= 65535";
    case DSA3D_ERR_WINDOW: return "each window dimension must be odd, >= 1 and not larger than the grid";
    case DSA3D_ERR_ALIGN: return "tensors and workspace must be 16-byte aligned (lse, offsets 4-byte)";
    case DSA3D_ERR_WORKSPACE: return "workspace is smaller than dsa3d_workspace_bytes()";
    case DSA3D_ERR_LAUNCH: return "a kernel launch failed";
    case DSA3D_ERR_SCALE: return "scale must be finite";
    default: return "unknown status";
  }
}

}  // extern "C"
