// dsa3d_forward_static (include/dsa3d.h): the forward with its scratch space in a
// file-scope device array instead of a caller-supplied workspace, for callers that
// cannot allocate device memory.  Everything here runs on the host except the array.
#include <mutex>

#include "dsa3d.h"
#include "internal.hpp"

using namespace dsa3d;

// One copy per GPU the library runs on, held until the process ends.  In host code
// `scratch` is only a host-side stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, per device, and only that address is ever handed to a kernel.
static __device__ __align__(256) char scratch[DSA3D_STATIC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_lock;
char* g_ptr[MAX_DEVICES] = {};

// Device address of the current device's copy of `scratch`, looked up on the first
// call on that device (with it current) and kept; null if the lookup fails.
char* scratch_ptr(int dev) {
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[dev] = static_cast<char*>(p);
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" int dsa3d_forward_static(const void* q, const void* k, const void* v, const int32_t* offsets, int F,
                                    int Hp, int Wp, int heads, int head_dim, int kt, int ky, int kx, float scale,
                                    int dtype, void* out, float* lse, hipStream_t stream) {
  const int st = check_forward_args(q, k, v, offsets, F, Hp, Wp, heads, head_dim, kt, ky, kx, scale, dtype, out, lse);
  if (st != DSA3D_OK) return st;
  const Geom g = make_geom(F, Hp, Wp, heads, kt, ky, kx);
  if (workspace_layout(g, false, nullptr, nullptr) > (size_t)DSA3D_STATIC_SCRATCH_BYTES) return DSA3D_ERR_SCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return DSA3D_ERR_LAUNCH;
  char* ws = scratch_ptr(dev);
  if (!ws) return DSA3D_ERR_LAUNCH;
  // every buffer carved from the scratch is written by the prep kernels before it is
  // read, so the previous call's contents need no clearing
  return run_forward(q, k, v, offsets, g, head_dim, scale, dtype, out, lse, ws, stream, 0u, nullptr);
}
