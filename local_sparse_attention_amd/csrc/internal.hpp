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
// ev (nullable): events recorded between the dQ and dK/dV kernels ([0]) and after them ([1]).
hipError_t launch_backward_v1(int dtype, int D, const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s,
                              const hipEvent_t* ev);
// Frame-sweeping kernels that share each staged key tile between the queries of
// kt slices: windows up to 8 x 9 x 9.
bool tube_eligible(const Geom& g, int dtype, int D);
hipError_t launch_forward_tube(int dtype, int D, const AttnArgs& a, const Geom& g, const Prep& p, hipStream_t s);

}  // namespace dsa3d
