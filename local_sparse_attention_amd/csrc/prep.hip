// Window starts and the query bucketing shared by the forward and backward passes.
//
// Every query's window start (the clamped, offset-shifted window of the 3D
// Deformable Slide Attention section) is turned into a start cell of the lattice
// (F-kt+1) x (Hp-ky+1) x (Wp-kx+1).  Queries are then stably sorted by cell (LSD
// radix sort, ascending query id inside a cell), which gives
//   - cell_ptr: the CSR of queries per start cell, walked in a fixed order by the
//     key-centric dK/dV pass (deterministic, no atomics on values);
//   - groups: up to 16 queries of one 1 x 4 x 4 start blob; the queries of a
//     group have windows inside a kt x (ky+3) x (kx+3) box, so they share most of
//     their keys.
#include "internal.hpp"

namespace dsa3d {

Geom make_geom(int F, int Hp, int Wp, int H, int kt, int ky, int kx) {
  Geom g;
  g.F = F; g.Hp = Hp; g.Wp = Wp;
  g.kt = kt; g.ky = ky; g.kx = kx;
  g.Lt = F - kt + 1; g.Ly = Hp - ky + 1; g.Lx = Wp - kx + 1;
  g.nby = (g.Ly + BLOB_Y - 1) / BLOB_Y;
  g.nbx = (g.Lx + BLOB_X - 1) / BLOB_X;
  g.H = H;
  g.N = F * Hp * Wp;
  g.nblobs = g.Lt * g.nby * g.nbx;
  g.keyspace = g.nblobs * BLOB_CELLS;
  return g;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Carves the workspace (base may be null to only size it).  Returns its size.
size_t workspace_layout(const Geom& g, bool backward, char* base, Prep* p) {
  const size_t N = (size_t)g.N;
  const int rb = (int)((N + RADIX_TILE - 1) / RADIX_TILE);
  int bits = 1;
  while ((1u << bits) < (uint32_t)g.keyspace) ++bits;
  const int passes = (bits + 7) / 8;
  const int max_groups = g.N / GROUP_Q + g.nblobs + 1;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* ptr = base ? base + off : nullptr;
    off += align256(bytes);
    return ptr;
  };
  Prep q;
  q.starts = (int4*)take(N * sizeof(int4));
  q.keys[0] = (uint32_t*)take(N * 4);
  q.keys[1] = (uint32_t*)take(N * 4);
  q.vals[0] = (int*)take(N * 4);
  q.vals[1] = (int*)take(N * 4);
  q.ghist = (uint32_t*)take((size_t)256 * rb * 4);
  q.cell_ptr = (int*)take(((size_t)g.keyspace + 1) * 4);
  q.goff = (int*)take(((size_t)g.nblobs + 1) * 4);
  q.groups = (int2*)take((size_t)max_groups * sizeof(int2));
  q.ngroups = (int*)take(4);
  q.delta = backward ? (float*)take(N * g.H * 4) : nullptr;
  const bool kv = backward && kv_items_geometry(g);
  q.kv_off = kv ? (int*)take(((size_t)kv_item_columns(g) * g.Lt + 1) * 4) : nullptr;
  q.kv_ids = kv ? (int*)take(max_kv_items(g) * KV_Q * 4) : nullptr;
  q.kv_st = kv ? (int2*)take(max_kv_items(g) * KV_Q * sizeof(int2)) : nullptr;
  const bool qsg = qs_geometry(g);
  q.qt_off = qsg ? (int*)take(((size_t)qs_items(g) + 1) * 4) : nullptr;
  q.qt = qsg ? (int*)take((size_t)max_groups * QT_INTS * 4) : nullptr;
  q.tq_ids = qsg ? (int*)take((size_t)max_groups * 16 * 4) : nullptr;
  q.tq_st = qsg ? (int2*)take((size_t)max_groups * 16 * sizeof(int2)) : nullptr;
  q.tq_dt = qsg ? (signed char*)take((size_t)max_groups * 16) : nullptr;
  q.qs_off = qsg ? (int*)take(((size_t)qs_items(g) + 1) * 4) : nullptr;
  q.qs = qsg ? (int*)take(qs_ints(g, max_groups) * 4) : nullptr;
  q.perm = q.vals[passes & 1];
  q.radix_blocks = rb;
  q.radix_passes = passes;
  q.max_groups = max_groups;
  if (p) *p = q;
  return off;
}

// ---- window starts ----------------------------------------------------------

__device__ __forceinline__ int clamp_start(int p, int o, int k, int G) {
  // |o| > G moves the centre off the grid either way; clamping o first keeps the
  // sum inside int32 and gives the same start.
  o = min(max(o, -G), G);
  const int s = p + o - (k - 1) / 2;
  return min(max(s, 0), G - k);
}

__device__ __forceinline__ int4 query_start(const int32_t* off, const Geom& g, int n) {
  const int plane = g.Hp * g.Wp;
  const int t = n / plane, rem = n - t * plane, y = rem / g.Wp, x = rem - y * g.Wp;
  int4 s;
  s.x = clamp_start(t, off[3 * n + 0], g.kt, g.F);
  s.y = clamp_start(y, off[3 * n + 1], g.ky, g.Hp);
  s.z = clamp_start(x, off[3 * n + 2], g.kx, g.Wp);
  s.w = 0;
  return s;
}

__global__ __launch_bounds__(256) void k_window_starts(const int32_t* off, Geom g, int32_t* starts3) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= g.N) return;
  const int4 s = query_start(off, g, n);
  starts3[3 * n + 0] = s.x;
  starts3[3 * n + 1] = s.y;
  starts3[3 * n + 2] = s.z;
}

__global__ __launch_bounds__(256) void k_starts_keys(const int32_t* off, Geom g, int4* starts, uint32_t* keys) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= g.N) return;
  const int4 s = query_start(off, g, n);
  starts[n] = s;
  keys[n] = (uint32_t)cell_key(g, s.x, s.y, s.z);
}

// ---- stable LSD radix sort (8-bit digits) ---------------------------------------
// Each block owns RADIX_TILE consecutive items.  hist: per-block digit counts,
// stored digit-major so one exclusive scan gives every (digit, block) its output
// base.  scatter: items are ranked in their original order (16 rounds of 256),
// which keeps the sort stable.

__global__ __launch_bounds__(256) void k_radix_hist(const uint32_t* keys, int n, int shift, uint32_t* ghist, int nblk) {
  __shared__ uint32_t h[256];
  const int tid = threadIdx.x;
  h[tid] = 0;
  __syncthreads();
  const int base = blockIdx.x * RADIX_TILE;
  for (int i = tid; i < RADIX_TILE; i += 256) {
    const int idx = base + i;
    if (idx < n) atomicAdd(&h[(keys[idx] >> shift) & 255u], 1u);
  }
  __syncthreads();
  ghist[(size_t)tid * nblk + blockIdx.x] = h[tid];
}

// In-place exclusive scan (one workgroup of 1024 threads): chunks of 16384 values,
// sixteen consecutive values per thread (four 16-byte loads), wave scans by lane
// shuffles, a running carry; the next chunk's loads are issued before this chunk's
// scan, so one chunk's latency hides behind the other's work.
constexpr int SCAN_PER = 16, SCAN_CHUNK = 1024 * SCAN_PER;
__device__ __forceinline__ void scan_load(const uint32_t* data, int n, int i0, uint32_t (&v)[SCAN_PER]) {
  if (i0 + SCAN_PER <= n) {
#pragma unroll
    for (int j = 0; j < SCAN_PER / 4; ++j) {
      const uint4 u = reinterpret_cast<const uint4*>(data + i0)[j];
      v[4 * j] = u.x;
      v[4 * j + 1] = u.y;
      v[4 * j + 2] = u.z;
      v[4 * j + 3] = u.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < SCAN_PER; ++j) v[j] = i0 + j < n ? data[i0 + j] : 0u;
  }
}
__global__ __launch_bounds__(1024) void k_scan_excl(uint32_t* data, int n) {
  __shared__ uint32_t wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t carry = 0;
  uint32_t v[SCAN_PER], nx[SCAN_PER];
  scan_load(data, n, SCAN_PER * tid, nx);
  for (int base = 0; base < n; base += SCAN_CHUNK) {
    const int i0 = base + SCAN_PER * tid;
#pragma unroll
    for (int j = 0; j < SCAN_PER; ++j) v[j] = nx[j];
    if (base + SCAN_CHUNK < n) scan_load(data, n, i0 + SCAN_CHUNK, nx);
    uint32_t t = 0;
#pragma unroll
    for (int j = 0; j < SCAN_PER; ++j) t += v[j];
    uint32_t inc = t;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t y = __shfl_up(inc, d, 64);
      if (lane >= d) inc += y;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const uint32_t x = wsum[w];
      before += w < wave ? x : 0u;
      total += x;
    }
    uint32_t run = carry + before + inc - t;
    if (i0 + SCAN_PER <= n) {
#pragma unroll
      for (int j = 0; j < SCAN_PER / 4; ++j) {
        uint4 u;
        u.x = run; run += v[4 * j];
        u.y = run; run += v[4 * j + 1];
        u.z = run; run += v[4 * j + 2];
        u.w = run; run += v[4 * j + 3];
        reinterpret_cast<uint4*>(data + i0)[j] = u;
      }
    } else {
#pragma unroll
      for (int j = 0; j < SCAN_PER; ++j) {
        if (i0 + j < n) data[i0 + j] = run;
        run += v[j];
      }
    }
    carry += total;
    __syncthreads();  // wsum is rewritten by the next chunk
  }
}

__global__ __launch_bounds__(256) void k_radix_scatter(const uint32_t* kin, const int* vin, int n, int shift,
                                                       const uint32_t* gbase, int nblk, uint32_t* kout, int* vout) {
  __shared__ uint32_t base[256], run[256];
  __shared__ uint32_t wcnt[4][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  base[tid] = gbase[(size_t)tid * nblk + blockIdx.x];
  run[tid] = 0;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = 0; r < RADIX_TILE / 256; ++r) {
    const int idx = blockIdx.x * RADIX_TILE + r * 256 + tid;
    const bool valid = idx < n;
    const uint32_t key = valid ? kin[idx] : 0u;
    const uint32_t d = (key >> shift) & 255u;
    const int val = valid ? (vin ? vin[idx] : idx) : 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) wcnt[w][tid] = 0;
    __syncthreads();
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (d >> b) & 1u;
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    const uint32_t rank = (uint32_t)__popcll(m & lt);
    if (valid && rank == 0) wcnt[wave][d] = (uint32_t)__popcll(m);
    __syncthreads();
    {
      uint32_t acc = run[tid];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t c = wcnt[w][tid];
        wcnt[w][tid] = acc;
        acc += c;
      }
      run[tid] = acc;
    }
    __syncthreads();
    if (valid) {
      const uint32_t pos = base[d] + wcnt[wave][d] + rank;
      kout[pos] = key;
      vout[pos] = val;
    }
    __syncthreads();
  }
}

// cell_ptr[c] = number of sorted keys below c, for c = 0 .. keyspace.
__global__ __launch_bounds__(256) void k_cell_ptr(const uint32_t* skeys, int n, int keyspace, int* cell_ptr) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c > keyspace) return;
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (skeys[mid] < (uint32_t)c) lo = mid + 1; else hi = mid;
  }
  cell_ptr[c] = lo;
}

__global__ __launch_bounds__(256) void k_blob_ngroups(const int* cell_ptr, int nblobs, int* goff) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b > nblobs) return;
  if (b == nblobs) { goff[b] = 0; return; }
  const int cnt = cell_ptr[(b + 1) * BLOB_CELLS] - cell_ptr[b * BLOB_CELLS];
  goff[b] = (cnt + GROUP_Q - 1) / GROUP_Q;
}

__global__ __launch_bounds__(256) void k_groups(const int* cell_ptr, const int* goff, int nblobs, int2* groups,
                                                int* ngroups) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b == 0) *ngroups = goff[nblobs];
  if (b >= nblobs) return;
  const int beg = cell_ptr[b * BLOB_CELLS];
  const int cnt = cell_ptr[(b + 1) * BLOB_CELLS] - beg;
  const int g0 = goff[b], ng = goff[b + 1] - g0;
  for (int i = 0; i < ng; ++i) groups[g0 + i] = make_int2(beg + i * GROUP_Q, min(GROUP_Q, cnt - i * GROUP_Q));
}

static unsigned blocks(long long n, int per) { return (unsigned)((n + per - 1) / per); }

hipError_t launch_scan_excl(uint32_t* data, int n, hipStream_t s) {
  k_scan_excl<<<1, 1024, 0, s>>>(data, n);
  return hipGetLastError();
}

hipError_t launch_window_starts(const int32_t* off, const Geom& g, int32_t* starts3, hipStream_t s) {
  k_window_starts<<<blocks(g.N, 256), 256, 0, s>>>(off, g, starts3);
  return hipGetLastError();
}

hipError_t launch_prep(const int32_t* off, const Geom& g, Prep& p, hipStream_t s) {
  const int n = g.N, nb = p.radix_blocks;
  k_starts_keys<<<blocks(n, 256), 256, 0, s>>>(off, g, p.starts, p.keys[0]);
  int cur = 0;
  for (int pass = 0; pass < p.radix_passes; ++pass) {
    k_radix_hist<<<nb, 256, 0, s>>>(p.keys[cur], n, 8 * pass, p.ghist, nb);
    k_scan_excl<<<1, 1024, 0, s>>>(p.ghist, 256 * nb);
    k_radix_scatter<<<nb, 256, 0, s>>>(p.keys[cur], pass == 0 ? nullptr : p.vals[cur], n, 8 * pass, p.ghist, nb,
                                       p.keys[cur ^ 1], p.vals[cur ^ 1]);
    cur ^= 1;
  }
  // p.perm was set to vals[passes & 1] == vals[cur]
  k_cell_ptr<<<blocks((long long)g.keyspace + 1, 256), 256, 0, s>>>(p.keys[cur], n, g.keyspace, p.cell_ptr);
  k_blob_ngroups<<<blocks((long long)g.nblobs + 1, 256), 256, 0, s>>>(p.cell_ptr, g.nblobs, p.goff);
  k_scan_excl<<<1, 1024, 0, s>>>(reinterpret_cast<uint32_t*>(p.goff), g.nblobs + 1);
  k_groups<<<blocks(g.nblobs > 0 ? g.nblobs : 1, 256), 256, 0, s>>>(p.cell_ptr, p.goff, g.nblobs, p.groups,
                                                                     p.ngroups);
  return hipGetLastError();
}

}  // namespace dsa3d
