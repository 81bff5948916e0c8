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
  g.h0 = 0;
  g.nh = H;
  g.ph = 1;
  g.N = F * Hp * Wp;
  g.nblobs = g.Lt * g.nby * g.nbx;
  g.keyspace = g.nblobs * BLOB_CELLS;
  return g;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Carves the workspace (base may be null to only size it).  Returns its size.  With
// g.ph heads of bucketing every array below holds g.ph blocks, one per head.
size_t workspace_layout(const Geom& g, bool backward, char* base, Prep* p) {
  const size_t NH = (size_t)g.N;            // tokens (delta is [H][N])
  const size_t N = NH * g.ph;               // bucketed queries
  const int rb = (int)((NH + RADIX_TILE - 1) / RADIX_TILE);  // radix blocks per head block
  int bits = 1;
  while ((1u << bits) < (uint32_t)g.keyspace) ++bits;  // keys are cells; head blocks sort apart
  const int passes = (bits + 7) / 8;
  const int max_groups = (g.N / GROUP_Q + g.nblobs + 1) * g.ph;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* ptr = base ? base + off : nullptr;
    off += align256(bytes);
    return ptr;
  };
  // The bucketing and the query-side schedules, which the forward and the backward build
  // alike, come first and at the same offsets in both layouts, so that a backward may use
  // what a forward built in the same workspace; the backward's own arrays follow.
  Prep q;
  q.starts = (int4*)take(N * sizeof(int4));
  q.keys[0] = (uint32_t*)take(N * 4);
  q.keys[1] = (uint32_t*)take(N * 4);
  q.vals[0] = (int*)take(N * 4);
  q.vals[1] = (int*)take(N * 4);
  q.ghist = (uint32_t*)take((size_t)256 * rb * g.ph * 4);
  q.cell_ptr = (int*)take(((size_t)g.keyspace * g.ph + 1) * 4);
  q.goff = (int*)take(((size_t)g.nblobs * g.ph + 1) * 4);
  q.groups = (int2*)take((size_t)max_groups * sizeof(int2));
  q.ngroups = (int*)take(4);
  const bool qsg = qs_geometry(g);
  q.qt_off = qsg ? (int*)take(((size_t)qs_items(g) * g.ph + 1) * 4) : nullptr;
  q.qt = qsg ? (int*)take((size_t)max_groups * QT_INTS * 4) : nullptr;
  q.tq_ids = qsg ? (int*)take((size_t)max_groups * 16 * 4) : nullptr;
  q.tq_st = qsg ? (int2*)take((size_t)max_groups * 16 * sizeof(int2)) : nullptr;
  q.tq_dt = qsg ? (signed char*)take((size_t)max_groups * 16) : nullptr;
  q.qs_off = qsg ? (int*)take(((size_t)qs_items(g) * g.ph + 1) * 4) : nullptr;
  q.qs = qsg ? (int*)take((qs_ints(g, max_groups / g.ph) * g.ph) * 4) : nullptr;
  // the longest scan of either pass: radix counts, blob group counts, work-list and item
  // offsets
  const bool kvg = kv_items_geometry(g);
  size_t scan_n = (size_t)256 * rb * g.ph;
  scan_n = max(scan_n, (size_t)g.nblobs * g.ph + 1);
  if (qsg) scan_n = max(scan_n, (size_t)qs_items(g) * g.ph + 1);
  if (kvg) scan_n = max(scan_n, (size_t)kv_item_columns(g) * g.Lt * g.ph + 1);
  q.scan_part = (uint32_t*)take(scan_part_words(scan_n) * 4);
  q.delta = backward ? (float*)take(NH * g.H * 4) : nullptr;
  const bool kv = backward && kvg;
  q.kv_off = kv ? (int*)take(((size_t)kv_item_columns(g) * g.Lt * g.ph + 1) * 4) : nullptr;
  q.kv_ids = kv ? (int*)take(max_kv_items(g) * g.ph * KV_Q * 4) : nullptr;
  q.kv_mask = kv ? (int*)take(max_kv_items(g) * g.ph * KV_Q * sizeof(int)) : nullptr;
  q.sorted_st = kv ? (int2*)take(N * sizeof(int2)) : nullptr;
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
  s.x = clamp_start(t, off[3 * (size_t)n + 0], g.kt, g.F);
  s.y = clamp_start(y, off[3 * (size_t)n + 1], g.ky, g.Hp);
  s.z = clamp_start(x, off[3 * (size_t)n + 2], g.kx, g.Wp);
  s.w = 0;
  return s;
}

__global__ __launch_bounds__(256) void k_window_starts(const int32_t* off, Geom g, int32_t* starts3) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= g.N) return;
  const int4 s = query_start(off, g, n);
  starts3[3 * (size_t)n + 0] = s.x;
  starts3[3 * (size_t)n + 1] = s.y;
  starts3[3 * (size_t)n + 2] = s.z;
}

// Query i of the bucketing is token n = i mod N of head block i / N (offsets of
// that block at off + 3 N (i / N)); the head blocks are sorted as separate segments.
__global__ __launch_bounds__(256) void k_starts_keys(const int32_t* off, Geom g, int4* starts, uint32_t* keys) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= g.N * g.ph) return;
  const int hb = i / g.N, n = i - hb * g.N;
  const int4 s = query_start(off + (size_t)3 * g.N * hb, g, n);
  starts[i] = s;
  keys[i] = (uint32_t)cell_key(g, s.x, s.y, s.z);
}

// k_starts_keys and the first radix pass's histogram in one launch, for sorts of few
// blocks (see k_radix_hist): block x takes RADIX_TILE queries of head block
// x / nbs, RADIX_TILE / 256 a thread, their offsets loaded before any start is formed.
__global__ __launch_bounds__(256) void k_starts_hist(const int32_t* off, Geom g, int nbs, int4* starts,
                                                     uint32_t* keys, uint32_t* ghist) {
  constexpr int PER = RADIX_TILE / 256;
  __shared__ uint32_t h[256];
  const int tid = threadIdx.x;
  h[tid] = 0;
  const int hb = blockIdx.x / nbs, b = blockIdx.x - hb * nbs;
  const int lim = min(RADIX_TILE, g.N - b * RADIX_TILE);
  const int32_t* o = off + (size_t)3 * g.N * hb;
  int os[PER][3];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int l = tid + 256 * j;
    const int n = b * RADIX_TILE + (l < lim ? l : 0);
#pragma unroll
    for (int c = 0; c < 3; ++c) os[j][c] = o[3 * (size_t)n + c];
  }
  __syncthreads();
  const int plane = g.Hp * g.Wp;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int l = tid + 256 * j;
    if (l < lim) {
      const int n = b * RADIX_TILE + l;
      const int t = n / plane, rem = n - t * plane, y = rem / g.Wp, x = rem - y * g.Wp;
      int4 st;
      st.x = clamp_start(t, os[j][0], g.kt, g.F);
      st.y = clamp_start(y, os[j][1], g.ky, g.Hp);
      st.z = clamp_start(x, os[j][2], g.kx, g.Wp);
      st.w = 0;
      const size_t i = (size_t)hb * g.N + n;
      const uint32_t key = (uint32_t)cell_key(g, st.x, st.y, st.z);
      starts[i] = st;
      keys[i] = key;
      atomicAdd(&h[key & 255u], 1u);
    }
  }
  __syncthreads();
  ghist[((size_t)hb * 256 + tid) * nbs + b] = h[tid];
}

// ---- stable LSD radix sort (8-bit digits), by segments --------------------------
// The items are nseg segments of seglen, each sorted on its own.  Block x owns
// RADIX_TILE consecutive items of segment x / nbs (nbs blocks per segment).  hist:
// per-block digit counts, stored segment-, then digit-major, so that one exclusive
// scan over all of them gives every (segment, digit, block) its output base: the
// counts of a segment add up to seglen, so segment i's bases start at i * seglen.
// scatter: items are ranked in their original order (RADIX_TILE / 256 rounds of 256),
// which keeps the sort stable.

__global__ __launch_bounds__(256) void k_radix_hist(const uint32_t* keys, int seglen, int nbs, int shift,
                                                    uint32_t* ghist) {
  __shared__ uint32_t h[256];
  const int tid = threadIdx.x;
  h[tid] = 0;
  __syncthreads();
  const int sg = blockIdx.x / nbs, b = blockIdx.x - sg * nbs;
  const size_t base = (size_t)sg * seglen + (size_t)b * RADIX_TILE;
  const int lim = min(RADIX_TILE, seglen - b * RADIX_TILE);
  for (int i = tid; i < lim; i += 256) atomicAdd(&h[(keys[base + i] >> shift) & 255u], 1u);
  __syncthreads();
  ghist[((size_t)sg * 256 + tid) * nbs + b] = h[tid];
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
// part == nullptr: one workgroup scans all n values, chunk after chunk with a
// running carry.  Otherwise workgroup b scans chunk b alone and leaves its total in
// part[b] (k_scan_add then adds the scanned totals).
static_assert(SCAN_CHUNK == SCAN_CHUNK_N, "scan chunk");
__device__ __forceinline__ void scan_range(uint32_t* data, int start, int end, uint32_t* part_slot) {
  __shared__ uint32_t wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t carry = 0;
  uint32_t v[SCAN_PER], nx[SCAN_PER];
  scan_load(data, end, start + SCAN_PER * tid, nx);
  for (int base = start; base < end; base += SCAN_CHUNK) {
    const int i0 = base + SCAN_PER * tid;
#pragma unroll
    for (int j = 0; j < SCAN_PER; ++j) v[j] = nx[j];
    if (base + SCAN_CHUNK < end) scan_load(data, end, i0 + SCAN_CHUNK, nx);
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
    if (i0 + SCAN_PER <= end) {
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
        if (i0 + j < end) data[i0 + j] = run;
        run += v[j];
      }
    }
    carry += total;
    __syncthreads();  // wsum is rewritten by the next chunk
  }
  if (part_slot && tid == 0) *part_slot = carry;
}

__global__ __launch_bounds__(1024) void k_scan_excl(uint32_t* data, int n, uint32_t* part) {
  const int start = part ? blockIdx.x * SCAN_CHUNK : 0;
  scan_range(data, start, part ? min(start + SCAN_CHUNK, n) : n, part ? part + blockIdx.x : nullptr);
}

// Two independent single-workgroup scans in one launch: block 0 scans a, block 1 b.
__global__ __launch_bounds__(1024) void k_scan_excl2(uint32_t* a, int na, uint32_t* b, int nb) {
  if (blockIdx.x == 0) scan_range(a, 0, na, nullptr);
  else scan_range(b, 0, nb, nullptr);
}

__global__ __launch_bounds__(256) void k_scan_add(uint32_t* data, int n, const uint32_t* part) {
  const int b = blockIdx.x / (SCAN_CHUNK / 256);
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) data[i] += part[b];
}

// gbase holds the scanned counts, or (raw) the counts k_radix_hist left: then each
// block forms its own bases from its segment's nbs counts per digit, the counts of the
// smaller digits in every block of the segment plus those of its digit in the blocks
// before it (the same values the scan gives, without its launches).
__global__ __launch_bounds__(256) void k_radix_scatter(const uint32_t* kin, const int* vin, int seglen, int nbs,
                                                       int shift, const uint32_t* gbase, int raw, uint32_t* kout,
                                                       int* vout) {
  __shared__ uint32_t base[256], run[256];
  __shared__ uint32_t wcnt[4][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sg = blockIdx.x / nbs, b = blockIdx.x - sg * nbs;
  if (raw) {
    const uint32_t* hc = gbase + ((size_t)sg * 256 + tid) * nbs;
    uint32_t tot = 0, pre = 0;
    for (int j = 0; j < nbs; ++j) {
      const uint32_t c = hc[j];
      pre += j < b ? c : 0u;
      tot += c;
    }
    uint32_t inc = tot;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t y = __shfl_up(inc, d, 64);
      if (lane >= d) inc += y;
    }
    if (lane == 63) run[wave] = inc;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) before += w < wave ? run[w] : 0u;
    __syncthreads();  // run is cleared below
    base[tid] = (uint32_t)sg * (uint32_t)seglen + before + inc - tot + pre;
  } else {
    base[tid] = gbase[((size_t)sg * 256 + tid) * nbs + b];
  }
  run[tid] = 0;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = 0; r < RADIX_TILE / 256; ++r) {
    const int local = b * RADIX_TILE + r * 256 + tid;
    const bool valid = local < seglen;
    const int idx = sg * seglen + local;
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

// cell_ptr[i keyspace + c]: position of the first key >= c of segment i (the end of
// the segment when there is none), for i keyspace + c = 0 .. nseg keyspace.  Thread
// j = 0 .. seglen of segment i writes the cells c with key[j - 1] < c <= key[j]
// (from cell 0 for j = 0, to the segment's last entry for j = seglen): exactly j keys
// of the segment lie below each of them, and every entry is written once.  The last
// entry of a segment is its own c = keyspace only in the last segment (elsewhere it
// is the next segment's c = 0); keys equal to keyspace (a sentinel sorted after every
// cell) are allowed there.
__global__ __launch_bounds__(256) void k_cell_ptr(const uint32_t* skeys, int seglen, int nseg, int keyspace,
                                                  int* cell_ptr) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long long)nseg * (seglen + 1)) return;
  const int sg = (int)(t / (seglen + 1)), j = (int)(t - (long long)sg * (seglen + 1));
  const uint32_t* k = skeys + (size_t)sg * seglen;
  const int lo = j > 0 ? (int)k[j - 1] + 1 : 0;
  const int fin = sg == nseg - 1 ? keyspace : keyspace - 1;  // the segment's last entry
  const int hi = j < seglen ? min((int)k[j], fin) : fin;
  int* cp = cell_ptr + (size_t)sg * keyspace;
  const int v = sg * seglen + j;
  for (int c = lo; c <= hi; ++c) cp[c] = v;
}

// Group counts of the blobs (up to GROUP_Q queries each) from cell_ptr, into goff
// (goff[nblobs] = 0), for an exclusive scan.
__global__ __launch_bounds__(256) void k_blob_ngroups(const int* cell_ptr, int nblobs, int* goff) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b > nblobs) return;
  const int cnt = b == nblobs ? 0 : cell_ptr[(b + 1) * BLOB_CELLS] - cell_ptr[b * BLOB_CELLS];
  goff[b] = (cnt + GROUP_Q - 1) / GROUP_Q;
}

static unsigned blocks(long long n, int per) { return (unsigned)((n + per - 1) / per); }

hipError_t launch_scan_excl(uint32_t* data, int n, hipStream_t s, uint32_t* part) {
  if (!part || n <= 4 * SCAN_CHUNK) {
    k_scan_excl<<<1, 1024, 0, s>>>(data, n, nullptr);
    return hipGetLastError();
  }
  const int nb = (n + SCAN_CHUNK - 1) / SCAN_CHUNK;
  k_scan_excl<<<nb, 1024, 0, s>>>(data, n, part);
  k_scan_excl<<<1, 1024, 0, s>>>(part, nb, nullptr);
  k_scan_add<<<blocks(n, 256), 256, 0, s>>>(data, n, part);
  return hipGetLastError();
}

hipError_t launch_scan_excl2(uint32_t* a, int na, uint32_t* b, int nb, hipStream_t s, uint32_t* part) {
  if (na <= 4 * SCAN_CHUNK && nb <= 4 * SCAN_CHUNK) {
    k_scan_excl2<<<2, 1024, 0, s>>>(a, na, b, nb);
    return hipGetLastError();
  }
  const hipError_t e = launch_scan_excl(a, na, s, part);
  return e != hipSuccess ? e : launch_scan_excl(b, nb, s, part);
}

hipError_t launch_window_starts(const int32_t* off, const Geom& g, int32_t* starts3, hipStream_t s) {
  k_window_starts<<<blocks(g.N, 256), 256, 0, s>>>(off, g, starts3);
  return hipGetLastError();
}

int radix_sort(uint32_t* keys[2], int* vals[2], uint32_t* ghist, int seglen, int nseg, int passes, hipStream_t s,
               uint32_t* part, bool first_hist_done) {
  const int nbs = (seglen + RADIX_TILE - 1) / RADIX_TILE, nb = nbs * nseg;
  const int raw = nbs <= RADIX_RAW_NBS;
  int cur = 0;
  for (int pass = 0; pass < passes; ++pass) {
    if (pass > 0 || !first_hist_done) k_radix_hist<<<nb, 256, 0, s>>>(keys[cur], seglen, nbs, 8 * pass, ghist);
    if (!raw && launch_scan_excl(ghist, 256 * nb, s, part) != hipSuccess) return -1;
    k_radix_scatter<<<nb, 256, 0, s>>>(keys[cur], pass == 0 ? nullptr : vals[cur], seglen, nbs, 8 * pass, ghist, raw,
                                       keys[cur ^ 1], vals[cur ^ 1]);
    cur ^= 1;
  }
  return hipGetLastError() == hipSuccess ? cur : -1;
}

hipError_t launch_cell_ptr(const uint32_t* sorted_keys, int seglen, int nseg, int keyspace, int* cell_ptr,
                           hipStream_t s) {
  k_cell_ptr<<<blocks((long long)nseg * (seglen + 1), 256), 256, 0, s>>>(sorted_keys, seglen, nseg, keyspace,
                                                                          cell_ptr);
  return hipGetLastError();
}

// Bucketing, and with qs the query-side work lists too:
//   window starts and keys (with the first radix pass's histogram for small sorts),
//   the radix passes, cell_ptr, the blob group counts [with the row tile counts],
//   the scans of the group [and tile] counts, the groups [and row tiles],
//   [the tile rows and the schedules].
hipError_t launch_prep(const int32_t* off, const Geom& g, Prep& p, bool qs, int nslots, hipStream_t s) {
  const int n = g.N * g.ph, nblobs = g.nblobs * g.ph;
  const int nbs = (g.N + RADIX_TILE - 1) / RADIX_TILE;
  const bool fused = nbs <= RADIX_RAW_NBS;  // the scatter then needs the raw counts the fused kernel leaves
  if (fused)
    k_starts_hist<<<(unsigned)(nbs * g.ph), 256, 0, s>>>(off, g, nbs, p.starts, p.keys[0], p.ghist);
  else
    k_starts_keys<<<blocks(n, 256), 256, 0, s>>>(off, g, p.starts, p.keys[0]);
  // each head block of the bucketing is a segment of its own
  const int cur = radix_sort(p.keys, p.vals, p.ghist, g.N, g.ph, p.radix_passes, s, p.scan_part, fused);
  if (cur < 0) return hipErrorLaunchFailure;
  // p.perm was set to vals[passes & 1] == vals[cur]
  if (launch_cell_ptr(p.keys[cur], g.N, g.ph, g.keyspace, p.cell_ptr, s) != hipSuccess) return hipGetLastError();
  hipError_t e;
  if (qs) {
    // the blob group counts ride along with the row tile counts
    if ((e = launch_qtile_count(g, p, s, true)) != hipSuccess) return e;
    e = launch_scan_excl2(reinterpret_cast<uint32_t*>(p.goff), nblobs + 1, reinterpret_cast<uint32_t*>(p.qt_off),
                          qs_items(g) * g.ph + 1, s, p.scan_part);
  } else {
    k_blob_ngroups<<<blocks((long long)nblobs + 1, 256), 256, 0, s>>>(p.cell_ptr, nblobs, p.goff);
    e = launch_scan_excl(reinterpret_cast<uint32_t*>(p.goff), nblobs + 1, s, p.scan_part);
  }
  if (e != hipSuccess) return e;
  if ((e = launch_groups_qtiles(g, p, true, qs, s)) != hipSuccess) return e;
  return qs ? launch_qsched_rows(g, p, nslots, s) : hipSuccess;
}

}  // namespace dsa3d
