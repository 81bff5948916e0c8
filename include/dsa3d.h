/*
 * dsa3d.h -- C ABI of the 3D Deformable Slide Attention (3D-DSA) library for
 * AMD MI355X (gfx950).  Library: libdsa3d.so.
 *
 * What is computed (MegaSlide-DiT paper, section "3D Deformable Slide
 * Attention": the attention term of Eq. (1) with the softmax weights alpha
 * defined under it, over the kt x kh x kw neighbourhood of each token of the
 * T x H' x W' token grid):
 *
 *   for every query token n at grid position p = (t, y, x) and head h,
 *     window W(n) = box of kt x ky x kx tokens starting at
 *       s_d = min(max(p_d + o_d - (k_d - 1) / 2, 0), G_d - k_d)     d = t, y, x
 *     (centred on p + o, o = the query's integer offset (dt, dy, dx), with the
 *     box clamped to lie inside the grid G = (F, Hp, Wp));
 *     z_j   = scale * <q[n,h,:], k[j,h,:]>                 j in W(n)
 *     lse   = log sum_j exp(z_j)                            (natural log)
 *     out[n,h,:] = sum_j exp(z_j - lse) * v[j,h,:]
 *   No causal mask.  The offset is shared by all window samples and heads;
 *   integer offsets make the paper's trilinear sampling an exact gather.
 *
 * Conventions for every entry point
 *   Token order      n = (t * Hp + y) * Wp + x, N = F * Hp * Wp.
 *   Tensors          q, k, v, out, dout, dq, dk, dv: contiguous [N][heads][head_dim],
 *                    all of one dtype (DSA3D_F32 or DSA3D_BF16).  lse: fp32
 *                    [heads][N].  offsets: int32 [N][3] in (dt, dy, dx) order (any
 *                    int32 value; values past the grid clamp to its border).
 *   Pointers         DEVICE pointers owned by the caller; tensor pointers and the
 *                    workspace 16-byte aligned.  Inputs are only read.  Outputs
 *                    are fully overwritten (dk, dv are not accumulated into).
 *   Limits           head_dim 64 or 128; each window dimension odd, >= 1 and not
 *                    larger than the grid dimension; N < 2^30; fewer than 2^27
 *                    blobs of 1 x 4 x 4 start cells, i.e.
 *                    (F-kt+1) * ceil((Hp-ky+1)/4) * ceil((Wp-kx+1)/4) < 2^27;
 *                    1 <= heads <= 65535.
 *   Memory           The library allocates nothing and keeps no state between
 *                    calls.  Scratch space is the caller's `workspace` of at least
 *                    dsa3d_workspace_bytes(...) bytes; concurrent calls need
 *                    distinct workspaces.
 *   Streams          Work is enqueued on `stream` (0 = the null stream) and the
 *                    call returns without synchronising.
 *   Errors           All arguments are checked before anything is enqueued: a
 *                    validation error (every negative status except
 *                    DSA3D_ERR_LAUNCH) means nothing was launched.
 *                    DSA3D_ERR_LAUNCH reports a failed launch; kernels of the same
 *                    call that were launched before it may already be on the
 *                    stream, so the outputs are then undefined.  Faults inside a
 *                    kernel surface at the caller's next synchronisation.  The
 *                    library never prints, raises or aborts.
 *   Determinism      Outputs are bitwise identical for identical inputs (no
 *                    floating-point atomics; the dk/dv reduction visits queries
 *                    in a fixed order).
 *   Finite inputs    q, k, v and dout are expected to be finite.  The kernels
 *                    multiply whole 16-token tiles, with zero weights outside a
 *                    query's window, so an inf or NaN in one row can reach the
 *                    outputs of other queries (keys) of the same tile.
 */
#ifndef DSA3D_H
#define DSA3D_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { DSA3D_F32 = 0, DSA3D_BF16 = 1 } dsa3d_dtype;

enum {
  DSA3D_OK = 0,
  DSA3D_ERR_NULL = -1,      /* a required pointer is null */
  DSA3D_ERR_DTYPE = -2,     /* dtype is not DSA3D_F32 / DSA3D_BF16 */
  DSA3D_ERR_HEAD_DIM = -3,  /* head_dim is not 64 or 128 */
  DSA3D_ERR_GRID = -4,      /* F, Hp, Wp < 1, N or the start-cell count too large, or heads out of range */
  DSA3D_ERR_WINDOW = -5,    /* a window dimension is even, < 1 or larger than the grid */
  DSA3D_ERR_ALIGN = -6,     /* a tensor or the workspace is not 16-byte aligned */
  DSA3D_ERR_WORKSPACE = -7, /* workspace_bytes is smaller than dsa3d_workspace_bytes() */
  DSA3D_ERR_LAUNCH = -8,    /* a kernel launch failed */
  DSA3D_ERR_SCALE = -9,     /* scale is not finite */
  DSA3D_ERR_FLAGS = -10,    /* flags holds a bit not defined below */
  DSA3D_ERR_SCRATCH = -11,  /* dsa3d_forward_static: the geometry needs more scratch than
                               DSA3D_STATIC_SCRATCH_BYTES */
  DSA3D_ERR_MODE = -12,     /* sampled windows: mode is not DSA3D_SAMPLE_BOX / DSA3D_SAMPLE_FREE */
  DSA3D_ERR_LAYOUT = -13    /* sampled windows: offset strides negative, overlapping, or a
                               per-sample stride in box mode */
};

/* Bits of the `flags` argument of dsa3d_forward_ex / dsa3d_backward_ex. */
enum {
  /* Run the per-group kernels, which serve every valid geometry, even where the
     frame-sweeping kernels would be chosen.  Results agree within the stated
     tolerances; used by the tests to cover both kernel families on one input. */
  DSA3D_FLAG_GENERIC_KERNELS = 1,
  /* Backward only (dsa3d_backward_ex, dsa3d_backward_heads): use the window starts,
     buckets and query-side row tiles that the forward call just before it built in the
     same workspace, instead of building them again (the pass schedules of the dQ
     kernel, which holds fewer row tiles in flight than the forward, are still built;
     they overwrite the forward's in the workspace).  The caller guarantees that the
     forward ran on this stream with the same workspace pointer and size (sized for the
     backward), offsets (same values), geometry, dtype, head_dim and
     DSA3D_FLAG_GENERIC_KERNELS bit, and that nothing wrote the workspace in between;
     results are then identical to the plain call.  The forward and backward layouts put
     those arrays first, at the same offsets.  dsa3d_backward_heads honours it on its
     all-heads-together route only (the one-head-at-a-time route keeps one head's
     buckets, so it rebuilds them). */
  DSA3D_FLAG_REUSE_PREP = 2
};

/* Bytes of workspace needed by dsa3d_forward (backward = 0) or dsa3d_backward
   (backward = 1) for this geometry; 0 when the geometry is invalid. */
size_t dsa3d_workspace_bytes(int F, int Hp, int Wp, int heads, int kt, int ky, int kx, int backward);

/* Window starts of every query, int32 [N][3] (st, sy, sx) = the s_d above.
   No workspace.  Same validation of grid and window as the other calls. */
int dsa3d_window_starts(const int32_t* offsets, int F, int Hp, int Wp, int kt, int ky, int kx, int32_t* starts,
                        hipStream_t stream);

/* Forward: out [N][heads][head_dim] (dtype) and lse [heads][N] (fp32, natural
   log of the softmax denominator of the scaled logits).  Arithmetic: products
   and sums in fp32 (matrix cores), the softmax weights rounded to the input
   dtype before they multiply V.  `scale` multiplies q.k (callers pass
   1/sqrt(head_dim)). */
int dsa3d_forward(const void* q, const void* k, const void* v, const int32_t* offsets, int F, int Hp, int Wp,
                  int heads, int head_dim, int kt, int ky, int kx, float scale, int dtype, void* out, float* lse,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Backward of the forward above for an output gradient dout: dq, dk, dv
   (dtype, [N][heads][head_dim]).  `out` and `lse` are the forward's results;
   the weights are recomputed from lse.  With P the weights of query n,
     Delta = <dout[n], out[n]>, dS_j = P_j (<dout[n], v_j> - Delta),
     dq[n] = scale sum_j dS_j k_j,  dk_j = scale sum_n dS_nj q_n,
     dv_j = sum_n P_nj dout[n].
   Offsets are integers and get no gradient. */
int dsa3d_backward(const void* q, const void* k, const void* v, const int32_t* offsets, const void* out,
                   const float* lse, const void* dout, int F, int Hp, int Wp, int heads, int head_dim, int kt,
                   int ky, int kx, float scale, int dtype, void* dq, void* dk, void* dv, void* workspace,
                   size_t workspace_bytes, hipStream_t stream);

/* Extended variants: the same work as dsa3d_forward / dsa3d_backward, with
   `flags` (DSA3D_FLAG_* bits; 0 = the plain call) and optional phase events:
   hipEventRecord(events[i], stream) at the phase boundaries, so the caller can
   time each kernel on the stream it runs on.  `events` holds caller-created
   events: forward 3 ([0] before the bucketing of queries by window start and the
   work lists, [1] before the attention kernel, [2] after it); backward 4 ([0]
   before the bucketing, the work lists and the Delta = rowsum(dO * O) pass, [1]
   before the dQ kernel, [2] before the dK/dV kernel, [3] after it).  A null
   `events` records nothing. */
int dsa3d_forward_ex(const void* q, const void* k, const void* v, const int32_t* offsets, int F, int Hp, int Wp,
                     int heads, int head_dim, int kt, int ky, int kx, float scale, int dtype, void* out, float* lse,
                     void* workspace, size_t workspace_bytes, hipStream_t stream, unsigned flags,
                     const hipEvent_t* events);
int dsa3d_backward_ex(const void* q, const void* k, const void* v, const int32_t* offsets, const void* out,
                      const float* lse, const void* dout, int F, int Hp, int Wp, int heads, int head_dim, int kt,
                      int ky, int kx, float scale, int dtype, void* dq, void* dk, void* dv, void* workspace,
                      size_t workspace_bytes, hipStream_t stream, unsigned flags, const hipEvent_t* events);

/* Per-head offsets.  The section learns offsets for each token and each attention
   head; here each head h has its own integer offsets, offsets_heads int32
   [heads][N][3] (head h's (dt, dy, dx) of token n at offsets_heads + 3 * (h * N + n)),
   and head h of out / lse (forward) or of dq / dk / dv (backward) is exactly what
   dsa3d_forward / dsa3d_backward compute for that head with those offsets.  Every
   other argument, the flags, tolerances, determinism and errors are those of the
   *_ex calls.  Workspace: at least dsa3d_workspace_bytes (same arguments); with
   at least dsa3d_workspace_bytes_heads, bf16 and no DSA3D_FLAG_GENERIC_KERNELS,
   the window starts, buckets and work lists of all heads are built together
   (head-major) and each attention kernel runs once over every head; otherwise
   they are built per head, one head after the other in stream order on the one
   workspace, and the kernels run per head.  The results are the same either way. */
size_t dsa3d_workspace_bytes_heads(int F, int Hp, int Wp, int heads, int kt, int ky, int kx, int backward);
int dsa3d_forward_heads(const void* q, const void* k, const void* v, const int32_t* offsets_heads, int F, int Hp,
                        int Wp, int heads, int head_dim, int kt, int ky, int kx, float scale, int dtype, void* out,
                        float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream, unsigned flags);
int dsa3d_backward_heads(const void* q, const void* k, const void* v, const int32_t* offsets_heads, const void* out,
                         const float* lse, const void* dout, int F, int Hp, int Wp, int heads, int head_dim, int kt,
                         int ky, int kx, float scale, int dtype, void* dq, void* dk, void* dv, void* workspace,
                         size_t workspace_bytes, hipStream_t stream, unsigned flags);

/* ---- Sampled windows: real offsets, trilinear sampling ------------------------
   The section samples keys and values from XW_k and XW_v at real positions by
   trilinear interpolation (its implementation paragraph: grid_sample, bilinear
   mode, 5-D tensors) and takes the softmax over the kt x kh x kw samples:
     z_j  = scale * <q[n,h,:], K~_j>,  K~_j = trilinear sample of k[., h, :] at P_j
     out[n,h,:] = sum_j softmax(z)_j * V~_j,  lse = log sum_j exp(z_j)
   A sample at P (token units along t, y, x) blends the 8 grid rows
   floor(P) + {0,1}^3 with weights prod_d (bit_d ? f_d : 1 - f_d), f = P - floor(P);
   rows outside the grid are zero (grid_sample's default padding; integer positions
   are grid points).  Where sample j = (u, v, w) (lexicographic, u over kt) of the
   query at p = (t, y, x) sits, for its offset o (float32 (dt, dy, dx)):
     DSA3D_SAMPLE_BOX   one offset per (query, head), shared by its samples:
                        P_j = s + (u, v, w), s_d = min(max(p_d + o_d - (k_d-1)/2, 0),
                        G_d - k_d) (real); integer offsets give exactly the windows of
                        dsa3d_forward; each k_d <= G_d.
     DSA3D_SAMPLE_FREE  P_j = p + (u, v, w) - (k - 1)/2 + o_j, each sample its own
                        offset (the section's per-sample offsets), zero padded.
   Offsets: float32, three consecutive values per entry, entry (n, h, j) at
   offsets + n * stride_token + h * stride_head + j * stride_sample (element
   strides; 0 = shared: [N][3] shared by heads and samples is (3, 0, 0), [H][N][3]
   per head is (3, 3N, 0), [N][H][K][3] per sample is (3HK, 3K, 3)).  Entries not
   shared must not overlap; box mode needs stride_sample == 0 (DSA3D_ERR_LAYOUT).
   Windows: odd extents, kt * ky * kx <= 4096.  q, k, v, out, dout, dq, dk, dv, lse:
   as for dsa3d_forward / dsa3d_backward (fp32 or bf16, head_dim 64 or 128).
   Arithmetic is fp32 throughout (bf16 inputs widened, outputs rounded to nearest
   even).  Results are bitwise deterministic. */
#define DSA3D_SAMPLE_BOX 0
#define DSA3D_SAMPLE_FREE 1

/* Workspace bytes of dsa3d_sampled_backward (backward = 1; the forward needs none and
   reports 256); 0 for an invalid geometry or one past the backward's limits
   (N * heads * kt*ky*kx < 2^31 samples, heads * (F+1)(Hp+1)(Wp+1) < 2^31 cells).
   About 61 bytes per sample in free mode.  Box mode works on the lattice of the
   L = (kt+1)(ky+1)(kx+1) grid rows that one offset's samples blend, when that lattice
   fits the kernels' LDS (4 (2L + 2 kt*ky*kx) floats <= 16384, so L <= 1024) and
   N * heads * L < 2^31: about 41 bytes per lattice point; otherwise it works per sample
   like free mode (about 49 bytes per sample). */
size_t dsa3d_sampled_workspace_bytes(int F, int Hp, int Wp, int heads, int kt, int ky, int kx, int mode,
                                     int backward);

/* Forward over sampled windows: out [N][heads][head_dim], lse [heads][N]. */
int dsa3d_sampled_forward(const void* q, const void* k, const void* v, const float* offsets, long long stride_token,
                          long long stride_head, long long stride_sample, int mode, int F, int Hp, int Wp, int heads,
                          int head_dim, int kt, int ky, int kx, float scale, int dtype, void* out, float* lse,
                          hipStream_t stream);

/* Backward: dq, dk, dv and doffsets, the gradient of the offsets, written in the
   layout of `offsets` (same strides; an entry shared by several heads or samples
   gets the sum of their gradients, in a fixed order).  The gradient of a sample
   position flows through the interpolation weights (at integer coordinates the
   one-sided derivative of floor-based weights); in box mode also through the clamp
   (1 where p_d + o_d - (k_d-1)/2 lies strictly inside (0, G_d - k_d), else 0).
   dk and dv are gathered per key from its samples (sorted by base cell, fixed
   order), or in box mode on the lattice from the lattice points on that key (sorted
   by token per head, in (query, point) order): no atomics. */
int dsa3d_sampled_backward(const void* q, const void* k, const void* v, const float* offsets, long long stride_token,
                           long long stride_head, long long stride_sample, int mode, const void* out,
                           const float* lse, const void* dout, int F, int Hp, int Wp, int heads, int head_dim, int kt,
                           int ky, int kx, float scale, int dtype, void* dq, void* dk, void* dv, float* doffsets,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- The DWConv3D term and the offset predictor --------------------------------
   Eq. (1) adds a 3-D depthwise convolution of X to the attention term, and the
   offsets are predicted by a depthwise 3-D convolution followed by a linear layer
   (the implementation paragraph: nn.Conv3d with groups equal to the hidden size, then
   pointwise convolutions).  Tensors here are [N][C] with C = heads * head_dim (the
   [N][heads][head_dim] tensors above, seen as one row of C channels per token).

   Depthwise 3-D convolution, one ct x cy x cx filter per channel (odd extents,
   ct*cy*cx <= 512), cross-correlation with zero padding that keeps the grid:
     y[n, c] = (accumulate ? y[n, c] : 0) + bias[c]
               + sum_{a,e,f} weight[c][a][e][f] * x[(t + a - (ct-1)/2, y + e - (cy-1)/2,
                                                    x + f - (cx-1)/2), c]
   x, y: dtype, 16-byte aligned, C a multiple of 8; weight fp32 [C][ct][cy][cx]; bias
   fp32 [C] or null.  accumulate = 1 adds the term into y in place (the attention
   output plus the convolution term, one rounding), 0 overwrites y; y must not overlap
   x (nor dx overlap dy).  fp32 arithmetic.
   Backward: dx (dtype, [N][C]) = the transposed convolution of dy; dweight (fp32,
   weight's shape) and dbias (fp32 [C], or null to skip) sum over the tokens in a
   fixed order (per-frame partial sums in the workspace, then frames in order). */
int dsa3d_dwconv3d_forward(const void* x, const float* weight, const float* bias, int F, int Hp, int Wp, int C, int ct,
                           int cy, int cx, int dtype, void* y, int accumulate, hipStream_t stream);
size_t dsa3d_dwconv3d_workspace_bytes(int F, int Hp, int Wp, int C, int ct, int cy, int cx);
int dsa3d_dwconv3d_backward(const void* x, const float* weight, const void* dy, int F, int Hp, int Wp, int C, int ct,
                            int cy, int cx, int dtype, void* dx, float* dweight, float* dbias, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* Linear (pointwise) layer: y[m][o] = sum_k x[m][k] * weight[o][k] + bias[o], for the
   predictor's map from C channels to heads * kt*ky*kx * 3 offsets per token (the
   free-mode offset layout [N][heads][kt*ky*kx][3] when the outputs are ordered (head,
   sample, axis)).  x [M][Kd] and weight [O][Kd] in dtype (16-byte aligned); y fp32
   [M][O] (the offsets); bias fp32 [O] or null.  Matrix cores, fp32 accumulation.
   Backward: dx (dtype [M][Kd]) = dy weight, dweight (fp32 [O][Kd]) = dy^T x, dbias
   (fp32 [O], or null) = column sums of dy in a fixed order; on the bf16 path dy is
   rounded to bf16 for the two products.  M*Kd, M*O, Kd*O < 2^31. */
int dsa3d_linear_forward(const void* x, const void* weight, const float* bias, int M, int Kd, int O, int dtype,
                         float* y, hipStream_t stream);
size_t dsa3d_linear_workspace_bytes(int M, int Kd, int O, int dtype);
int dsa3d_linear_backward(const void* x, const void* weight, const float* dy, int M, int Kd, int O, int dtype,
                          void* dx, float* dweight, float* dbias, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* Size of the library's static scratch array (one per GPU), used by
   dsa3d_forward_static only. */
#define DSA3D_STATIC_SCRATCH_BYTES (64 * 1024 * 1024)

/* The forward of dsa3d_forward without a workspace, for callers that cannot
   allocate device memory: code under HIP graph capture, tight serving loops and
   harnesses that forbid hipMalloc.  The call allocates nothing (no hipMalloc,
   hipFree or allocating library routine): its scratch is a file-scope device array
   of DSA3D_STATIC_SCRATCH_BYTES in the library, one copy per GPU, held until the
   process ends.  Arguments, outputs, results and errors are those of dsa3d_forward;
   in addition it returns DSA3D_ERR_SCRATCH (nothing launched) when
   dsa3d_workspace_bytes(F, Hp, Wp, heads, kt, ky, kx, 0) exceeds
   DSA3D_STATIC_SCRATCH_BYTES (about 85 bytes per token: N up to ~790,000).  The
   work runs on the current device (`stream` must belong to it); the first call on
   a device looks up that device's copy of the array.  Every call on one GPU shares
   its array, so calls that overlap on one GPU (other streams, other host threads)
   race and must be serialised by the caller; back-to-back calls on one stream are
   safe (every byte read is written earlier in the same call). */
int dsa3d_forward_static(const void* q, const void* k, const void* v, const int32_t* offsets, int F, int Hp, int Wp,
                         int heads, int head_dim, int kt, int ky, int kx, float scale, int dtype, void* out,
                         float* lse, hipStream_t stream);

/* Static string for a status code. */
const char* dsa3d_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DSA3D_H */
