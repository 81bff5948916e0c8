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
 *                    larger than the grid dimension; N < 2^30; 1 <= heads <= 65535.
 *   Memory           The library allocates nothing and keeps no state between
 *                    calls.  Scratch space is the caller's `workspace` of at least
 *                    dsa3d_workspace_bytes(...) bytes; concurrent calls need
 *                    distinct workspaces.
 *   Streams          Work is enqueued on `stream` (0 = the null stream) and the
 *                    call returns without synchronising.
 *   Errors           All arguments are checked before anything is enqueued: a
 *                    negative status means nothing was launched.
 *                    DSA3D_ERR_LAUNCH reports a failed launch.  Faults inside a
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
  DSA3D_ERR_GRID = -4,      /* F, Hp, Wp < 1, N too large, or heads out of range */
  DSA3D_ERR_WINDOW = -5,    /* a window dimension is even, < 1 or larger than the grid */
  DSA3D_ERR_ALIGN = -6,     /* a tensor or the workspace is not 16-byte aligned */
  DSA3D_ERR_WORKSPACE = -7, /* workspace_bytes is smaller than dsa3d_workspace_bytes() */
  DSA3D_ERR_LAUNCH = -8,    /* a kernel launch failed */
  DSA3D_ERR_SCALE = -9      /* scale is not finite */
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

/* Profiling variants: the same work as dsa3d_forward / dsa3d_backward, plus
   hipEventRecord(events[i], stream) at the phase boundaries, so the caller can
   time each kernel on the stream it runs on.  `events` holds caller-created
   events: forward 3 ([0] before the bucketing of queries by window start and the
   work lists, [1] before the attention kernel, [2] after it); backward 4 ([0]
   before the bucketing, the work lists and the Delta = rowsum(dO * O) pass, [1]
   before the dQ kernel, [2] before the dK/dV kernel, [3] after it).  A null
   `events` gives the untimed call. */
int dsa3d_forward_timed(const void* q, const void* k, const void* v, const int32_t* offsets, int F, int Hp, int Wp,
                        int heads, int head_dim, int kt, int ky, int kx, float scale, int dtype, void* out,
                        float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream,
                        const hipEvent_t* events);
int dsa3d_backward_timed(const void* q, const void* k, const void* v, const int32_t* offsets, const void* out,
                         const float* lse, const void* dout, int F, int Hp, int Wp, int heads, int head_dim,
                         int kt, int ky, int kx, float scale, int dtype, void* dq, void* dk, void* dv,
                         void* workspace, size_t workspace_bytes, hipStream_t stream, const hipEvent_t* events);

/* Static string for a status code. */
const char* dsa3d_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DSA3D_H */
