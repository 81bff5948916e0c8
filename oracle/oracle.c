/*
 * oracle.c -- plain, slow CPU reference for the attention term of 3D Deformable
 * Slide Attention (3D-DSA), computed in double precision.
 *
 * TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
 * baseline call it.  It shares no code, header or table with the HIP library.
 *
 * Source: "MegaSlide-DiT: Memory-Centric Adaptation and Deformable Local
 * Attention for Efficient Video Diffusion", section on 3D Deformable Slide
 * Attention: Eq. (1) (second term, the attention sum over the kt x kh x kw
 * neighbourhood), the softmax weights alpha written under it, and the reshape of
 * X (N x d) into T x H' x W' x d.  Readings of what the section leaves open:
 *   - one integer offset (dt, dy, dx) per query token, shared by every window
 *     sample and every head (integer positions make trilinear sampling exact);
 *   - the window is centred on the query's own position plus its offset (the
 *     fixed-window ablation of the results section: zero offsets give fixed local
 *     attention of kernel size 3 x 7 x 7);
 *   - the window is kept inside the grid by clamping its start:
 *       s_d = min(max(p_d + o_d - (k_d - 1) / 2, 0), G_d - k_d);
 *   - the logit scale is a parameter (the workloads use 1/sqrt(head_dim));
 *   - only the attention term: the DWConv3D term of Eq. (1) is additive and is
 *     not part of this operator.  No causal mask (the method section says none is
 *     needed).
 * Token order: n = (t * Hp + y) * Wp + x.  Tensors are [N][H][D], fp32 or raw
 * bf16 bits (fp64 too, for the finite-difference checks); offsets are int32
 * [N][3] in (dt, dy, dx) order.
 *
 * Also here (same section): the depthwise 3-D convolution of Eq. (1)'s first term and
 * of the offset predictor (oracle_dwconv3d_forward / _backward); per-head integer offsets (oracle_forward_heads,
 * oracle_backward_heads), and sampled windows with real offsets and trilinear
 * sampling, with the gradient of the offsets (oracle_sampled_forward,
 * oracle_sampled_backward; their readings are written above those functions).
 *
 * Backward: the standard softmax-attention gradient.  With P the weights of one
 * query and dO its output gradient:
 *   Delta = sum_e dO_e O_e,  dP_j = dO . v_j,  dS_j = P_j (dP_j - Delta),
 *   dq = scale sum_j dS_j k_j,  dk_j += scale dS_j q,  dv_j += P_j dO.
 * Offsets are integers and receive no gradient.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int F, Hp, Wp; /* grid */
  int H, D;      /* heads, head size */
  int kt, ky, kx;
  double scale;
  int dtype; /* 0: fp32, 1: bf16 bits, 2: fp64 */
} oracle_cfg;

#define MAXD 256

/* ---- window ------------------------------------------------------------- */

/* Start of the window along one axis: centre p + o, clamped so that the whole
   k-wide window lies in [0, G). */
static int64_t win_start(int64_t p, int64_t o, int64_t k, int64_t G) {
  int64_t s = p + o - (k - 1) / 2;
  if (s < 0) s = 0;
  if (s > G - k) s = G - k;
  return s;
}

static void query_start(const oracle_cfg* c, const int32_t* off, int64_t n, int64_t s[3]) {
  const int64_t plane = (int64_t)c->Hp * c->Wp;
  const int64_t t = n / plane, y = (n / c->Wp) % c->Hp, x = n % c->Wp;
  s[0] = win_start(t, off[3 * n + 0], c->kt, c->F);
  s[1] = win_start(y, off[3 * n + 1], c->ky, c->Hp);
  s[2] = win_start(x, off[3 * n + 2], c->kx, c->Wp);
}

void oracle_window_starts(const int32_t* off, int F, int Hp, int Wp, int kt, int ky, int kx, int32_t* starts) {
  oracle_cfg c = {F, Hp, Wp, 1, 1, kt, ky, kx, 1.0, 0};
  const int64_t N = (int64_t)F * Hp * Wp;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    int64_t s[3];
    query_start(&c, off, n, s);
    starts[3 * n + 0] = (int32_t)s[0];
    starts[3 * n + 1] = (int32_t)s[1];
    starts[3 * n + 2] = (int32_t)s[2];
  }
}

/* The K = kt*ky*kx keys of query n, in lexicographic (u, v, w) order. */
static void window_keys(const oracle_cfg* c, const int32_t* off, int64_t n, int64_t* keys) {
  int64_t s[3];
  query_start(c, off, n, s);
  int64_t i = 0;
  for (int u = 0; u < c->kt; ++u)
    for (int v = 0; v < c->ky; ++v)
      for (int w = 0; w < c->kx; ++w)
        keys[i++] = ((s[0] + u) * c->Hp + (s[1] + v)) * c->Wp + (s[2] + w);
}

/* ---- data access -------------------------------------------------------- */

static void load_row(const oracle_cfg* c, const void* base, int64_t n, int h, double* out) {
  const size_t off = ((size_t)n * c->H + h) * c->D;
  if (c->dtype == 0) {
    const float* p = (const float*)base + off;
    for (int e = 0; e < c->D; ++e) out[e] = p[e];
  } else if (c->dtype == 2) {
    const double* p = (const double*)base + off;
    for (int e = 0; e < c->D; ++e) out[e] = p[e];
  } else {
    const uint16_t* p = (const uint16_t*)base + off;
    for (int e = 0; e < c->D; ++e) {
      uint32_t b = (uint32_t)p[e] << 16;
      float f;
      memcpy(&f, &b, 4);
      out[e] = f;
    }
  }
}

static double dot(const double* a, const double* b, int D) {
  double s = 0.0;
  for (int e = 0; e < D; ++e) s += a[e] * b[e];
  return s;
}

/* ---- forward ------------------------------------------------------------ */

/* Attention of query n, head h: fills keys[K], the weights p[K], the output row
   o[D] and returns the natural-log log-sum-exp of the scaled logits. */
static double attend(const oracle_cfg* c, const void* q, const void* k, const void* v, const int32_t* off, int64_t n,
                     int h, int64_t* keys, double* p, double* o) {
  const int K = c->kt * c->ky * c->kx, D = c->D;
  double qr[MAXD], row[MAXD];
  window_keys(c, off, n, keys);
  load_row(c, q, n, h, qr);
  double m = -INFINITY;
  for (int j = 0; j < K; ++j) {
    load_row(c, k, keys[j], h, row);
    p[j] = c->scale * dot(qr, row, D);
    if (p[j] > m) m = p[j];
  }
  double sum = 0.0;
  for (int j = 0; j < K; ++j) sum += exp(p[j] - m);
  const double lse = m + log(sum);
  for (int j = 0; j < K; ++j) p[j] = exp(p[j] - lse);
  for (int e = 0; e < D; ++e) o[e] = 0.0;
  for (int j = 0; j < K; ++j) {
    load_row(c, v, keys[j], h, row);
    for (int e = 0; e < D; ++e) o[e] += p[j] * row[e];
  }
  return lse;
}

/* O [N][H][D] and LSE [H][N] for every (query, head). */
void oracle_forward(const oracle_cfg* c, const void* q, const void* k, const void* v, const int32_t* off, double* out,
                    double* lse) {
  const int64_t N = (int64_t)c->F * c->Hp * c->Wp, K = (int64_t)c->kt * c->ky * c->kx;
#pragma omp parallel
  {
    int64_t* keys = malloc(sizeof(int64_t) * K);
    double* p = malloc(sizeof(double) * K);
#pragma omp for schedule(dynamic, 64)
    for (int64_t r = 0; r < N * c->H; ++r) {
      const int64_t n = r / c->H;
      const int h = (int)(r % c->H);
      lse[(int64_t)h * N + n] = attend(c, q, k, v, off, n, h, keys, p, out + (size_t)r * c->D);
    }
    free(keys);
    free(p);
  }
}

/* Same, for a list of rows r = n * H + h only: out[i][D], lse[i]. */
void oracle_forward_rows(const oracle_cfg* c, const void* q, const void* k, const void* v, const int32_t* off,
                         int64_t nrows, const int64_t* rows, double* out, double* lse) {
  const int64_t K = (int64_t)c->kt * c->ky * c->kx;
#pragma omp parallel
  {
    int64_t* keys = malloc(sizeof(int64_t) * K);
    double* p = malloc(sizeof(double) * K);
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; ++i)
      lse[i] = attend(c, q, k, v, off, rows[i] / c->H, (int)(rows[i] % c->H), keys, p, out + (size_t)i * c->D);
    free(keys);
    free(p);
  }
}

/* The window keys and weights of one (query, head): keys[K], p[K]; returns LSE. */
double oracle_weights(const oracle_cfg* c, const void* q, const void* k, const void* v, const int32_t* off, int64_t n,
                      int h, int64_t* keys, double* p) {
  double o[MAXD];
  return attend(c, q, k, v, off, n, h, keys, p, o);
}

/* ---- backward ----------------------------------------------------------- */

/* Backward of one head h with the offsets `off` ([N][3]): dq rows of head h and the
   dk, dv rows of head h (zeroed here, then scattered into). */
static void backward_head(const oracle_cfg* c, const void* q, const void* k, const void* v, const void* dout,
                          const int32_t* off, int h, double* dq, double* dk, double* dv) {
  const int64_t N = (int64_t)c->F * c->Hp * c->Wp, K = (int64_t)c->kt * c->ky * c->kx;
  const int D = c->D;
  int64_t* keys = malloc(sizeof(int64_t) * K);
  double* p = malloc(sizeof(double) * K);
  double o[MAXD], qr[MAXD], dor[MAXD], row[MAXD];
  for (int64_t n = 0; n < N; ++n) {
    double* dkr = dk + ((size_t)n * c->H + h) * D;
    double* dvr = dv + ((size_t)n * c->H + h) * D;
    for (int e = 0; e < D; ++e) dkr[e] = dvr[e] = 0.0;
  }
  for (int64_t n = 0; n < N; ++n) {
    attend(c, q, k, v, off, n, h, keys, p, o);
    load_row(c, q, n, h, qr);
    load_row(c, dout, n, h, dor);
    const double delta = dot(dor, o, D);
    double* dqr = dq + ((size_t)n * c->H + h) * D;
    for (int e = 0; e < D; ++e) dqr[e] = 0.0;
    for (int j = 0; j < K; ++j) {
      load_row(c, v, keys[j], h, row);
      const double ds = p[j] * (dot(dor, row, D) - delta);
      load_row(c, k, keys[j], h, row);
      double* dkr = dk + ((size_t)keys[j] * c->H + h) * D;
      double* dvr = dv + ((size_t)keys[j] * c->H + h) * D;
      for (int e = 0; e < D; ++e) {
        dqr[e] += c->scale * ds * row[e];
        dkr[e] += c->scale * ds * qr[e];
        dvr[e] += p[j] * dor[e];
      }
    }
  }
  free(keys);
  free(p);
}

/* dq, dk, dv [N][H][D] for every row.  One head per thread; within a head the
   queries are visited in order and each scatters into the keys of its window. */
void oracle_backward(const oracle_cfg* c, const void* q, const void* k, const void* v, const void* dout,
                     const int32_t* off, double* dq, double* dk, double* dv) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int h = 0; h < c->H; ++h) backward_head(c, q, k, v, dout, off, h, dq, dk, dv);
}

/* ---- per-head offsets ------------------------------------------------------
   The section learns offsets for each token and each attention head m.  With
   integer offsets of one 3-vector per (head, query), head h is the computation
   above with that head's offsets: off_heads is int32 [H][N][3]. */

void oracle_forward_heads(const oracle_cfg* c, const void* q, const void* k, const void* v, const int32_t* off_heads,
                          double* out, double* lse) {
  const int64_t N = (int64_t)c->F * c->Hp * c->Wp, K = (int64_t)c->kt * c->ky * c->kx;
#pragma omp parallel
  {
    int64_t* keys = malloc(sizeof(int64_t) * K);
    double* p = malloc(sizeof(double) * K);
#pragma omp for schedule(dynamic, 64)
    for (int64_t r = 0; r < N * c->H; ++r) {
      const int64_t n = r / c->H;
      const int h = (int)(r % c->H);
      const int32_t* off = off_heads + (size_t)3 * N * h;
      lse[(int64_t)h * N + n] = attend(c, q, k, v, off, n, h, keys, p, out + (size_t)r * c->D);
    }
    free(keys);
    free(p);
  }
}

void oracle_backward_heads(const oracle_cfg* c, const void* q, const void* k, const void* v, const void* dout,
                           const int32_t* off_heads, double* dq, double* dk, double* dv) {
  const int64_t N = (int64_t)c->F * c->Hp * c->Wp;
#pragma omp parallel for schedule(dynamic, 1)
  for (int h = 0; h < c->H; ++h) backward_head(c, q, k, v, dout, off_heads + (size_t)3 * N * h, h, dq, dk, dv);
}

/* dq for a list of rows r = n * H + h: dq[i][D]. */
void oracle_backward_q_rows(const oracle_cfg* c, const void* q, const void* k, const void* v, const void* dout,
                            const int32_t* off, int64_t nrows, const int64_t* rows, double* dq) {
  const int64_t K = (int64_t)c->kt * c->ky * c->kx;
  const int D = c->D;
#pragma omp parallel
  {
    int64_t* keys = malloc(sizeof(int64_t) * K);
    double* p = malloc(sizeof(double) * K);
    double o[MAXD], dor[MAXD], row[MAXD];
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; ++i) {
      const int64_t n = rows[i] / c->H;
      const int h = (int)(rows[i] % c->H);
      attend(c, q, k, v, off, n, h, keys, p, o);
      load_row(c, dout, n, h, dor);
      const double delta = dot(dor, o, D);
      double* dqr = dq + (size_t)i * D;
      for (int e = 0; e < D; ++e) dqr[e] = 0.0;
      for (int j = 0; j < K; ++j) {
        load_row(c, v, keys[j], h, row);
        const double ds = p[j] * (dot(dor, row, D) - delta);
        load_row(c, k, keys[j], h, row);
        for (int e = 0; e < D; ++e) dqr[e] += c->scale * ds * row[e];
      }
    }
    free(keys);
    free(p);
  }
}

/* dk, dv for a list of key rows r = j * H + h: dk[i][D], dv[i][D].
   Key-centric: every query whose window can contain key j lies within
   2 * (k_d - 1) / 2 + max|o_d| of j along each axis (the clamp moves a window
   by at most (k_d - 1) / 2 past the shifted centre), so the queries of that box
   are scanned and those whose window holds j contribute. */
void oracle_backward_kv_rows(const oracle_cfg* c, const void* q, const void* k, const void* v, const void* dout,
                             const int32_t* off, int64_t nrows, const int64_t* rows, double* dk, double* dv) {
  const int64_t N = (int64_t)c->F * c->Hp * c->Wp, K = (int64_t)c->kt * c->ky * c->kx;
  const int D = c->D;
  int64_t maxo[3] = {0, 0, 0};
  for (int64_t n = 0; n < N; ++n)
    for (int d = 0; d < 3; ++d) {
      int64_t a = off[3 * n + d];
      if (a < 0) a = -a;
      if (a > maxo[d]) maxo[d] = a;
    }
  const int64_t R[3] = {2 * ((c->kt - 1) / 2) + maxo[0], 2 * ((c->ky - 1) / 2) + maxo[1],
                        2 * ((c->kx - 1) / 2) + maxo[2]};
  const int64_t G[3] = {c->F, c->Hp, c->Wp};
  const int64_t kk[3] = {c->kt, c->ky, c->kx};
#pragma omp parallel
  {
    int64_t* keys = malloc(sizeof(int64_t) * K);
    double* p = malloc(sizeof(double) * K);
    double o[MAXD], qr[MAXD], dor[MAXD], row[MAXD];
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; ++i) {
      const int64_t j = rows[i] / c->H;
      const int h = (int)(rows[i] % c->H);
      const int64_t jp[3] = {j / ((int64_t)c->Hp * c->Wp), (j / c->Wp) % c->Hp, j % c->Wp};
      int64_t lo[3], hi[3];
      for (int d = 0; d < 3; ++d) {
        lo[d] = jp[d] - R[d] < 0 ? 0 : jp[d] - R[d];
        hi[d] = jp[d] + R[d] > G[d] - 1 ? G[d] - 1 : jp[d] + R[d];
      }
      double* dkr = dk + (size_t)i * D;
      double* dvr = dv + (size_t)i * D;
      for (int e = 0; e < D; ++e) dkr[e] = dvr[e] = 0.0;
      for (int64_t t = lo[0]; t <= hi[0]; ++t)
        for (int64_t y = lo[1]; y <= hi[1]; ++y)
          for (int64_t x = lo[2]; x <= hi[2]; ++x) {
            const int64_t n = (t * c->Hp + y) * c->Wp + x;
            int64_t s[3];
            query_start(c, off, n, s);
            int inside = 1;
            for (int d = 0; d < 3; ++d) inside &= (jp[d] >= s[d]) && (jp[d] < s[d] + kk[d]);
            if (!inside) continue;
            attend(c, q, k, v, off, n, h, keys, p, o);
            const int64_t idx = ((jp[0] - s[0]) * c->ky + (jp[1] - s[1])) * c->kx + (jp[2] - s[2]);
            load_row(c, q, n, h, qr);
            load_row(c, dout, n, h, dor);
            load_row(c, v, j, h, row);
            const double ds = p[idx] * (dot(dor, row, D) - dot(dor, o, D));
            for (int e = 0; e < D; ++e) {
              dkr[e] += c->scale * ds * qr[e];
              dvr[e] += p[idx] * dor[e];
            }
          }
    }
    free(keys);
    free(p);
  }
}

/* ---- sampled windows: real offsets and trilinear sampling --------------------
   The section samples keys and values from XW_k and XW_v at real positions by
   trilinear interpolation (the implementation paragraph: grid_sample, bilinear mode,
   on 5-D tensors) and takes the softmax over the kt x kh x kw samples.  Positions
   are in token units along (t, y, x); a sample at P blends the 8 grid rows
   floor(P) + {0,1}^3 with weights prod_d (bit_d ? f_d : 1 - f_d), f = P - floor(P);
   rows outside the grid count as zero (grid_sample's default zero padding, with
   align_corners semantics: integer positions are the grid points).

   Offsets are float64 with element strides (sn, sh, ss) between tokens, heads and
   samples (0 = shared), three consecutive values (dt, dy, dx) per entry.  Two
   readings of where sample (u, v, w) of the query at p = (t, y, x) sits:
     box  (mode 0): one offset o per (query, head), shared by its samples; the window
                    is the kt x ky x kx box starting at
                      s_d = min(max(p_d + o_d - (k_d - 1) / 2, 0), G_d - k_d)  (real)
                    and sample (u, v, w) sits at s + (u, v, w).  Integer offsets give
                    exactly the integer windows above (the clamp keeps every sample
                    inside the grid).
     free (mode 1): sample (u, v, w) sits at p + (u - r_t, v - r_y, w - r_x) plus its
                    own offset (the deformable-convolution reading: grid term plus
                    learned offset), zero padded where it leaves the grid.
   Backward adds the gradient of the offsets through the interpolation weights
   (d w / d P_d = (bit_d ? 1 : -1) prod_{d' != d} ...); in box mode through the
   clamp as well (derivative 1 strictly inside (0, G_d - k_d), else 0). */

static void sample_positions(const oracle_cfg* c, const double* off, int64_t sn, int64_t sh, int64_t ss, int mode,
                             int64_t n, int h, double* P, int active[3]) {
  const int64_t plane = (int64_t)c->Hp * c->Wp;
  const double p[3] = {(double)(n / plane), (double)((n / c->Wp) % c->Hp), (double)(n % c->Wp)};
  const int kk[3] = {c->kt, c->ky, c->kx};
  const double G[3] = {c->F, c->Hp, c->Wp};
  const double* o = off + n * sn + (int64_t)h * sh;
  double s[3];
  for (int d = 0; d < 3; ++d) {
    const double x = p[d] + o[d] - (kk[d] - 1) / 2;
    s[d] = x < 0 ? 0 : (x > G[d] - kk[d] ? G[d] - kk[d] : x);
    active[d] = x > 0 && x < G[d] - kk[d];
  }
  int j = 0;
  for (int u = 0; u < c->kt; ++u)
    for (int v = 0; v < c->ky; ++v)
      for (int w = 0; w < c->kx; ++w, ++j) {
        const int g[3] = {u, v, w};
        for (int d = 0; d < 3; ++d) {
          if (mode == 0)
            P[3 * j + d] = s[d] + g[d];
          else
            P[3 * j + d] = p[d] + g[d] - (kk[d] - 1) / 2 + o[(int64_t)j * ss + d];
        }
      }
}

/* The 8 corners of a sample at P: token ids (-1 outside the grid), weights and the
   weights' derivatives along t, y, x. */
static void corners(const oracle_cfg* c, const double* P, int64_t tok[8], double w[8], double dw[8][3]) {
  const int64_t G[3] = {c->F, c->Hp, c->Wp};
  int64_t i0[3];
  double f[3];
  for (int d = 0; d < 3; ++d) {
    i0[d] = (int64_t)floor(P[d]);
    f[d] = P[d] - (double)i0[d];
  }
  for (int cn = 0; cn < 8; ++cn) {
    const int b[3] = {(cn >> 2) & 1, (cn >> 1) & 1, cn & 1};
    double phi[3];
    int inside = 1;
    int64_t idx[3];
    for (int d = 0; d < 3; ++d) {
      idx[d] = i0[d] + b[d];
      inside &= idx[d] >= 0 && idx[d] < G[d];
      phi[d] = b[d] ? f[d] : 1.0 - f[d];
    }
    tok[cn] = inside ? (idx[0] * c->Hp + idx[1]) * c->Wp + idx[2] : -1;
    w[cn] = phi[0] * phi[1] * phi[2];
    for (int d = 0; d < 3; ++d) {
      double g = b[d] ? 1.0 : -1.0;
      for (int e = 0; e < 3; ++e)
        if (e != d) g *= phi[e];
      dw[cn][d] = g;
    }
  }
}

/* Trilinear sample of head h of `base` at P into out[D]. */
static void sample_row(const oracle_cfg* c, const void* base, const double* P, int h, double* out) {
  int64_t tok[8];
  double w[8], dw[8][3], row[MAXD];
  corners(c, P, tok, w, dw);
  for (int e = 0; e < c->D; ++e) out[e] = 0.0;
  for (int cn = 0; cn < 8; ++cn) {
    if (tok[cn] < 0) continue;
    load_row(c, base, tok[cn], h, row);
    for (int e = 0; e < c->D; ++e) out[e] += w[cn] * row[e];
  }
}

/* Attention of (query n, head h) over its K samples: weights p[K], output o[D];
   returns the natural-log log-sum-exp. */
static double attend_sampled(const oracle_cfg* c, const void* q, const void* k, const void* v, const double* off,
                             int64_t sn, int64_t sh, int64_t ss, int mode, int64_t n, int h, double* P, double* p,
                             double* o) {
  const int K = c->kt * c->ky * c->kx, D = c->D;
  double qr[MAXD], row[MAXD];
  int active[3];
  sample_positions(c, off, sn, sh, ss, mode, n, h, P, active);
  load_row(c, q, n, h, qr);
  double m = -INFINITY;
  for (int j = 0; j < K; ++j) {
    sample_row(c, k, P + 3 * j, h, row);
    p[j] = c->scale * dot(qr, row, D);
    if (p[j] > m) m = p[j];
  }
  double sum = 0.0;
  for (int j = 0; j < K; ++j) sum += exp(p[j] - m);
  const double lse = m + log(sum);
  for (int j = 0; j < K; ++j) p[j] = exp(p[j] - lse);
  for (int e = 0; e < D; ++e) o[e] = 0.0;
  for (int j = 0; j < K; ++j) {
    sample_row(c, v, P + 3 * j, h, row);
    for (int e = 0; e < D; ++e) o[e] += p[j] * row[e];
  }
  return lse;
}

/* O [N][H][D] and LSE [H][N] with sampled windows. */
void oracle_sampled_forward(const oracle_cfg* c, const void* q, const void* k, const void* v, const double* off,
                            int64_t sn, int64_t sh, int64_t ss, int mode, double* out, double* lse) {
  const int64_t N = (int64_t)c->F * c->Hp * c->Wp, K = (int64_t)c->kt * c->ky * c->kx;
#pragma omp parallel
  {
    double* P = malloc(sizeof(double) * 3 * K);
    double* p = malloc(sizeof(double) * K);
#pragma omp for schedule(dynamic, 64)
    for (int64_t r = 0; r < N * c->H; ++r) {
      const int64_t n = r / c->H;
      const int h = (int)(r % c->H);
      lse[(int64_t)h * N + n] = attend_sampled(c, q, k, v, off, sn, sh, ss, mode, n, h, P, p, out + (size_t)r * c->D);
    }
    free(P);
    free(p);
  }
}

/* dq, dk, dv [N][H][D] and the offset gradient of every (query, head) (box mode,
   doff [N][H][3]) or every (query, head, sample) (free mode, doff [N][H][K][3]),
   each offset entry taken as its own variable (sums over shared entries are the
   caller's).  One head per thread; queries in order, scattering into the 8 corner
   rows of each sample. */
void oracle_sampled_backward(const oracle_cfg* c, const void* q, const void* k, const void* v, const void* dout,
                             const double* off, int64_t sn, int64_t sh, int64_t ss, int mode, double* dq, double* dk,
                             double* dv, double* doff) {
  const int64_t N = (int64_t)c->F * c->Hp * c->Wp, K = (int64_t)c->kt * c->ky * c->kx;
  const int D = c->D;
  memset(dk, 0, sizeof(double) * N * c->H * D);
  memset(dv, 0, sizeof(double) * N * c->H * D);
#pragma omp parallel for schedule(dynamic, 1)
  for (int h = 0; h < c->H; ++h) {
    double* P = malloc(sizeof(double) * 3 * K);
    double* p = malloc(sizeof(double) * K);
    double o[MAXD], qr[MAXD], dor[MAXD], row[MAXD], kt_[MAXD], vt[MAXD];
    for (int64_t n = 0; n < N; ++n) {
      int active[3];
      attend_sampled(c, q, k, v, off, sn, sh, ss, mode, n, h, P, p, o);
      sample_positions(c, off, sn, sh, ss, mode, n, h, P, active);
      load_row(c, q, n, h, qr);
      load_row(c, dout, n, h, dor);
      const double delta = dot(dor, o, D);
      double* dqr = dq + ((size_t)n * c->H + h) * D;
      for (int e = 0; e < D; ++e) dqr[e] = 0.0;
      double gbox[3] = {0, 0, 0};
      for (int j = 0; j < K; ++j) {
        sample_row(c, k, P + 3 * j, h, kt_);
        sample_row(c, v, P + 3 * j, h, vt);
        const double dz = p[j] * (dot(dor, vt, D) - delta);
        for (int e = 0; e < D; ++e) dqr[e] += c->scale * dz * kt_[e];
        int64_t tok[8];
        double w[8], dw[8][3], gP[3] = {0, 0, 0};
        corners(c, P + 3 * j, tok, w, dw);
        for (int cn = 0; cn < 8; ++cn) {
          if (tok[cn] < 0) continue;
          double* dkr = dk + ((size_t)tok[cn] * c->H + h) * D;
          double* dvr = dv + ((size_t)tok[cn] * c->H + h) * D;
          for (int e = 0; e < D; ++e) {
            dkr[e] += w[cn] * c->scale * dz * qr[e];
            dvr[e] += w[cn] * p[j] * dor[e];
          }
          load_row(c, k, tok[cn], h, row);
          const double sk = c->scale * dz * dot(qr, row, D);
          load_row(c, v, tok[cn], h, row);
          const double sv = p[j] * dot(dor, row, D);
          for (int d = 0; d < 3; ++d) gP[d] += dw[cn][d] * (sk + sv);
        }
        if (mode == 0) {
          for (int d = 0; d < 3; ++d) gbox[d] += gP[d];
        } else {
          double* g = doff + (((size_t)n * c->H + h) * K + j) * 3;
          for (int d = 0; d < 3; ++d) g[d] = gP[d];
        }
      }
      if (mode == 0) {
        double* g = doff + ((size_t)n * c->H + h) * 3;
        for (int d = 0; d < 3; ++d) g[d] = active[d] ? gbox[d] : 0.0;
      }
    }
    free(P);
    free(p);
  }
}

/* ---- depthwise 3-D convolution ------------------------------------------------
   The first term of Eq. (1), and the first stage of the offset predictor (the
   implementation paragraph: nn.Conv3d with groups equal to the hidden size, i.e. one
   ct x cy x cx filter per channel).  Cross-correlation over the T x H' x W' grid with
   zero padding that keeps the grid ("same"; extents odd):
     y[n, c] = b[c] + sum_{a, e, f} w[c][a][e][f] x[(t + a - rt, y + e - ry, x + f - rx), c]
   x is [N][C] (fp32, bf16 bits or fp64, `dtype` as above); w [C][ct][cy][cx], b [C]
   and y [N][C] are fp64.  Backward: dx[n, c] = sum_{a,e,f} w[c][a][e][f] dy[n - (a - rt,
   e - ry, f - rx), c], dw[c][a][e][f] = sum_n dy[n, c] x[n + (a - rt, e - ry, f - rx), c],
   db[c] = sum_n dy[n, c]. */

static double load_elem(int dtype, const void* base, size_t i) {
  if (dtype == 0) return ((const float*)base)[i];
  if (dtype == 2) return ((const double*)base)[i];
  uint32_t b = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &b, 4);
  return f;
}

void oracle_dwconv3d_forward(const void* x, int dtype, const double* w, const double* b, int F, int Hp, int Wp, int C,
                             int ct, int cy, int cx, double* y) {
  const int64_t N = (int64_t)F * Hp * Wp;
  const int rt = (ct - 1) / 2, ry = (cy - 1) / 2, rx = (cx - 1) / 2;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    const int64_t t = n / ((int64_t)Hp * Wp), yy = (n / Wp) % Hp, xx = n % Wp;
    for (int c = 0; c < C; ++c) {
      double s = b ? b[c] : 0.0;
      for (int a = 0; a < ct; ++a)
        for (int e = 0; e < cy; ++e)
          for (int f = 0; f < cx; ++f) {
            const int64_t ts = t + a - rt, ys = yy + e - ry, xs = xx + f - rx;
            if (ts < 0 || ts >= F || ys < 0 || ys >= Hp || xs < 0 || xs >= Wp) continue;
            const int64_t m = (ts * Hp + ys) * Wp + xs;
            s += w[(((size_t)c * ct + a) * cy + e) * cx + f] * load_elem(dtype, x, (size_t)m * C + c);
          }
      y[(size_t)n * C + c] = s;
    }
  }
}

void oracle_dwconv3d_backward(const void* x, int dtype, const double* w, const double* dy, int F, int Hp, int Wp,
                              int C, int ct, int cy, int cx, double* dx, double* dw, double* db) {
  const int64_t N = (int64_t)F * Hp * Wp;
  const int rt = (ct - 1) / 2, ry = (cy - 1) / 2, rx = (cx - 1) / 2;
  const int taps = ct * cy * cx;
  /* dx: gather form, every input position collects the outputs whose window holds it */
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    const int64_t t = n / ((int64_t)Hp * Wp), yy = (n / Wp) % Hp, xx = n % Wp;
    for (int c = 0; c < C; ++c) {
      double s = 0.0;
      for (int a = 0; a < ct; ++a)
        for (int e = 0; e < cy; ++e)
          for (int f = 0; f < cx; ++f) {
            const int64_t to = t - (a - rt), yo = yy - (e - ry), xo = xx - (f - rx);
            if (to < 0 || to >= F || yo < 0 || yo >= Hp || xo < 0 || xo >= Wp) continue;
            const int64_t m = (to * Hp + yo) * Wp + xo;
            s += w[(((size_t)c * ct + a) * cy + e) * cx + f] * dy[(size_t)m * C + c];
          }
      dx[(size_t)n * C + c] = s;
    }
  }
  /* dw, db: one channel per thread, tokens in order */
#pragma omp parallel for schedule(static)
  for (int c = 0; c < C; ++c) {
    double sb = 0.0;
    for (int k = 0; k < taps; ++k) dw[(size_t)c * taps + k] = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double g = dy[(size_t)n * C + c];
      sb += g;
      const int64_t t = n / ((int64_t)Hp * Wp), yy = (n / Wp) % Hp, xx = n % Wp;
      for (int a = 0; a < ct; ++a)
        for (int e = 0; e < cy; ++e)
          for (int f = 0; f < cx; ++f) {
            const int64_t ts = t + a - rt, ys = yy + e - ry, xs = xx + f - rx;
            if (ts < 0 || ts >= F || ys < 0 || ys >= Hp || xs < 0 || xs >= Wp) continue;
            const int64_t m = (ts * Hp + ys) * Wp + xs;
            dw[(size_t)c * taps + (a * cy + e) * cx + f] += g * load_elem(dtype, x, (size_t)m * C + c);
          }
    }
    db[c] = sb;
  }
}
