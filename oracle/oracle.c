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

/* dq, dk, dv [N][H][D] for every row.  One head per thread; within a head the
   queries are visited in order and each scatters into the keys of its window. */
void oracle_backward(const oracle_cfg* c, const void* q, const void* k, const void* v, const void* dout,
                     const int32_t* off, double* dq, double* dk, double* dv) {
  const int64_t N = (int64_t)c->F * c->Hp * c->Wp, K = (int64_t)c->kt * c->ky * c->kx;
  const int D = c->D;
  memset(dk, 0, sizeof(double) * N * c->H * D);
  memset(dv, 0, sizeof(double) * N * c->H * D);
#pragma omp parallel for schedule(dynamic, 1)
  for (int h = 0; h < c->H; ++h) {
    int64_t* keys = malloc(sizeof(int64_t) * K);
    double* p = malloc(sizeof(double) * K);
    double o[MAXD], qr[MAXD], dor[MAXD], row[MAXD];
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
