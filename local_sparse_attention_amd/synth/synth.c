/*
 * Seeded synthetic inputs for 3D Deformable Slide Attention workloads.
 *
 * This module only draws random numbers; it holds none of the attention
 * arithmetic.  Both the GPU tests and the CPU oracle take their inputs from
 * here, so the two sides see bit-identical values.
 *
 * Generator (counter based, so the values do not depend on the thread count):
 *   - stream state   s0 = mix64((seed << 16) ^ stream)
 *   - word number i  w_i = mix64(s0 + (i + 1) * 0x9E3779B97F4A7C15)
 *     i.e. the i-th output of SplitMix64 (Steele, Lea & Flood, "Fast
 *     splittable pseudorandom number generators", OOPSLA 2014) started at s0,
 *     where mix64 is SplitMix64's output function.
 *   - uniform        u(i) = (w_i >> 11) * 2^-53 in [0, 1)
 *   - normal N(0,1)  element e uses the pair j = e / 2:
 *                    u1 = 1 - u(2j) in (0, 1], u2 = u(2j + 1),
 *                    r = sqrt(-2 ln u1); even e -> r cos(2 pi u2),
 *                    odd e -> r sin(2 pi u2)   (Box & Muller, 1958),
 *                    evaluated in double.
 *   - fp32 values are the double value times `scale`, rounded to nearest
 *     fp32; bf16 values are that fp32 rounded to nearest-even bf16.
 *
 * Streams: q = 0, k = 1, v = 2, dO = 3, block / per-token offsets = 4,
 * jitter = 5, drift = 6.  Tensor element e of a [N][H][D] tensor is word e.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_state(uint64_t seed, uint64_t stream) {
  return mix64((seed << 16) ^ stream);
}

static inline uint64_t word_at(uint64_t s0, uint64_t i) {
  return mix64(s0 + (i + 1) * 0x9E3779B97F4A7C15ULL);
}

static inline double unif_at(uint64_t s0, uint64_t i) {
  return (double)(word_at(s0, i) >> 11) * (1.0 / 9007199254740992.0);
}

static inline double normal_at(uint64_t s0, uint64_t e) {
  const uint64_t j = e >> 1;
  const double u1 = 1.0 - unif_at(s0, 2 * j);
  const double u2 = unif_at(s0, 2 * j + 1);
  const double r = sqrt(-2.0 * log(u1));
  const double a = 6.283185307179586476925 * u2;
  return (e & 1) ? r * sin(a) : r * cos(a);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  if ((b & 0x7f800000u) == 0x7f800000u) return (uint16_t)((b >> 16) | ((b & 0xffffu) ? 0x40u : 0u));
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

/* n normal values * scale, as fp32. Element e is word `first + e`. */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t first, int64_t n, double scale, float* out) {
  const uint64_t s0 = stream_state(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < n; ++e) out[e] = (float)(scale * normal_at(s0, first + (uint64_t)e));
}

/* Same values rounded once more to bf16 (stored as raw uint16 bits). */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t first, int64_t n, double scale, uint16_t* out) {
  const uint64_t s0 = stream_state(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < n; ++e) out[e] = f32_to_bf16_rne((float)(scale * normal_at(s0, first + (uint64_t)e)));
}

/* Per-token offsets, each component uniform in {lo, ..., hi}: word 3n + c. */
void synth_offsets_uniform(uint64_t seed, int64_t ntok, int lo, int hi, int32_t* off) {
  const uint64_t s0 = stream_state(seed, 4);
  const double span = (double)(hi - lo + 1);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < 3 * ntok; ++i) off[i] = lo + (int32_t)floor(unif_at(s0, (uint64_t)i) * span);
}

/* Per-token offsets round(sigma * Z) clamped to [-lim, lim]: word 3n + c. */
void synth_offsets_round_normal(uint64_t seed, int64_t ntok, double sigma, int lim, int32_t* off) {
  const uint64_t s0 = stream_state(seed, 4);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < 3 * ntok; ++i) {
    double z = round(sigma * normal_at(s0, (uint64_t)i));
    if (z < -lim) z = -lim;
    if (z > lim) z = lim;
    off[i] = (int32_t)z;
  }
}

/*
 * Smooth motion field on a grid F x Hp x Wp with `blk` x `blk` spatial blocks
 * (ceil(Hp/blk) x ceil(Wp/blk) of them).  Per block and component:
 *   drift == 0: b = round(sigma * Z), the same for every frame;
 *   drift != 0: b_0 = clamp(sigma * Z, -lim, lim),
 *               b_f = clamp(b_{f-1} + Z_f, -lim, lim) (real valued),
 *               and the frame uses round(b_f).
 * Token offset = block value of its block + J, J uniform in {-1, 0, 1}
 * (word 3n + c of stream 5).  Z is stream 4 word 3*block + c; Z_f is
 * stream 6 word 3*(f * nblocks + block) + c.
 */
void synth_offsets_blocks(uint64_t seed, int F, int Hp, int Wp, int blk, double sigma, int drift, double lim,
                          int32_t* off) {
  const int nby = (Hp + blk - 1) / blk, nbx = (Wp + blk - 1) / blk;
  const int64_t nb = (int64_t)nby * nbx;
  const uint64_t s_blk = stream_state(seed, 4), s_jit = stream_state(seed, 5), s_dr = stream_state(seed, 6);
  const int64_t plane = (int64_t)Hp * Wp;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b) {
    const int by = (int)(b / nbx), bx = (int)(b % nbx);
    for (int c = 0; c < 3; ++c) {
      double val = sigma * normal_at(s_blk, (uint64_t)(3 * b + c));
      if (drift) {
        if (val < -lim) val = -lim;
        if (val > lim) val = lim;
      } else {
        val = round(val);
      }
      for (int f = 0; f < F; ++f) {
        if (drift && f > 0) {
          val += normal_at(s_dr, (uint64_t)(3 * ((int64_t)f * nb + b) + c));
          if (val < -lim) val = -lim;
          if (val > lim) val = lim;
        }
        const int32_t base = (int32_t)(drift ? round(val) : val);
        for (int y = by * blk; y < by * blk + blk && y < Hp; ++y)
          for (int x = bx * blk; x < bx * blk + blk && x < Wp; ++x) {
            const int64_t n = (int64_t)f * plane + (int64_t)y * Wp + x;
            const int32_t j = -1 + (int32_t)floor(unif_at(s_jit, (uint64_t)(3 * n + c)) * 3.0);
            off[3 * n + c] = base + j;
          }
      }
    }
  }
}
