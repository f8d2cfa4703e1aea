/*
 * Seeded synthetic inputs for the CRISP sparse-prefill path.
 *
 * This file only prepares inputs: Gaussian base tensors, rotary position
 * embedding, additive planting of attention structure and rounding to the
 * storage precision.  It holds none of the method's arithmetic (no scores,
 * softmax, routing or selection), and both the CPU oracle and the GPU path
 * consume the exact bytes it writes.
 *
 * Random numbers: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), one independent stream per
 * (seed, tensor, head, row), so the output does not depend on thread count.
 * Normals come from the Box-Muller transform in double precision.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t next64(uint64_t* s) {
  *s += 0x9E3779B97F4A7C15ULL;
  return mix64(*s);
}

static inline double unit_open(uint64_t x) { /* (0,1) */
  return ((double)(x >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

static inline float round_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u; /* round to nearest even */
  memcpy(&f, &u, 4);
  return f;
}

/* Fill out[heads][n][d] (fp32 storage).
 *   x = scale * N(0,1)                      base value
 *   x = rope(x, position = row)             if rope_theta > 0 (rotate-half pairs k, k + d/2)
 *   x += head_add[h][:]                     if head_add (e.g. a query-side planted direction)
 *   x += row_gain[h][row] * head_dir[h][:]  if row_gain (key-side planted sinks / columns)
 * then rounded once to fp32, and to bf16 (round to nearest even) if round_bf16. */
void synth_fill(float* out, int32_t heads, int64_t n, int64_t row_start, int32_t d, uint64_t seed,
                uint32_t tensor_id, double scale, double rope_theta, const double* head_add,
                const double* row_gain, const double* head_dir, int32_t round_bf16) {
  const int64_t rows = n - row_start;
  const int32_t half = d / 2;
  double* cs = NULL;
  if (rope_theta > 0.0) {
    cs = (double*)malloc(sizeof(double) * 2 * (size_t)rows * half);
#pragma omp parallel for schedule(static)
    for (int64_t i = row_start; i < n; ++i) {
      for (int32_t k = 0; k < half; ++k) {
        double inv_freq = pow(rope_theta, -2.0 * (double)k / (double)d);
        double ang = (double)i * inv_freq;
        cs[(2 * (i - row_start)) * half + k] = cos(ang);
        cs[(2 * (i - row_start) + 1) * half + k] = sin(ang);
      }
    }
  }
  const uint64_t sk = mix64(seed);
#pragma omp parallel for collapse(2) schedule(static)
  for (int32_t h = 0; h < heads; ++h) {
    for (int64_t i = row_start; i < n; ++i) {
      double x[256];
      double y[256];
      uint64_t st = sk ^ mix64(((uint64_t)tensor_id << 56) ^ ((uint64_t)h << 40) ^ (uint64_t)i);
      for (int32_t k = 0; k < d; k += 2) {
        double u1 = unit_open(next64(&st));
        double u2 = unit_open(next64(&st));
        double r = sqrt(-2.0 * log(u1));
        x[k] = scale * r * cos(6.283185307179586 * u2);
        x[k + 1] = scale * r * sin(6.283185307179586 * u2);
      }
      if (cs) {
        const double* c = cs + (2 * (i - row_start)) * half;
        const double* s = cs + (2 * (i - row_start) + 1) * half;
        for (int32_t k = 0; k < half; ++k) {
          y[k] = x[k] * c[k] - x[k + half] * s[k];
          y[k + half] = x[k + half] * c[k] + x[k] * s[k];
        }
      } else {
        for (int32_t k = 0; k < d; ++k) y[k] = x[k];
      }
      if (head_add)
        for (int32_t k = 0; k < d; ++k) y[k] += head_add[(size_t)h * d + k];
      if (row_gain) {
        double g = row_gain[(size_t)h * n + i];
        if (g != 0.0)
          for (int32_t k = 0; k < d; ++k) y[k] += g * head_dir[(size_t)h * d + k];
      }
      float* o = out + ((size_t)h * rows + (i - row_start)) * d;
      for (int32_t k = 0; k < d; ++k) {
        float f = (float)y[k];
        o[k] = round_bf16 ? round_to_bf16(f) : f;
      }
    }
  }
  free(cs);
}

/* fp32 -> bf16 bit patterns (round to nearest even), for uploading stored values. */
void synth_to_bf16_bits(const float* in, uint16_t* out, int64_t count) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) {
    uint32_t u;
    memcpy(&u, &in[i], 4);
    u = u + 0x7FFFu + ((u >> 16) & 1u);
    out[i] = (uint16_t)(u >> 16);
  }
}
