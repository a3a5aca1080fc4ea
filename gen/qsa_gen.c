/*
 * Seeded, counter-based input generator for the sparse-attention harness.
 *
 * This module only makes synthetic inputs (bf16 bit patterns). It holds none
 * of the method's arithmetic and is shared, as the single source of inputs,
 * by the CPU oracle's tests and by the GPU tests / benchmark.
 *
 * Definition (every element is a pure function of (seed, stream, index), so
 * any sub-range can be regenerated bit-identically and in parallel):
 *   key      = splitmix64(seed * 256 + stream)
 *   h(c)     = splitmix64(key ^ c)                       (64-bit word, counter c)
 *   element e of a normal stream takes the 16-bit lane (e & 3) of h(e >> 2)
 *   and maps it through NTAB: NTAB[i] = fp32(Phi^-1((i + 0.5) / 65536)),
 *   Phi the standard normal CDF; the value is then rounded to bf16 (RNE).
 * splitmix64 is the mixer published by Steele, Lea and Flood (OOPSLA 2014).
 * NTAB is built once per process by bisection on erfc() in double.
 *
 * Planted "needle" micro-blocks (indexer keys only): for batch row b and
 * window w of `window` tokens, one block of r tokens at block offset
 *   o(b, w) = splitmix64(key7 ^ ((b << 32) | w)) mod (window / r)
 * gets, on every dimension d of every token key, + 3 * u_d added in double
 * before rounding to fp32 and then bf16; u is the normalised vector of 64
 * draws (NTAB values, in double) from stream 6.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static inline uint64_t splitmix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ULL;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static float g_ntab[65536];
static int g_ntab_ready = 0;

static double phi_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

static void build_ntab(void) {
  if (g_ntab_ready) return;
  for (int i = 0; i < 65536; ++i) {
    double p = (i + 0.5) / 65536.0;
    double lo = -12.0, hi = 12.0;
    for (int it = 0; it < 80; ++it) {
      double mid = 0.5 * (lo + hi);
      if (phi_cdf(mid) < p) lo = mid; else hi = mid;
    }
    g_ntab[i] = (float)(0.5 * (lo + hi));
  }
  g_ntab_ready = 1;
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline uint64_t stream_key(uint64_t seed, uint32_t stream) {
  return splitmix64(seed * 256ull + (uint64_t)stream);
}

static inline uint32_t lane16(uint64_t key, uint64_t e) {
  uint64_t h = splitmix64(key ^ (e >> 2));
  return (uint32_t)((h >> (16 * (e & 3))) & 0xFFFFu);
}

/* Make sure the table exists (call once before any parallel use). */
void qsa_gen_init(void) { build_ntab(); }

/* Copy of the normal table, for tests of the generator itself. */
void qsa_gen_ntab(float* out) {
  build_ntab();
  memcpy(out, g_ntab, sizeof(g_ntab));
}

/* out[i] = bf16(NTAB[lane(e0 + i)] * scale), i < n. scale is applied in fp32
   (use a power of two to keep values exact). */
void qsa_gen_normal_bf16(uint64_t seed, uint32_t stream, uint64_t e0, uint64_t n, float scale,
                         uint16_t* out) {
  build_ntab();
  const uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    float v = g_ntab[lane16(key, e0 + (uint64_t)i)] * scale;
    out[i] = f32_to_bf16_rne(v);
  }
}

/* Integer-valued bf16 in [lo, hi] (uniform by modulo; exact in bf16 for |v| <= 256). */
void qsa_gen_int_bf16(uint64_t seed, uint32_t stream, uint64_t e0, uint64_t n, int lo, int hi,
                      uint16_t* out) {
  const uint64_t key = stream_key(seed, stream);
  const uint32_t span = (uint32_t)(hi - lo + 1);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    int v = lo + (int)(lane16(key, e0 + (uint64_t)i) % span);
    out[i] = f32_to_bf16_rne((float)v);
  }
}

/* The needle direction u (unit vector, double) of dimension d. */
void qsa_gen_needle_dir(uint64_t seed, int d, double* u) {
  build_ntab();
  const uint64_t key = stream_key(seed, 6);
  double nrm = 0.0;
  for (int i = 0; i < d; ++i) {
    u[i] = (double)g_ntab[lane16(key, (uint64_t)i)];
    nrm += u[i] * u[i];
  }
  nrm = sqrt(nrm);
  for (int i = 0; i < d; ++i) u[i] /= nrm;
}

/* Block offset (in blocks, within its window) of the needle of window w of batch row b. */
int64_t qsa_gen_needle_offset(uint64_t seed, int64_t b, int64_t w, int64_t window, int r) {
  const uint64_t key = stream_key(seed, 7);
  uint64_t h = splitmix64(key ^ (((uint64_t)b << 32) | (uint64_t)w));
  return (int64_t)(h % (uint64_t)(window / r));
}

/* Indexer keys of batch row b, tokens [s0, s0 + ns), dimension d, as the flat
   stream 5 of a [B, L, d] tensor (element index (b*L + s)*d + i). window == 0
   plants no needles. */
void qsa_gen_idx_keys_bf16(uint64_t seed, int64_t b, int64_t L, int64_t s0, int64_t ns, int d,
                           int64_t window, int r, uint16_t* out) {
  build_ntab();
  const uint64_t key = stream_key(seed, 5);
  double u[1024];
  if (window > 0) qsa_gen_needle_dir(seed, d, u);
#pragma omp parallel for schedule(static)
  for (int64_t s = s0; s < s0 + ns; ++s) {
    int needle = 0;
    if (window > 0) {
      int64_t w = s / window;
      int64_t o = qsa_gen_needle_offset(seed, b, w, window, r);
      needle = ((s % window) / r) == o;
    }
    uint16_t* row = out + (s - s0) * d;
    const uint64_t ebase = ((uint64_t)b * (uint64_t)L + (uint64_t)s) * (uint64_t)d;
    for (int i = 0; i < d; ++i) {
      float v = g_ntab[lane16(key, ebase + (uint64_t)i)];
      if (needle) v = (float)((double)v + 3.0 * u[i]);
      row[i] = f32_to_bf16_rne(v);
    }
  }
}
