/*
 * Seeded synthetic input generator shared by the CPU oracle and the GPU
 * library's tests and benchmark.  It holds none of the MoE layer's
 * arithmetic: it only draws numbers and rounds them to the storage types
 * the layer consumes.
 *
 * Pseudo-random source: Marsaglia's xorshift32 (shift triple 13/17/5;
 * G. Marsaglia, "Xorshift RNGs", J. Stat. Softw. 8(14), 2003), the family
 * and the base seed 0x9E3779B9 that the qwen35moe golden-vector page names
 * (section "qwen35moe CPU-reference golden vectors", intro).  Instead of one
 * stream threaded through every tensor, each tensor row is its own stream,
 * seeded from (base seed, stream id) by the murmur3 32-bit finaliser, so
 * rows can be drawn in parallel and the result does not depend on the
 * thread count.
 *
 * Draw mappings:
 *   uniform  u = ((s >> 8) + 1) * 2^-24, in (0, 1]
 *   normal   Box-Muller in double (both outputs used, cos first), scaled by
 *            the standard deviation, rounded to fp32 (then to bf16 by
 *            round-to-nearest-even for bf16 tensors)
 *   bytes    the top 8 bits of a draw
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

static inline uint32_t fmix32(uint32_t h) {
  h ^= h >> 16; h *= 0x85EBCA6Bu;
  h ^= h >> 13; h *= 0xC2B2AE35u;
  h ^= h >> 16;
  return h;
}

uint32_t synth_stream_seed(uint32_t base, uint64_t stream) {
  uint32_t h = fmix32(base ^ fmix32((uint32_t)stream) ^ fmix32((uint32_t)(stream >> 32) * 0x9E3779B9u + 0x7F4A7C15u));
  return h ? h : 0x9E3779B9u;
}

static inline uint32_t xs32(uint32_t* s) {
  uint32_t x = *s;
  x ^= x << 13; x ^= x >> 17; x ^= x << 5;
  *s = x;
  return x;
}

static inline double unif(uint32_t* s) { return ((double)((xs32(s) >> 8) + 1u)) * (1.0 / 16777216.0); }

uint32_t synth_xorshift32_next(uint32_t s) { return xs32(&s); }

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u; memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

uint16_t synth_f32_to_bf16(float f) { return f32_to_bf16_rne(f); }

/* n normal draws from one stream; the odd tail takes only the cosine half. */
static void normal_stream(uint32_t seed, double stddev, float* out, size_t n) {
  uint32_t s = seed;
  const double two_pi = 6.283185307179586476925286766559;
  size_t i = 0;
  while (i < n) {
    double u1 = unif(&s), u2 = unif(&s);
    double r = sqrt(-2.0 * log(u1));
    out[i++] = (float)(stddev * r * cos(two_pi * u2));
    if (i < n) out[i++] = (float)(stddev * r * sin(two_pi * u2));
  }
}

/* rows x cols normal matrix, row r drawn from stream (stream0 + r). */
void synth_normal_f32(uint32_t base, uint64_t stream0, double stddev, int64_t rows, int64_t cols, float* out) {
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t r = 0; r < rows; ++r)
    normal_stream(synth_stream_seed(base, stream0 + (uint64_t)r), stddev, out + r * cols, (size_t)cols);
}

void synth_normal_bf16(uint32_t base, uint64_t stream0, double stddev, int64_t rows, int64_t cols, uint16_t* out) {
#pragma omp parallel
  {
    float buf[4096];
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < rows; ++r) {
      uint32_t seed = synth_stream_seed(base, stream0 + (uint64_t)r);
      /* a row longer than the buffer continues the same stream */
      uint32_t s = seed;
      const double two_pi = 6.283185307179586476925286766559;
      int64_t c = 0;
      while (c < cols) {
        int64_t m = cols - c < 4096 ? cols - c : 4096;
        int64_t j = 0;
        while (j < m) {
          double u1 = unif(&s), u2 = unif(&s);
          double rr = sqrt(-2.0 * log(u1));
          buf[j++] = (float)(stddev * rr * cos(two_pi * u2));
          if (j < m) buf[j++] = (float)(stddev * rr * sin(two_pi * u2));
        }
        for (j = 0; j < m; ++j) out[r * cols + c + j] = f32_to_bf16_rne(buf[j]);
        c += m;
      }
    }
  }
}

/* rows x cols uniform random bytes (the top 8 bits of each draw). */
void synth_bytes(uint32_t base, uint64_t stream0, int64_t rows, int64_t cols, uint8_t* out) {
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t r = 0; r < rows; ++r) {
    uint32_t s = synth_stream_seed(base, stream0 + (uint64_t)r);
    for (int64_t c = 0; c < cols; ++c) out[r * cols + c] = (uint8_t)(xs32(&s) >> 24);
  }
}

/* rows x cols bytes lo + (draw mod span): block exponents in [lo, lo+span). */
void synth_range_bytes(uint32_t base, uint64_t stream0, int64_t rows, int64_t cols, uint32_t lo, uint32_t span, uint8_t* out) {
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t r = 0; r < rows; ++r) {
    uint32_t s = synth_stream_seed(base, stream0 + (uint64_t)r);
    for (int64_t c = 0; c < cols; ++c) out[r * cols + c] = (uint8_t)(lo + xs32(&s) % span);
  }
}

/* Seeded Fisher-Yates shuffle of 0..n-1 (one stream). */
void synth_permutation(uint32_t base, uint64_t stream, int32_t n, int32_t* out) {
  uint32_t s = synth_stream_seed(base, stream);
  for (int32_t i = 0; i < n; ++i) out[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    int32_t j = (int32_t)(xs32(&s) % (uint32_t)(i + 1));
    int32_t t = out[i]; out[i] = out[j]; out[j] = t;
  }
}

/*
 * Router logits whose top-k load over experts is Zipf-skewed:
 * l[t][e] = -exponent * ln(rank[e]) + G[t][e], G ~ Gumbel(0,1) = -ln(-ln u),
 * rank a seeded permutation of 1..E (one stream), token t's Gumbel noise its
 * own stream.  Taking the k largest of these is sampling k experts without
 * replacement with probability proportional to rank^-exponent
 * (the Gumbel-top-k trick, Kool, van Hoof and Welling, ICML 2019).
 */
void synth_zipf_logits(uint32_t base, uint64_t stream0, int32_t T, int32_t E, double exponent, float* out) {
  int32_t perm[65536];
  if (E > 65536) return;
  synth_permutation(base, stream0, E, perm);
#pragma omp parallel for schedule(dynamic, 16)
  for (int32_t t = 0; t < T; ++t) {
    uint32_t s = synth_stream_seed(base, stream0 + 1u + (uint64_t)t);
    for (int32_t e = 0; e < E; ++e) {
      double u = unif(&s);
      if (u >= 1.0) u = 1.0 - 1.0 / 16777216.0; /* ln(1) = 0 would make -ln(0) */
      double g = -log(-log(u));
      out[(int64_t)t * E + e] = (float)(-exponent * log((double)(perm[e] + 1)) + g);
    }
  }
}
