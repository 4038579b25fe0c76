/*
 * Seeded synthetic inputs shared by the oracle and the GPU path.
 *
 * This file holds only random-number generation: no step of the decoder is
 * computed here.  Both sides receive the bytes it writes, so libm differences
 * between hosts cannot make the two sides disagree.
 *
 * Generator (counter based, so any element can be produced independently):
 *   sm(x)      = SplitMix64 output for state x (Steele, Lea, Flood 2014;
 *                constants as published by Vigna): z = x + 0x9E3779B97F4A7C15,
 *                z = (z ^ z>>30) * 0xBF58476D1CE4E5B9,
 *                z = (z ^ z>>27) * 0x94D049BB133111EB, return z ^ z>>31.
 *   key(s,t)   = sm(sm(s) + t)                    seed s, stream id t
 *   pair j     : r1 = sm(key + 2j), r2 = sm(key + 2j + 1)
 *                u1 = ((r1>>11)+1) * 2^-53  in (0,1]
 *                u2 =  (r2>>11)    * 2^-53  in [0,1)
 *                Box-Muller (1958): rad = sqrt(-2 ln u1),
 *                element 2j = rad cos(2 pi u2), element 2j+1 = rad sin(2 pi u2)
 *   value      = bf16 round-to-nearest-even of (float)(mean + std * z)
 *                (mean 0 for weights; mean 1 for the optional non-unit
 *                RMSNorm gains)
 *   token k    = sm(key(s,t) + k) mod vocab
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t sm(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ULL;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return sm(sm(seed) + stream);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) { /* inf / nan: keep, quiet nan */
    return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  }
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* n normal samples N(mean, std^2) rounded to bf16, for stream `stream`,
 * starting at element index `first` (so a tensor can be produced in pieces). */
void synth_normal_mean_bf16(uint64_t seed, uint64_t stream, double mean, double stdev,
                            uint64_t first, uint64_t n, uint16_t* out) {
  const uint64_t key = stream_key(seed, stream);
  const double two_pi = 6.283185307179586476925286766559;
  const double inv53 = 1.0 / 9007199254740992.0; /* 2^-53 */
  if (n == 0) return;
  /* pairs j0..j1 cover elements first..first+n-1; both outputs of a pair
     are computed together and stored when inside the range */
  const uint64_t j0 = first >> 1, j1 = (first + n - 1) >> 1;
  long long jj;
#pragma omp parallel for schedule(static)
  for (jj = (long long)j0; jj <= (long long)j1; ++jj) {
    uint64_t j = (uint64_t)jj;
    uint64_t r1 = sm(key + 2 * j), r2 = sm(key + 2 * j + 1);
    double u1 = (double)((r1 >> 11) + 1) * inv53;
    double u2 = (double)(r2 >> 11) * inv53;
    double rad = sqrt(-2.0 * log(u1));
    double ang = two_pi * u2;
    uint64_t e0 = 2 * j, e1 = 2 * j + 1;
    double z0 = stdev * rad * cos(ang), z1 = stdev * rad * sin(ang);
    if (mean != 0.0) { /* mean 0 keeps the signed zeros of the weight formula */
      z0 += mean;
      z1 += mean;
    }
    if (e0 >= first && e0 < first + n) out[e0 - first] = f32_to_bf16_rne((float)z0);
    if (e1 >= first && e1 < first + n) out[e1 - first] = f32_to_bf16_rne((float)z1);
  }
}

/* N(0, std^2): the weight generator */
void synth_normal_bf16(uint64_t seed, uint64_t stream, double stdev,
                       uint64_t first, uint64_t n, uint16_t* out) {
  synth_normal_mean_bf16(seed, stream, 0.0, stdev, first, n, out);
}

/* n tokens uniform in [0, vocab) for stream `stream`. */
void synth_tokens(uint64_t seed, uint64_t stream, int64_t vocab, uint64_t n,
                  int32_t* out) {
  const uint64_t key = stream_key(seed, stream);
  for (uint64_t k = 0; k < n; ++k) out[k] = (int32_t)(sm(key + k) % (uint64_t)vocab);
}

/* fill with a constant bf16 pattern (norm weights are 1.0 = 0x3F80) */
void synth_fill_u16(uint16_t v, uint64_t n, uint16_t* out) {
  long long i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < (long long)n; ++i) out[i] = v;
}

/* raw SplitMix64 value, exported so tests can pin the generator itself */
uint64_t synth_splitmix64(uint64_t x) { return sm(x); }
