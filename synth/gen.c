/*
 * Seeded synthetic inputs for the shard-decomposed GEMM: the activation A,
 * the weight B and the producer's release schedule.
 *
 * This module holds no arithmetic of the method itself. It is the one piece
 * shared by the CPU oracle and the GPU path, so that both see identical bytes.
 *
 * Value recipe (counter based, so any slice can be generated on its own):
 *   h    = splitmix64(seed XOR i)         i = row-major index in the unsharded matrix
 *   u    = h >> 40                         24 uniform bits
 *   x    = u * 2^-23 - 1                   exact in binary64, x in [-1, 1)
 *   bits = binary16(x), round to nearest, ties to even
 * splitmix64 is the mixing function of Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators" (OOPSLA 2014), as popularised by Vigna.
 *
 * Schedule recipe (the order and times at which the producer releases the
 * T = W*KT (shard, k-tile) flags):
 *   order:  Fisher-Yates shuffle of 0..T-1, for i = T-1 .. 1 swap i with
 *           j = ((splitmix64(seed XOR i) >> 32) * (i+1)) >> 32
 *   delays: d_p = floor(u_p * max_delay_ns / 2^24), u_p = splitmix64(seed XOR (2^32 + p)) >> 40
 *   offset: offset_ns[p] = d_0 + ... + d_p (cumulative), tile order[p] released at offset_ns[p]
 *
 * fp32 recipe (the per-rank partial outputs and log-sum-exp statistics fed to
 * the Flash-Decode combine): x = lo + (hi - lo) * u * 2^-24 in binary64 with
 * u = splitmix64(seed XOR i) >> 40, then rounded to binary32 (round to
 * nearest even). With lo = -1, hi = 1 every value is exact in binary32.
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <pthread.h>

static inline uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t synth_splitmix64(uint64_t x) { return splitmix64(x); }

/* binary64 -> binary16, round to nearest, ties to even. Written from the
 * IEEE 754-2008 binary16 format: 1 sign bit, 5 exponent bits (bias 15),
 * 10 fraction bits; subnormals below 2^-14; overflow to infinity.
 * Only finite inputs with |x| < 65520 occur here, but the routine handles
 * the general finite case. */
static uint16_t f64_to_f16_rne(double x) {
  uint64_t b;
  memcpy(&b, &x, 8);
  uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  int e = (int)((b >> 52) & 0x7FF);
  uint64_t m = b & 0xFFFFFFFFFFFFFull;
  if (e == 0x7FF) return (uint16_t)(sign | 0x7C00u | (m ? 0x200u : 0u));
  if (e == 0 && m == 0) return sign;
  /* value = (1.m) * 2^(e-1023) for normals; binary64 subnormals are far below
   * the binary16 range and round to zero below. */
  int E = e - 1023;
  uint64_t sig = (e == 0) ? m : (m | (1ull << 52)); /* 53-bit significand */
  if (e == 0) E = -1022;
  /* target: binary16 normal needs E >= -14; subnormal quantum is 2^-24. */
  int shift; /* right shift applied to the 53-bit significand */
  uint16_t exp_field;
  if (E >= -14) {
    shift = 52 - 10;
    exp_field = (uint16_t)(E + 15);
  } else {
    /* subnormal: value = sig * 2^(E-52); quantum 2^-24 -> shift = (-24) - (E-52) */
    shift = (-24) - (E - 52);
    exp_field = 0;
  }
  if (shift >= 64) return sign; /* below 2^-35: rounds to a signed zero */
  uint64_t q = sig >> shift;
  uint64_t rem = sig & ((1ull << shift) - 1);
  uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) q += 1;
  uint32_t out;
  if (exp_field == 0) {
    out = (uint32_t)q; /* may carry into the smallest normal (q == 1024), which is exactly right */
  } else {
    /* q holds the 11-bit significand with the hidden bit; carry may overflow to 2048 */
    if (q == 2048) { q = 1024; exp_field++; }
    if (exp_field >= 31) return (uint16_t)(sign | 0x7C00u);
    out = ((uint32_t)exp_field << 10) | (uint32_t)(q & 0x3FF);
  }
  return (uint16_t)(sign | out);
}

uint16_t synth_f64_to_f16(double x) { return f64_to_f16_rne(x); }

static inline double uniform_pm1(uint64_t seed, uint64_t i) {
  uint64_t u = splitmix64(seed ^ i) >> 40;
  return (double)u * (1.0 / 8388608.0) - 1.0; /* 2^-23 */
}

double synth_uniform(uint64_t seed, uint64_t i) { return uniform_pm1(seed, i); }

typedef struct {
  uint64_t seed;
  uint64_t start;
  uint16_t* out;
  size_t count;
} fill_job;

static void* fill_worker(void* arg) {
  fill_job* j = (fill_job*)arg;
  for (size_t k = 0; k < j->count; k++) j->out[k] = f64_to_f16_rne(uniform_pm1(j->seed, j->start + k));
  return NULL;
}

/* Fills out[k] = binary16 bits of element (start + k) of the stream `seed`. */
int synth_fill_f16(uint64_t seed, uint64_t start, uint16_t* out, size_t count, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if (count < (size_t)1 << 16) nthreads = 1;
  pthread_t th[64];
  int created[64];
  fill_job jobs[64];
  size_t per = (count + (size_t)nthreads - 1) / (size_t)nthreads;
  for (int t = 0; t < nthreads; t++) {
    created[t] = 0;
    size_t b = (size_t)t * per;
    if (b >= count) break;
    size_t n = (count - b < per) ? count - b : per;
    jobs[t].seed = seed; jobs[t].start = start + b; jobs[t].out = out + b; jobs[t].count = n;
    if (nthreads > 1 && pthread_create(&th[t], NULL, fill_worker, &jobs[t]) == 0) created[t] = 1;
    else fill_worker(&jobs[t]);
  }
  for (int t = 0; t < nthreads; t++) {
    if ((size_t)t * per >= count) break;
    if (created[t]) pthread_join(th[t], NULL);
  }
  return 0;
}

/* Fills out[k] = binary32 value of element (start + k) of the stream `seed` in [lo, hi). */
int synth_fill_f32(uint64_t seed, uint64_t start, float* out, size_t count, double lo, double hi) {
  for (size_t k = 0; k < count; k++) {
    uint64_t u = splitmix64(seed ^ (start + k)) >> 40;
    out[k] = (float)(lo + (hi - lo) * ((double)u * (1.0 / 16777216.0))); /* 2^-24 */
  }
  return 0;
}

/* Release schedule for T tiles: order[p] is the tile released p-th, at offset_ns[p]. */
int synth_schedule(uint64_t seed, int32_t T, int64_t max_delay_ns, int32_t* order, int64_t* offset_ns) {
  if (T < 1 || !order || !offset_ns || max_delay_ns < 0) return -1;
  for (int32_t i = 0; i < T; i++) order[i] = i;
  for (int32_t i = T - 1; i >= 1; i--) {
    uint64_t h = splitmix64(seed ^ (uint64_t)i) >> 32;
    int32_t j = (int32_t)((h * (uint64_t)(i + 1)) >> 32);
    int32_t t = order[i]; order[i] = order[j]; order[j] = t;
  }
  int64_t acc = 0;
  for (int32_t p = 0; p < T; p++) {
    uint64_t u = splitmix64(seed ^ ((1ull << 32) + (uint64_t)p)) >> 40;
    int64_t d = (int64_t)(((unsigned __int128)u * (uint64_t)max_delay_ns) >> 24);
    acc += d;
    offset_ns[p] = acc;
  }
  return 0;
}
