/*
 * CPU oracle for the shard-decomposed, flag-gated AG+GEMM.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it. It shares no code with the HIP library.
 *
 * What it computes ("Eliminating Multi-GPU Performance Taxes" analysis page,
 * symbol table and the AG+GEMM core identity):
 *   A (M x K) is split along K into W shards A_s (M x K/W), B is K x N, and
 *   C = [A_0 | A_1 | ... | A_{W-1}] . B = sum_{s=0}^{W-1} A_s . B[sK/W:(s+1)K/W, :]
 * The page also states the consumer's loop order: an outer loop over the
 * shards s = 0 .. W-1 and, inside it, the partial product of that shard.
 *
 * The oracle follows that order literally, in binary64:
 *   P_s[m,n] = sum_{j=0}^{KS-1} A_s[m,j] * B[s*KS + j, n]   (j ascending)
 *   C[m,n]   = sum_{s=0}^{W-1} P_s[m,n]                      (s ascending)
 * Inputs are binary16 bit patterns, decoded exactly to binary64 by
 * oracle_f16_to_f64 (written from the IEEE 754 binary16 format). A, B and C
 * are row-major; shard s is its own M x KS row-major buffer.
 *
 * Pins (see tests): exhaustive decode check against an independent binary16
 * implementation, W = 1 versus the direct product, an unrelated fp64 matrix
 * product, exact integer arithmetic (every input is a multiple of 2^-24), the
 * shard-order permutation invariance, and closed-form special cases.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <pthread.h>

/* binary16: sign(1) | exponent(5, bias 15) | fraction(10).
 * exponent 0: subnormal, value = fraction * 2^-24
 * exponent 31: infinity (fraction 0) or NaN
 * otherwise:   value = (1024 + fraction) * 2^(exponent - 25) */
double oracle_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1F;
  int f = h & 0x3FF;
  double v;
  if (e == 0) {
    v = (double)f;
    for (int i = 0; i < 24; i++) v *= 0.5; /* exact: scaling by powers of two */
  } else if (e == 31) {
    if (f == 0) v = 1.0 / 0.0;
    else v = 0.0 / 0.0;
  } else {
    v = (double)(1024 + f);
    int p = e - 25;
    if (p >= 0) for (int i = 0; i < p; i++) v *= 2.0;
    else for (int i = 0; i < -p; i++) v *= 0.5;
  }
  return sign ? -v : v;
}

static double* decode_all(const uint16_t* src, size_t n) {
  double* d = (double*)malloc(n * sizeof(double) + 1);
  if (!d) return NULL;
  for (size_t i = 0; i < n; i++) d[i] = oracle_f16_to_f64(src[i]);
  return d;
}

typedef struct {
  int W;
  int64_t M, KS, N;
  const double* const* A; /* W decoded shards, M x KS */
  const double* B;        /* K x N decoded */
  double* C;              /* M x N */
  double* P;              /* per-thread scratch row, N */
  int64_t row0, row1;
  int shard_only;         /* -1: full sum; s >= 0: only P_s */
} job_t;

/* For row m: P_s[m, :] accumulated over j ascending (each element's sum runs
 * j = 0, 1, ..., KS-1 in order), then added to C[m, :] in shard order. */
static void* row_worker(void* arg) {
  job_t* jb = (job_t*)arg;
  const int64_t KS = jb->KS, N = jb->N;
  for (int64_t m = jb->row0; m < jb->row1; m++) {
    double* c = jb->C + m * N;
    for (int64_t n = 0; n < N; n++) c[n] = 0.0;
    for (int s = 0; s < jb->W; s++) {
      if (jb->shard_only >= 0 && s != jb->shard_only) continue;
      double* p = jb->P;
      for (int64_t n = 0; n < N; n++) p[n] = 0.0;
      const double* a = jb->A[s] + m * KS;
      for (int64_t j = 0; j < KS; j++) {
        const double aj = a[j];
        const double* b = jb->B + (s * KS + j) * N;
        for (int64_t n = 0; n < N; n++) p[n] += aj * b[n];
      }
      for (int64_t n = 0; n < N; n++) c[n] += p[n];
    }
  }
  return NULL;
}

static int run(int W, int64_t M, int64_t K, int64_t N, const uint16_t* const* A_shards,
               const uint16_t* B, double* C, int nthreads, int shard_only) {
  if (W < 1 || M < 0 || K < 0 || N < 0 || (W && K % W) || !A_shards || !B || !C) return -1;
  if (M == 0 || N == 0) return 0;
  const int64_t KS = K / W;
  double** A = (double**)calloc((size_t)W, sizeof(double*));
  double* Bd = decode_all(B, (size_t)(K * N));
  int rc = 0;
  if (!A || !Bd) { rc = -2; goto done; }
  for (int s = 0; s < W; s++) {
    A[s] = decode_all(A_shards[s], (size_t)(M * KS));
    if (!A[s]) { rc = -2; goto done; }
  }
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > M) nthreads = (int)M;
  {
    pthread_t th[256];
    int created[256];
    job_t jobs[256];
    double* scratch = (double*)malloc((size_t)nthreads * (size_t)N * sizeof(double));
    if (!scratch) { rc = -2; goto done; }
    int64_t per = (M + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; t++) {
      jobs[t].W = W; jobs[t].M = M; jobs[t].KS = KS; jobs[t].N = N;
      jobs[t].A = (const double* const*)A; jobs[t].B = Bd; jobs[t].C = C;
      jobs[t].P = scratch + (size_t)t * (size_t)N;
      jobs[t].row0 = t * per;
      jobs[t].row1 = (t + 1) * per < M ? (t + 1) * per : M;
      jobs[t].shard_only = shard_only;
      created[t] = 0;
      if (jobs[t].row0 >= jobs[t].row1) continue;
      if (nthreads > 1 && pthread_create(&th[t], NULL, row_worker, &jobs[t]) == 0) created[t] = 1;
      else row_worker(&jobs[t]);
    }
    for (int t = 0; t < nthreads; t++) if (created[t]) pthread_join(th[t], NULL);
    free(scratch);
  }
done:
  if (A) for (int s = 0; s < W; s++) free(A[s]);
  free(A);
  free(Bd);
  return rc;
}

/* C (M x N, binary64) = sum_s A_s . B_s, shards in ascending order. */
int oracle_sharded_gemm(int W, int64_t M, int64_t K, int64_t N, const uint16_t* const* A_shards,
                        const uint16_t* B, double* C, int nthreads) {
  return run(W, M, K, N, A_shards, B, C, nthreads, -1);
}

/* P_s (M x N, binary64) = A_s . B[s*KS:(s+1)*KS, :] for one shard s. */
int oracle_shard_partial(int W, int s, int64_t M, int64_t K, int64_t N, const uint16_t* const* A_shards,
                         const uint16_t* B, double* P, int nthreads) {
  if (s < 0 || s >= W) return -1;
  return run(W, M, K, N, A_shards, B, P, nthreads, s);
}

/* The same definition evaluated at `count` chosen entries (rows[i], cols[i]):
 * out[i] = sum_s sum_j A_s[r, j] * B[s*KS + j, c], j ascending inside each shard,
 * shards ascending. Used for full-size workloads where only samples are checked. */
int oracle_sharded_gemm_entries(int W, int64_t M, int64_t K, int64_t N, const uint16_t* const* A_shards,
                                const uint16_t* B, int64_t count, const int64_t* rows, const int64_t* cols,
                                double* out) {
  if (W < 1 || K % W || !A_shards || !B || (count && (!rows || !cols || !out))) return -1;
  const int64_t KS = K / W;
  for (int64_t i = 0; i < count; i++) {
    int64_t r = rows[i], c = cols[i];
    if (r < 0 || r >= M || c < 0 || c >= N) return -1;
    double acc = 0.0;
    for (int s = 0; s < W; s++) {
      double p = 0.0;
      for (int64_t j = 0; j < KS; j++)
        p += oracle_f16_to_f64(A_shards[s][r * KS + j]) * oracle_f16_to_f64(B[(s * KS + j) * N + c]);
      acc += p;
    }
    out[i] = acc;
  }
  return 0;
}
