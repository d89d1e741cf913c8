// Flag-gated shard-decomposed GEMM for few rows (M <= 8): streaming B.
//
// With one (or a handful of) rows of A, C = sum_s A_s . B[s*KS:(s+1)*KS, :]
// ("Eliminating Multi-GPU Performance Taxes" analysis page, AG+GEMM core
// identity) is bound by reading B once from HBM. The page's bandwidth budget
// for M = 1 notes that the data exchanged is tiny and launch costs dominate;
// here the goal is to stream B at HBM speed and hide the flag wait under it.
//
// Work split: one workgroup per (flag tile f = (s, kt), block of 512 columns).
// The four waves take interleaved rows of the tile's BKf rows of B; each lane
// owns 8 consecutive columns and keeps M x 8 fp32 sums. The B loads of the
// first rows are issued before the flag wait (B does not depend on the
// flag); A's k-tile is read only after the acquire. Per-tile partial sums go
// to a workspace; the last workgroup of a column block (counted with an
// acq_rel atomic) adds the T partials in tile order (shard-major, so shards
// are summed in ascending order) and writes C. The result does not depend on
// arrival order.
#include "agemm_internal.h"

namespace agemm {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kCols = 512;   // columns per workgroup: 64 lanes x 8

__device__ inline uint64_t wall_clock() { return __builtin_amdgcn_s_memrealtime(); }

template <int MT, bool GATED, bool OUTF32>
__global__ __launch_bounds__(kThreads) void gemm_small_m_kernel(SmallMArgs sa) {
  constexpr int kChunk = MT <= 2 ? 16 : 8;  // B rows in flight per lane
  const GemmArgs& g = sa.g;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int64_t M = g.M, N = g.N;
  const int NBLK = (int)((N + kCols - 1) / kCols);
  const int T = g.gate.t;
  const int bkf = (int)(g.KS / g.gate.kt);
  const int items = T * NBLK;
  const int rows_per_wave = bkf / 4;  // wave w takes rows w, w+4, w+8, ...

  extern __shared__ float lds[];  // A tile [4 waves][MT][bkf/4], then a [4][kCols] reduction buffer
  float* lds_a = lds;
  float* lds_r = lds + 4 * MT * (bkf / 4);
  __shared__ int s_abort;
  __shared__ int s_last;

  // Persistent loop over work items (flag tile f, column block nb), tile-major
  // so that items become ready in the producer's shard order.
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int f = item / NBLK;
    const int nb = item - f * NBLK;
    const int s = f / g.gate.kt;
    const int kt = f - s * g.gate.kt;
    const int64_t n = (int64_t)nb * kCols + lane * 8;
    const int64_t nl = n < N ? n : N - 8;  // idle lanes read a valid address
    const int64_t k0 = (int64_t)s * g.KS + (int64_t)kt * bkf;
    const _Float16* bp = g.B + (k0 + wave) * N + nl;
    const int64_t bstep = 4 * N;

    float acc[MT][8];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[m][j] = 0.f;

    // B does not depend on the flag: start streaming it before the wait.
    half8 buf[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) buf[i] = *reinterpret_cast<const half8*>(bp + i * bstep);

    __syncthreads();  // the previous item is done with LDS
    if constexpr (GATED) {
      if (tid == 0) {
        const uint64_t start = wall_clock();
        int abort = 0;
        uint32_t v = 0;
        while (true) {
          v = __hip_atomic_load(const_cast<uint32_t*>(g.gate.flags) + f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((int32_t)(v - g.gate.target) >= 0) break;
          if (wall_clock() - start > g.gate.timeout_ticks) {
            abort = 1;
            __hip_atomic_store(&g.gate.err->tile, (uint32_t)f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            __hip_atomic_store(&g.gate.err->target, g.gate.target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            __hip_atomic_store(&g.gate.err->seen, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            __hip_atomic_store(&g.gate.err->code, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        s_abort = abort;
      }
      __syncthreads();
      if (__builtin_amdgcn_readfirstlane(s_abort)) break;  // C is left undefined
    }
    // Stage A's k-tile (rows < M) in LDS as fp32, so that wave w finds its rows contiguous.
    {
      const _Float16* ap = g.a.base[s] + (int64_t)kt * bkf;
      for (int idx = tid; idx < MT * bkf; idx += kThreads) {
        const int m = idx / bkf;
        const int k = idx - m * bkf;
        const float v = (m < M) ? (float)ap[(int64_t)m * g.a.lda + k] : 0.f;
        lds_a[((k & 3) * MT + m) * rows_per_wave + (k >> 2)] = v;
      }
    }
    __syncthreads();

    const float* aw = lds_a + wave * MT * rows_per_wave;
    for (int r0 = 0; r0 < rows_per_wave; r0 += kChunk) {
#pragma unroll
      for (int i = 0; i < kChunk; ++i) {
        const half8 b = buf[i];
        // refill this slot with the row kChunk further on
        if (r0 + kChunk + i < rows_per_wave)
          buf[i] = *reinterpret_cast<const half8*>(bp + (r0 + kChunk + i) * bstep);
        float bf[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) bf[j] = (float)b[j];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const float a = aw[m * rows_per_wave + r0 + i];
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[m][j] = __builtin_fmaf(a, bf[j], acc[m][j]);
        }
      }
    }

    // Sum the four waves' partials (in wave order), one row of C at a time.
    float* ws_tile = sa.ws + (int64_t)f * M * N;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= M) break;
#pragma unroll
      for (int j = 0; j < 8; ++j) lds_r[wave * kCols + lane * 8 + j] = acc[m][j];
      __syncthreads();
      for (int c = tid; c < kCols; c += kThreads) {
        const int64_t col = (int64_t)nb * kCols + c;
        if (col < N) {
          float v = lds_r[c];
          v += lds_r[kCols + c];
          v += lds_r[2 * kCols + c];
          v += lds_r[3 * kCols + c];
          ws_tile[(int64_t)m * N + col] = v;
        }
      }
      __syncthreads();
    }

    // The last workgroup to finish a column block adds the T partials in tile order.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (tid == 0) {
      const uint32_t old = __hip_atomic_fetch_add(sa.counters + nb, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      s_last = (old == (uint32_t)(T - 1));
    }
    __syncthreads();
    if (!__builtin_amdgcn_readfirstlane(s_last)) continue;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    for (int idx = tid; idx < MT * kCols; idx += kThreads) {
      const int m = idx / kCols;
      const int c = idx - m * kCols;
      const int64_t col = (int64_t)nb * kCols + c;
      if (m < M && col < N) {
        float v = 0.f;
        for (int t = 0; t < T; ++t) v += sa.ws[((int64_t)t * M + m) * N + col];
        if constexpr (OUTF32) static_cast<float*>(g.C)[(int64_t)m * N + col] = v;
        else static_cast<_Float16*>(g.C)[(int64_t)m * N + col] = (_Float16)v;
      }
    }
    if (tid == 0) __hip_atomic_store(sa.counters + nb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

size_t small_m_lds_bytes(int mt, int bkf) { return sizeof(float) * (size_t)(mt * bkf + 4 * kCols); }

template <int MT>
hipError_t launch_mt(const SmallMArgs& a, bool out_f32, hipStream_t s) {
  const int bkf = (int)(a.g.KS / a.g.gate.kt);
  const int nblk = (int)((a.g.N + kCols - 1) / kCols);
  // Persistent grid of two workgroups per CU: well under what fits on a CU,
  // so producer workgroups always find room next to spinning consumers.
  const int64_t items = (int64_t)a.g.gate.t * nblk;
  const int64_t cap = 2 * (int64_t)a.g.num_cus;
  const dim3 grid((unsigned)(items < cap ? items : cap));
  const size_t lds = small_m_lds_bytes(MT, bkf);
  const bool gated = a.g.gate.flags != nullptr;
  if (gated) {
    if (out_f32) hipLaunchKernelGGL((gemm_small_m_kernel<MT, true, true>), grid, dim3(kThreads), lds, s, a);
    else hipLaunchKernelGGL((gemm_small_m_kernel<MT, true, false>), grid, dim3(kThreads), lds, s, a);
  } else {
    if (out_f32) hipLaunchKernelGGL((gemm_small_m_kernel<MT, false, true>), grid, dim3(kThreads), lds, s, a);
    else hipLaunchKernelGGL((gemm_small_m_kernel<MT, false, false>), grid, dim3(kThreads), lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace

int small_m_limit() { return 8; }

bool small_m_fits(int64_t M, int64_t bkf) {
  int mt = 1;
  while (mt < M) mt *= 2;
  return M <= small_m_limit() && small_m_lds_bytes(mt, (int)bkf) <= 64 * 1024;
}

int64_t small_m_column_blocks(int64_t N) { return (N + kCols - 1) / kCols; }

hipError_t launch_gemm_small_m(const SmallMArgs& a, bool out_f32, hipStream_t s) {
  const int64_t M = a.g.M;
  if (M <= 1) return launch_mt<1>(a, out_f32, s);
  if (M <= 2) return launch_mt<2>(a, out_f32, s);
  if (M <= 4) return launch_mt<4>(a, out_f32, s);
  return launch_mt<8>(a, out_f32, s);
}

}  // namespace agemm
