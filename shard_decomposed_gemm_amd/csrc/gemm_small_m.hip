// Flag-gated shard-decomposed GEMM for few rows (M <= 8): streaming B.
//
// With one (or a handful of) rows of A, C = sum_s A_s . B[s*KS:(s+1)*KS, :]
// ("Eliminating Multi-GPU Performance Taxes" analysis page, AG+GEMM core
// identity) is bound by reading B once from HBM. The page's bandwidth budget
// for M = 1 notes that the data exchanged is tiny and launch costs dominate;
// here the goal is to stream B at HBM speed and hide the flag waits under it.
//
// Work item = (shard s, block of 512 columns). A workgroup has four streaming
// waves and one control wave:
//   * each streaming lane owns 8 consecutive columns; wave w takes the shard's
//     rows w, w+4, w+8, ... and keeps a ring of 16-byte B loads in flight that
//     runs straight across k-tile boundaries (B does not depend on the flags);
//   * the control wave, for k-tile kt = 0 .. KT-1 of the shard, polls
//     Flags(s, kt), acquires, copies A_s's k-tile (rows < M) into LDS as fp32
//     and then meets the streaming waves at a barrier; the streaming waves
//     read A only from LDS, so they never execute a fence that would drain
//     their B loads.
// Partial sums go to a workspace per shard; the last workgroup of a column
// block (counted with an acq_rel atomic) adds the W partials in shard order
// and writes C. The result does not depend on arrival order.
#include <type_traits>

#include "agemm_internal.h"

namespace agemm {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

constexpr int kStreamWaves = 4;
constexpr int kThreads = 64 * (kStreamWaves + 1);
constexpr int kCols = 512;  // columns per work item: 64 lanes x 8

__device__ inline uint64_t wall_clock() { return __builtin_amdgcn_s_memrealtime(); }
__device__ inline void barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int MT, bool GATED, bool OUTF32>
__global__ __launch_bounds__(kThreads) void gemm_small_m_kernel(SmallMArgs sa) {
  constexpr int kChunk = MT <= 2 ? 16 : 8;  // B rows in flight per lane
  const GemmArgs& g = sa.g;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int64_t M = g.M, N = g.N;
  const int W = g.W;
  const int KT = g.gate.kt;
  const int NBLK = (int)((N + kCols - 1) / kCols);
  const int bkf = (int)(g.KS / KT);
  const int tile_rows = bkf / kStreamWaves;     // rows of one k-tile per streaming wave
  const int rows = (int)(g.KS / kStreamWaves);  // rows of the shard per streaming wave
  const int items = W * NBLK;

  // LDS: A of the whole shard as fp32, [kt][wave][m][row of the wave's share],
  // then a [4][kCols] buffer for the cross-wave reduction.
  extern __shared__ float lds[];
  float* lds_a = lds;
  float* lds_r = lds + (size_t)MT * g.KS;
  __shared__ int s_abort;
  __shared__ int s_last;
  if (tid == 0) s_abort = 0;
  __syncthreads();

  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int s = item / NBLK;
    const int nb = item - s * NBLK;
    float acc[MT][8];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[m][j] = 0.f;

    if (wave == kStreamWaves) {
      // ---- control wave: per k-tile, wait for the flag, then stage A in LDS
      for (int kt = 0; kt < KT; ++kt) {
        if constexpr (GATED) {
          if (!s_abort) {
            const int f = s * KT + kt;
            const uint64_t start = wall_clock();
            uint32_t v = 0;
            int abort = 0;
            while (true) {
              v = __hip_atomic_load(const_cast<uint32_t*>(g.gate.flags) + f, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
              if ((int32_t)(v - g.gate.target) >= 0) break;
              if (wall_clock() - start > g.gate.timeout_ticks) {
                abort = 1;
                break;
              }
              __builtin_amdgcn_s_sleep(2);
            }
            // See the MFMA consumer: no line of this k-tile was read in this
            // launch before its flag, and the A loads below are device-scope
            // loads ordered after the flag by control dependency. The strict
            // mode adds the formal agent-scope acquire.
            if (g.gate.strict) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            asm volatile("" ::: "memory");
            if (abort && lane == 0) {
              __hip_atomic_store(&g.gate.err->tile, (uint32_t)f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
              __hip_atomic_store(&g.gate.err->target, g.gate.target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
              __hip_atomic_store(&g.gate.err->seen, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
              __hip_atomic_store(&g.gate.err->code, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
              s_abort = 1;
            }
          }
        }
        if (!s_abort) {
          // A's k-tile, two halves per device-scope (agent) 32-bit load.
          const _Float16* ap = g.a.base[s] + (int64_t)kt * bkf;
          float* dst = lds_a + (size_t)kt * MT * bkf;
          for (int idx = lane; idx < MT * bkf / 2; idx += 64) {
            const int m = (2 * idx) / bkf;
            const int k = 2 * idx - m * bkf;
            float v0 = 0.f, v1 = 0.f;
            if (m < M) {
              const uint32_t w = __hip_atomic_load(
                  reinterpret_cast<uint32_t*>(const_cast<_Float16*>(ap + (int64_t)m * g.a.lda + k)), __ATOMIC_RELAXED,
                  __HIP_MEMORY_SCOPE_AGENT);
              v0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
              v1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
            }
            dst[((k % kStreamWaves) * MT + m) * tile_rows + k / kStreamWaves] = v0;
            dst[(((k + 1) % kStreamWaves) * MT + m) * tile_rows + (k + 1) / kStreamWaves] = v1;
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        barrier();  // k-tile kt is in LDS (or the item was abandoned)
      }
    } else {
      // ---- streaming waves: chunks of kChunk rows alternate between two register
      // sets (chunk c in X if c is even, else Y). A set is refilled only after its
      // rows have been used, so no loop-carried copies (and no drain) are needed.
      const int64_t n = (int64_t)nb * kCols + lane * 8;
      const int64_t nl = n < N ? n : N - 8;  // idle lanes read a valid address
      const _Float16* bp = g.B + ((int64_t)s * g.KS + wave) * N + nl;
      const int64_t bstep = kStreamWaves * N;
      const int nchunks = rows / kChunk;
      const int chunks_per_tile = tile_rows / kChunk;
      half8 X[kChunk], Y[kChunk];
      auto fetch = [&](half8 (&R)[kChunk], int c) {
#pragma unroll
        for (int i = 0; i < kChunk; ++i) R[i] = *reinterpret_cast<const half8*>(bp + (c * kChunk + i) * bstep);
      };
      auto use = [&](const half8 (&R)[kChunk], int c) {
        const int kt = c / chunks_per_tile;
        const int rr = (c - kt * chunks_per_tile) * kChunk;
        const float* aw = lds_a + (size_t)kt * MT * bkf + wave * MT * tile_rows;
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
          float bf[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) bf[j] = (float)R[i][j];
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const float a = aw[m * tile_rows + rr + i];
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[m][j] = __builtin_fmaf(a, bf[j], acc[m][j]);
          }
        }
      };
      // Entering a new k-tile: meet the control wave (its A tile is staged).
      auto tile_gate = [&](int c) {
        if (c % chunks_per_tile == 0) barrier();
        return s_abort == 0;
      };
      // Every chunk calls tile_gate, so the streaming waves meet the control wave
      // at exactly one barrier per k-tile even after an abort. Inside the loop
      // every fetch is unconditional (the last one or two chunks are peeled), and
      // a scheduling barrier keeps each refill after the FMAs that read the old
      // contents of its registers.
      fetch(X, 0);
      int c = 0;
      for (; c + 2 < nchunks; c += 2) {
        fetch(Y, c + 1);
        if (tile_gate(c)) use(X, c);
        __builtin_amdgcn_sched_barrier(0);
        fetch(X, c + 2);
        if (tile_gate(c + 1)) use(Y, c + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (nchunks - c == 2) {
        fetch(Y, c + 1);
        if (tile_gate(c)) use(X, c);
        if (tile_gate(c + 1)) use(Y, c + 1);
      } else {
        if (tile_gate(c)) use(X, c);
      }
    }
    __syncthreads();
    if (s_abort) break;  // C is left undefined

    // Sum the four streaming waves' partials (in wave order), one row at a time.
    float* ws_s = sa.ws + (int64_t)s * M * N;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= M) break;
      if (wave < kStreamWaves) {
#pragma unroll
        for (int j = 0; j < 8; ++j) lds_r[wave * kCols + lane * 8 + j] = acc[m][j];
      }
      __syncthreads();
      for (int c = tid; c < kCols; c += kThreads) {
        const int64_t col = (int64_t)nb * kCols + c;
        if (col < N) {
          float v = lds_r[c];
          v += lds_r[kCols + c];
          v += lds_r[2 * kCols + c];
          v += lds_r[3 * kCols + c];
          ws_s[(int64_t)m * N + col] = v;
        }
      }
      __syncthreads();
    }

    // The last workgroup to finish a column block adds the W partials in shard order.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (tid == 0) {
      const uint32_t old = __hip_atomic_fetch_add(sa.counters + nb, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      s_last = (old == (uint32_t)(W - 1));
    }
    __syncthreads();
    if (!__builtin_amdgcn_readfirstlane(s_last)) continue;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    for (int idx = tid; idx < MT * kCols; idx += kThreads) {
      const int m = idx / kCols;
      const int c = idx - m * kCols;
      const int64_t col = (int64_t)nb * kCols + c;
      if (m < M && col < N) {
        float part[kMaxShards];
#pragma unroll
        for (int t = 0; t < kMaxShards; ++t) part[t] = t < W ? sa.ws[((int64_t)t * M + m) * N + col] : 0.f;
        float v = 0.f;
#pragma unroll
        for (int t = 0; t < kMaxShards; ++t)
          if (t < W) v += part[t];
        if constexpr (OUTF32) static_cast<float*>(g.C)[(int64_t)m * N + col] = v;
        else static_cast<_Float16*>(g.C)[(int64_t)m * N + col] = (_Float16)v;
      }
    }
    if (tid == 0) __hip_atomic_store(sa.counters + nb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

size_t small_m_lds_bytes(int mt, int64_t ks) { return sizeof(float) * (size_t)(mt * ks + 4 * kCols); }

int mt_of(int64_t M) {
  int mt = 1;
  while (mt < M) mt *= 2;
  return mt;
}

template <int MT>
hipError_t launch_mt(const SmallMArgs& a, bool out_f32, hipStream_t s) {
  const int nblk = (int)((a.g.N + kCols - 1) / kCols);
  // Persistent grid of up to two workgroups per CU: well under what fits on a
  // CU, so producer workgroups always find room next to waiting consumers.
  const int64_t items = (int64_t)a.g.W * nblk;
  const int64_t cap = 2 * (int64_t)a.g.num_cus;
  const dim3 grid((unsigned)(items < cap ? items : cap));
  const size_t lds = small_m_lds_bytes(MT, a.g.KS);
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

bool small_m_fits(int64_t M, int64_t KS) {
  return M <= small_m_limit() && small_m_lds_bytes(mt_of(M), KS) <= 64 * 1024;
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
