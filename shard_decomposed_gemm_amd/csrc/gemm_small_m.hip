// Flag-gated shard-decomposed GEMM for few rows (M <= 8; the default
// consumer at M = 1, see small_m_default_max below): streaming B.
//
// With one (or a handful of) rows of A, C = sum_s A_s . B[s*KS:(s+1)*KS, :]
// ("Eliminating Multi-GPU Performance Taxes" analysis page, AG+GEMM core
// identity) is bound by reading B once from HBM. The page's bandwidth budget
// for M = 1 notes that the data exchanged is tiny and launch costs dominate;
// here the goal is to stream B at HBM speed and hide the flag waits under it.
//
// Work item = (K-range r, column block). A K-range is W/R consecutive shards,
// a column block 8 * lanes columns (rows read in 1 KiB or 512 B segments);
// the host picks R and lanes to spread the items evenly over the CUs, two
// concurrent workgroups per CU.
// A workgroup has four waves; each active lane owns 8 consecutive columns,
// and wave w takes the range's rows w, w+4, w+8, ... with two register sets
// of 16-byte B loads in flight (B does not depend on the flags). A is read
// from LDS: each wave stages its own rows of A there (no workgroup barrier).
// The gate works at the granularity of the K-range: a wave looks at all of
// its range's flags once and, if any is down, waits for them in tile order
// with its first B loads already in flight; then it stages the range's A and
// streams without a single wait. (Different ranges, i.e. shards, are still
// consumed as their flags arrive; a finer, per-k-tile gate inside the stream
// loop costs the loop registers and issue slots even when never taken.) The
// A copies are plain loads issued after the flags were seen (a compiler
// barrier keeps them there): no line of an inbox k-tile is read in a launch
// before its flag, so no cache holds a stale copy. Four small waves per
// workgroup let two workgroups share a CU, which keeps enough B in flight to
// stream at HBM speed.
// Partial sums go to a workspace per K-range; the last workgroup of a column
// block (counted with an atomic) adds the R partials in range order and writes
// C. The result does not depend on arrival order. In a fused launch each item
// is also counted out of the inbox at its end (the inbox guard, see the
// producer), so the producer of a later epoch may overwrite the inbox without
// a stream dependency.
#include "agemm_internal.h"

namespace agemm {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr size_t kLdsLimit = 64 * 1024;
constexpr int kWgPerCu = 2;  // concurrent workgroups per CU: 8 waves keep enough B in flight

__device__ inline uint64_t wall_clock() { return __builtin_amdgcn_s_memrealtime(); }

// Device-coherent (agent-scope) fp32 store and load of the split-K partials.
__device__ inline void store_coherent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __builtin_bit_cast(uint32_t, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float load_coherent(const float* p) {
  return __builtin_bit_cast(float, __hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<float*>(p)),
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

template <int MT, bool GATED, bool OUTF32>
__global__ __launch_bounds__(kThreads) void gemm_small_m_kernel(SmallMArgs sa) {
  constexpr int kChunk = MT <= 2 ? 16 : 8;  // B rows in flight per lane and register set
  const GemmArgs& g = sa.g;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int64_t M = g.M, N = g.N;
  const int W = g.W;
  const int KT = g.gate.kt;
  const int L = sa.plan.lanes, R = sa.plan.ranges, NBLK = sa.plan.nblk;
  const int cw = 8 * L;                          // columns per item
  const int SPR = W / R;                         // shards per K-range
  const int bkf = (int)(g.KS / KT);
  const int tiles = SPR * KT;                    // k-tiles per K-range
  const int tile_rows = bkf / kWaves;            // rows of one k-tile per wave
  const int rows = tiles * tile_rows;            // rows of the range per wave
  const int items = R * NBLK;
  const int nchunks = rows / kChunk;
  const int chunks_per_tile = tile_rows / kChunk;

  // LDS: A of the whole K-range as fp32, [tile][wave][m][row of the wave's
  // share] (each wave writes and reads only its own part), then a [4][cw]
  // buffer for the cross-wave reduction.
  extern __shared__ float lds[];
  float* lds_a = lds;
  float* lds_r = lds + (size_t)MT * tiles * bkf;
  __shared__ int s_last;

  bool dead = false;  // a flag wait timed out: stop waiting, C is undefined
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int r = item / NBLK;
    const int nb = item - r * NBLK;
    const int s0 = r * SPR;
    float acc[MT][8];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[m][j] = 0.f;

    // This wave's share of the range's A, as fp32 in LDS: of k-tile i (k-tile
    // i % KT of shard s0 + i / KT), rows wave, wave+4, ... Loads go out in
    // batches of 8 per lane before their values are written.
    auto stage = [&]() {
      const int jb = (tile_rows + 63) / 64;      // 64-row blocks per tile
      const int units = tiles * jb * MT;
      for (int u0 = 0; u0 < units; u0 += 8) {
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int u = u0 + q;
          const int i = u / (jb * MT), rem = u - i * (jb * MT);
          const int m = rem / jb, j = (rem - m * jb) * 64 + lane;
          v[q] = 0.f;
          if (u < units && j < tile_rows && m < M) {
            const int sh = s0 + i / KT, kt = i - (i / KT) * KT;
            v[q] = (float)g.a.base[sh][(int64_t)m * g.a.lda + (int64_t)kt * bkf + (int64_t)j * kWaves + wave];
          }
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int u = u0 + q;
          const int i = u / (jb * MT), rem = u - i * (jb * MT);
          const int m = rem / jb, j = (rem - m * jb) * 64 + lane;
          if (u < units && j < tile_rows)
            lds_a[(((size_t)i * kWaves + wave) * MT + m) * tile_rows + j] = v[q];
        }
      }
    };
    // Waits (bounded) for flag f of this epoch; on a timeout records it once.
    auto wait_flag = [&](int f) {
      if constexpr (GATED) {
        if (dead) return;
        const uint64_t start = wall_clock();
        uint32_t v = 0;
        while (true) {
          v = __hip_atomic_load(const_cast<uint32_t*>(g.gate.flags) + f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((int32_t)(v - g.gate.target) >= 0) break;
          if (wall_clock() - start > g.gate.timeout_ticks) {
            dead = true;
            if (lane == 0) {
              __hip_atomic_store(&g.gate.err->tile, (uint32_t)f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
              __hip_atomic_store(&g.gate.err->target, g.gate.target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
              __hip_atomic_store(&g.gate.err->seen, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
              __hip_atomic_store(&g.gate.err->code, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
            }
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
        // See the MFMA consumer: no line of this k-tile was read in this launch
        // before its flag was seen; the strict mode adds the formal agent-scope
        // acquire. The compiler barrier keeps the A loads after the wait.
        if (g.gate.strict) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        asm volatile("" ::: "memory");
      }
    };

    // Lanes past the block's columns load the block's first columns again: the
    // same lines as lane 0 in the same instruction, so no extra memory traffic
    // and no divergent branch in the loop (their sums are dropped).
    const int64_t n = (int64_t)nb * cw + lane * 8;
    const bool active = lane < L && n < N;
    const _Float16* bp = g.B + ((int64_t)s0 * g.KS + wave) * N + (active ? n : (int64_t)nb * cw);
    const int64_t bstep = kWaves * N;
    half8 X[kChunk], Y[kChunk];
    // B is read exactly once: nontemporal loads (no L2 allocation) stream it
    // at 6.3 TB/s on MI355X against 5.75 TB/s with default-policy loads.
    auto fetch = [&](half8 (&Rg)[kChunk], int c) {
#pragma unroll
      for (int i = 0; i < kChunk; ++i)
        Rg[i] = __builtin_nontemporal_load(reinterpret_cast<const half8*>(bp + (c * kChunk + i) * bstep));
    };
    auto use = [&](const half8 (&Rg)[kChunk], int c) {
      const int t = c / chunks_per_tile;
      const int rr = (c - t * chunks_per_tile) * kChunk;
      const float* aw = lds_a + ((size_t)t * kWaves + wave) * MT * tile_rows;
#pragma unroll
      for (int i = 0; i < kChunk; ++i) {
        float bf[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) bf[j] = (float)Rg[i][j];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const float a = aw[m * tile_rows + rr + i];
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[m][j] = __builtin_fmaf(a, bf[j], acc[m][j]);
        }
      }
    };

    // One look at every flag of the range (ids s0*KT .. s0*KT + tiles - 1);
    // if any is still down, wait for them in tile order. The first B loads
    // are already in flight meanwhile (B does not depend on the flags). Then
    // the range's A is staged and the stream runs without a single wait.
    fetch(X, 0);
    if constexpr (GATED) {
      // Plain loads (served by the L2 after one miss; see the MFMA consumer):
      // a cached flag can only lag, so "all up" is safe to trust, and any
      // flag seen down is then waited for with device-coherent polls.
      bool up = true;
      if (lane < tiles) up = (int32_t)(g.gate.flags[s0 * KT + lane] - g.gate.target) >= 0;
      if (__ballot(!up) != 0) {
        for (int i = 0; i < tiles; ++i) wait_flag(s0 * KT + i);
      }
      if (g.gate.strict) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      asm volatile("" ::: "memory");
    }
    stage();
    // Inside the loop every fetch is unconditional (the last one or two chunks
    // are peeled). Scheduling barriers pin the order: a refill is issued after
    // the FMAs that read the old contents of its registers, and before the
    // FMAs of the other set, so while one set is used the other is in flight
    // (without them the scheduler sinks the refill below the other set's
    // wait, which then drains every load).
    int c = 0;
    for (; c + 2 < nchunks; c += 2) {
      fetch(Y, c + 1);
      __builtin_amdgcn_sched_barrier(0);
      use(X, c);
      __builtin_amdgcn_sched_barrier(0);
      fetch(X, c + 2);
      __builtin_amdgcn_sched_barrier(0);
      use(Y, c + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (nchunks - c == 2) {
      fetch(Y, c + 1);
      __builtin_amdgcn_sched_barrier(0);
      use(X, c);
      use(Y, c + 1);
    } else {
      use(X, c);
    }

    // Inbox guard (thread 0, once the workgroup has passed a barrier after its
    // waves waited for all their loads, the A copies from the inbox long
    // among them): counts the item out of the inbox, with no returned value.
    // It is issued after the item's last loads (the last arriver's partials
    // too): a load issued after it would wait for it. Counting right after
    // the copies, mid-item, cost 2 us per launch that way.
    auto count_out = [&]() {
      if constexpr (GATED) {
        if (g.consumed != nullptr)
          __hip_atomic_fetch_add(g.consumed + guard_counter(item) * kGuardStride, 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
    };

    // Sum the four waves' partials (in wave order), one row at a time.
    float* ws_r = sa.ws + (int64_t)r * M * N;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= M) break;
      if (lane < L) {
#pragma unroll
        for (int j = 0; j < 8; ++j) lds_r[wave * cw + lane * 8 + j] = acc[m][j];
      }
      __syncthreads();
      for (int cc = tid; cc < cw; cc += kThreads) {
        const int64_t col = (int64_t)nb * cw + cc;
        if (col < N) {
          float v = lds_r[cc];
          v += lds_r[cw + cc];
          v += lds_r[2 * cw + cc];
          v += lds_r[3 * cw + cc];
          store_coherent(ws_r + (int64_t)m * N + col, v);
        }
      }
      __syncthreads();
    }

    // The last workgroup to finish a column block adds the R partials in range
    // order. The partials travel only through device-coherent accesses
    // (relaxed agent-scope atomic stores and loads, which bypass the per-XCD
    // L2), so the hand-off needs no L2-wide fence: every thread waits until
    // its partial stores have completed, then one thread counts the
    // workgroup in. (An agent-scope release/acquire pair here writes back and
    // invalidates whole L2s and cost a third of the kernel's time.)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      const uint32_t old = __hip_atomic_fetch_add(sa.counters + nb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = (old == (uint32_t)(R - 1));
      if (!s_last) count_out();
    }
    __syncthreads();
    if (!__builtin_amdgcn_readfirstlane(s_last)) continue;
    for (int idx = tid; idx < MT * cw; idx += kThreads) {
      const int m = idx / cw;
      const int cc = idx - m * cw;
      const int64_t col = (int64_t)nb * cw + cc;
      if (m < M && col < N) {
        float part[kMaxShards];
#pragma unroll
        for (int t = 0; t < kMaxShards; ++t) part[t] = t < R ? load_coherent(sa.ws + ((int64_t)t * M + m) * N + col) : 0.f;
        float v = 0.f;
#pragma unroll
        for (int t = 0; t < kMaxShards; ++t)
          if (t < R) v += part[t];
        if constexpr (OUTF32) static_cast<float*>(g.C)[(int64_t)m * N + col] = v;
        else static_cast<_Float16*>(g.C)[(int64_t)m * N + col] = (_Float16)v;
      }
    }
    if (tid == 0) {
      __hip_atomic_store(sa.counters + nb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      count_out();
    }
    __syncthreads();  // s_last and lds_r are reused by the next item
  }
}

int mt_of(int64_t M) {
  int mt = 1;
  while (mt < M) mt *= 2;
  return mt;
}

size_t lds_bytes(int mt, int64_t rows_per_range, int lanes) {
  return sizeof(float) * ((size_t)mt * rows_per_range + (size_t)kWaves * 8 * lanes);
}

template <int MT, bool G, bool F>
void launch_one(const SmallMArgs& a, dim3 grid, size_t lds, hipStream_t s, const LaunchTiming& t) {
  if (t.start)
    hipExtLaunchKernelGGL((gemm_small_m_kernel<MT, G, F>), grid, dim3(kThreads), (uint32_t)lds, s, t.start, t.stop, 0,
                          a);
  else
    hipLaunchKernelGGL((gemm_small_m_kernel<MT, G, F>), grid, dim3(kThreads), lds, s, a);
}

template <int MT>
hipError_t launch_mt(const SmallMArgs& a, bool out_f32, hipStream_t s, const LaunchTiming& t) {
  const SmallMPlan& p = a.plan;
  // Persistent grid of at most wg_per_cu workgroups per CU (the plan spreads
  // the items evenly): well under what fits on a CU, so producer workgroups
  // always find room next to waiting consumers.
  const int64_t items = (int64_t)p.ranges * p.nblk;
  const int64_t cap = (int64_t)p.wg_per_cu * a.g.num_cus;
  const dim3 grid((unsigned)(items < cap ? items : cap));
  const size_t lds = lds_bytes(MT, a.g.KS * (a.g.W / p.ranges), p.lanes);
  const bool gated = a.g.gate.flags != nullptr;
  if (gated) {
    if (out_f32) launch_one<MT, true, true>(a, grid, lds, s, t);
    else launch_one<MT, true, false>(a, grid, lds, s, t);
  } else {
    if (out_f32) launch_one<MT, false, true>(a, grid, lds, s, t);
    else launch_one<MT, false, false>(a, grid, lds, s, t);
  }
  return hipGetLastError();
}

}  // namespace

int small_m_limit() { return 8; }

// Largest M for which the small-M kernel is the default consumer. From M = 2
// on, the MFMA kernel on 128x128 tiles (k-panel inbox, nontemporal B) streams
// B at least as fast. Consumer alone at K = 8192, N = 28672, W = 8, us:
//   M          1      2      3      4      6      8
//   small-M   76.5   81.7   96.5  100.1  114.4  121.7
//   MFMA      78.4   78.8   78.3   78.8   77.9   79.8
int small_m_default_max() { return 1; }

// Picks (lanes, ranges) for the shape: the highest ratio of useful work to
// the work of the busiest rounds of workgroup slots (kWgPerCu per CU; 1.0 =
// every slot streams the same number of B bytes), then the fewest K-ranges
// (smaller workspace), then the widest block.
SmallMPlan small_m_plan(int W, int64_t M, int64_t KS, int64_t N, int num_cus) {
  SmallMPlan best;
  if (M < 1 || M > small_m_limit() || W < 1 || num_cus < 1) return best;
  const int mt = mt_of(M);
  double best_eff = 0.0;
  for (int ranges = 1; ranges <= W; ++ranges) {
    if (W % ranges) continue;
    const int64_t rows = KS * (W / ranges);
    if ((KS / 64) * 64 != KS) continue;
    // Row segments of 1 KiB or 512 B only: a segment that is not a power of
    // two (e.g. 56 lanes, 896 B) streams far slower (measured).
    for (int lanes = 64; lanes >= 32; lanes /= 2) {
      if (lds_bytes(mt, rows, lanes) > kLdsLimit) continue;
      const int64_t cw = 8 * (int64_t)lanes;
      const int64_t nblk = (N + cw - 1) / cw;
      const int64_t items = nblk * ranges;
      const int64_t slots = (int64_t)kWgPerCu * num_cus;
      const int64_t rounds = (items + slots - 1) / slots;
      const double eff = (double)N * (double)(KS * W) / ((double)rounds * slots * (double)cw * (double)rows);
      if (eff > best_eff + 1e-9) {
        best_eff = eff;
        best.lanes = lanes;
        best.ranges = ranges;
        best.nblk = (int32_t)nblk;
        best.wg_per_cu = kWgPerCu;
        best.ok = true;
      }
    }
  }
  return best;
}

SmallMPlan small_m_plan_with(int W, int64_t M, int64_t KS, int64_t N, int lanes, int ranges, int wg_per_cu) {
  SmallMPlan p;
  if (M < 1 || M > small_m_limit() || W < 1 || ranges < 1 || W % ranges || lanes < 1 || lanes > 64 ||
      wg_per_cu < 1 || wg_per_cu > 4)
    return p;
  if (lds_bytes(mt_of(M), KS * (W / ranges), lanes) > kLdsLimit) return p;
  p.lanes = lanes;
  p.ranges = ranges;
  p.nblk = (int32_t)((N + 8 * lanes - 1) / (8 * lanes));
  p.wg_per_cu = wg_per_cu;
  p.ok = true;
  return p;
}

hipError_t launch_gemm_small_m(const SmallMArgs& a, bool out_f32, hipStream_t s, const LaunchTiming& t) {
  const int64_t M = a.g.M;
  if (M <= 1) return launch_mt<1>(a, out_f32, s, t);
  if (M <= 2) return launch_mt<2>(a, out_f32, s, t);
  if (M <= 4) return launch_mt<4>(a, out_f32, s, t);
  return launch_mt<8>(a, out_f32, s, t);
}

}  // namespace agemm
