// Flag-gated shard-decomposed GEMM on gfx950 matrix cores.
//
// Computes C = sum_{s=0}^{W-1} A_s . B[s*KS:(s+1)*KS, :] ("Eliminating
// Multi-GPU Performance Taxes" analysis page, AG+GEMM core identity): each
// workgroup owns a BM x BN tile of C and walks the K dimension shard by shard
// (outer loop over s, inner loop over the shard's k-steps), which is the
// loop order the page gives for the Pull and Push GEMMs. With the gate on
// (Push model), before the first k-step of each (shard, k-tile) the workgroup
// makes sure that tile's flag has reached the epoch's target: one wave polls
// all T flags with relaxed agent-scope loads, then issues an agent-scope
// acquire fence; the workgroup remembers which tiles it has already acquired,
// so a launch that finds every flag raised pays for one poll.
//
// Data path (per 64-wide k-step, double buffered in LDS):
//   A_s rows  : global -> LDS with 16-byte direct loads, rows of 128 B with the
//               16-byte chunk index XOR-swizzled by (row & 7);
//   B rows    : global -> LDS the same way, rows of BN*2 bytes, chunk index
//               XOR-swizzled by a function of k;
//   operands  : A by 16-byte LDS reads, B by LDS transpose reads
//               (ds_read_b64_tr_b16), which turn the N-contiguous B rows into
//               the K-contiguous operand the matrix core wants;
//   math      : v_mfma_f32_32x32x16_f16 with the roles swapped (the B^T tile
//               is the first operand), so each lane ends up holding four
//               consecutive C columns and stores them with one vector store.
#include "agemm_internal.h"

namespace agemm {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
#define LDS_PTR(T) __attribute__((address_space(3))) T*

constexpr int BK = 64;

__device__ inline uint64_t wall_clock() { return __builtin_amdgcn_s_memrealtime(); }

__device__ inline int swz_b(int k) { return ((k & 3) << 1) ^ (((k >> 3) & 1) << 3); }

// Per-lane read offsets into one LDS stage (bytes), fixed for the whole launch.
struct ReadOffsets {
  int a[4];   // A fragment of k16-substep ks (fm adds fm * 32 rows)
  int b[4];   // B fragment of 32-column block fn (ks, h add whole rows)
};

// One k-step: issue the direct loads of the next stage (if any) and run the
// MFMAs of the current stage. The two stage pointers are restrict-qualified
// so the compiler can tell that the LDS reads of `cur` do not depend on the
// loads still in flight into `nxt`.
template <int BM, int BN, int WM, int WN, bool ISSUE>
__device__ __attribute__((always_inline)) inline void kstep(
    char* __restrict__ nxt, const char* __restrict__ cur, const _Float16* a_src, const _Float16* b_src,
    const int64_t* a_off, const int64_t* b_off, int wave, const ReadOffsets& ro,
    f32x16 (&acc)[BM / WM / 32][BN / WN / 32]) {
  constexpr int NT = 64 * WM * WN;
  constexpr int FM = BM / WM / 32, FN = BN / WN / 32;
  constexpr int A_BYTES = BM * BK * 2;
  constexpr int A_ITERS = (BM * BK / 8) / NT;
  constexpr int B_ITERS = (BK * BN / 8) / NT;
  constexpr int ROWB = BN * 2;  // bytes per B row in LDS

  if constexpr (ISSUE) {
#pragma unroll
    for (int j = 0; j < A_ITERS; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(a_src + a_off[j]),
                                       (LDS_PTR(void))(nxt + (j * NT + wave * 64) * 16), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < B_ITERS; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(b_src + b_off[j]),
                                       (LDS_PTR(void))(nxt + A_BYTES + (j * NT + wave * 64) * 16), 16, 0, 0);
  }

  const char* lds_a = cur;
  const char* lds_b = cur + A_BYTES;
  half8 af[2][FM];
  half8 bf[2][FN];
  auto load = [&](int ks, int slot) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
      af[slot][fm] = *reinterpret_cast<const half8*>(lds_a + ro.a[ks] + fm * 32 * (BK * 2));
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const char* p = lds_b + ro.b[fn] + ks * 16 * ROWB;
      half4 lo = __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((LDS_PTR(fp16x4_t))(p)));
      half4 hi = __builtin_bit_cast(half4,
                                    __builtin_amdgcn_ds_read_tr16_b64_v4f16((LDS_PTR(fp16x4_t))(p + 4 * ROWB)));
      bf[slot][fn] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  load(0, 0);
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    const int cs = ks & 1;
    if (ks + 1 < BK / 16) load(ks + 1, cs ^ 1);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[cs][fn], af[cs][fm], acc[fm][fn], 0, 0, 0);
  }
}

template <int BM, int BN, int WM, int WN, bool GATED, bool OUTF32>
__global__ __launch_bounds__(64 * WM * WN) void gemm_mfma_kernel(GemmArgs g) {
  constexpr int NT = 64 * WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int A_BYTES = BM * BK * 2;
  constexpr int B_BYTES = BK * BN * 2;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_ITERS = (BM * BK / 8) / NT;  // 16-byte chunks per thread
  constexpr int B_ITERS = (BK * BN / 8) / NT;
  constexpr int CPR_B = BN / 8;
  static_assert(FM >= 1 && FN >= 1, "wave tile too small");
  static_assert(A_ITERS * NT == BM * BK / 8 && B_ITERS * NT == BK * BN / 8, "tile/thread mismatch");
  static_assert(CPR_B >= 16, "B row must hold at least 16 chunks for the swizzle");

  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
  __shared__ uint64_t s_ready;
  __shared__ int s_abort;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int lane = tid & 63;
  const int wm = wave / WN;
  const int wn = wave - wm * WN;

  const int64_t M = g.M, N = g.N;
  const int MB = (int)((M + BM - 1) / BM);
  const int NB = (int)((N + BN - 1) / BN);
  const int total = MB * NB;
  const int SPS = (int)(g.KS / BK);  // k-steps per shard
  const int NS = (int)(g.K / BK);    // k-steps in all

  // LDS read offsets (tile independent). A: row (wm*TM + fm*32 + lane%32),
  // 16-byte chunk (2*ks + lane/32) ^ (row & 7). B (transpose read, 16-lane
  // groups): lane supplies row k = 16*ks + 8*(g/2) + 4*h + (i/4) and columns
  // n = fn*32 + 16*(g%2) + 4*(i%4) of the wave's range, chunk (n/8) ^ swz(k);
  // swz(k) does not depend on ks or h.
  ReadOffsets ro;
  {
    const int row = wm * TM + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) ro.a[ks] = row * (BK * 2) + (((ks * 2 + (lane >> 5)) ^ (row & 7)) * 16);
    const int g16 = lane >> 4, i16 = lane & 15;
    const int k = (g16 >> 1) * 8 + (i16 >> 2);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int n = wn * TN + fn * 32 + (g16 & 1) * 16 + (i16 & 3) * 4;
      ro.b[fn] = k * (BN * 2) + (((n >> 3) ^ swz_b(k)) * 16) + (n & 7) * 2;
    }
  }

  uint64_t ready = 0;  // flags this workgroup has already acquired (persists across its tiles)
  // Returns false if the workgroup must stop (flag wait timed out).
  auto gate = [&](int t) -> bool {
    if constexpr (!GATED) {
      return true;
    } else {
      const int s = t / SPS;
      const int tile = s * g.gate.kt + (t - s * SPS) / g.gate.steps_per_tile;
      if ((ready >> tile) & 1ull) return true;
      if (wave == 0) {
        const uint64_t start = wall_clock();
        uint64_t mask = 0;
        int abort = 0;
        uint32_t seen = 0;
        while (true) {
          bool ok = false;
          if (lane < g.gate.t) {
            const uint32_t v = __hip_atomic_load(const_cast<uint32_t*>(g.gate.flags) + lane, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
            ok = (int32_t)(v - g.gate.target) >= 0;
            if (lane == tile) seen = v;
          }
          mask = __ballot(ok);
          if ((mask >> tile) & 1ull) break;
          if (wall_clock() - start > g.gate.timeout_ticks) {
            abort = 1;
            if (lane == tile) {
              __hip_atomic_store(&g.gate.err->tile, (uint32_t)tile, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
              __hip_atomic_store(&g.gate.err->target, g.gate.target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
              __hip_atomic_store(&g.gate.err->seen, seen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
              __hip_atomic_store(&g.gate.err->code, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
            }
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        if (lane == 0) {
          s_ready = mask;
          s_abort = abort;
        }
      }
      __syncthreads();
      const uint64_t r = s_ready;
      ready = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(r >> 32)) << 32) |
              (uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)r);
      return __builtin_amdgcn_readfirstlane(s_abort) == 0;
    }
  };

  // Persistent loop over output tiles. Workgroups are dealt round-robin to
  // the 8 XCDs; each XCD gets a contiguous range of logical tiles, ordered in
  // groups of 8 row-blocks, so tiles running together on one XCD share A and
  // B rows in its L2.
  const int G = gridDim.x;
  const bool xcd_split = (total % 8 == 0) && (G % 8 == 0);
  bool ok = true;
  for (int w = blockIdx.x; w < total; w += G) {
    const int logical = xcd_split ? (w % 8) * (total / 8) + (w / 8) : w;
    constexpr int GM = 8;
    const int group = logical / (GM * NB);
    const int first_m = group * GM;
    const int gsize = (MB - first_m) < GM ? (MB - first_m) : GM;
    const int in_group = logical - group * GM * NB;
    const int mb = first_m + in_group % gsize;
    const int nb = in_group / gsize;
    const int64_t m0 = (int64_t)mb * BM;
    const int64_t n0 = (int64_t)nb * BN;

    // Global source offsets (elements) of this thread's 16-byte chunks; the
    // LDS destination of chunk q is byte q*16 of the stage.
    int64_t a_off[A_ITERS];
#pragma unroll
    for (int j = 0; j < A_ITERS; ++j) {
      const int q = j * NT + wave * 64 + lane;
      const int r = q >> 3;
      const int c = (q & 7) ^ (r & 7);
      int64_t m = m0 + r;
      if (m > M - 1) m = M - 1;  // rows past M load a valid row; their results are not stored
      a_off[j] = m * g.a.lda + c * 8;
    }
    int64_t b_off[B_ITERS];
#pragma unroll
    for (int j = 0; j < B_ITERS; ++j) {
      const int q = j * NT + wave * 64 + lane;
      const int k = q / CPR_B;
      const int c = (q % CPR_B) ^ swz_b(k);
      int64_t n = n0 + c * 8;
      if (n > N - 8) n = N - 8;
      b_off[j] = (int64_t)k * N + n;
    }

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    auto a_src = [&](int t) {
      const int s = t / SPS;
      return g.a.base[s] + (int64_t)(t - s * SPS) * BK;
    };
    auto b_src = [&](int t) { return g.B + (int64_t)t * BK * N; };

    __syncthreads();  // the previous tile's last reads of LDS are done
    ok = gate(0);
    if (!ok) break;
    {
      const _Float16* as = a_src(0);
      const _Float16* bs = b_src(0);
#pragma unroll
      for (int j = 0; j < A_ITERS; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(as + a_off[j]),
                                         (LDS_PTR(void))(smem + (j * NT + wave * 64) * 16), 16, 0, 0);
#pragma unroll
      for (int j = 0; j < B_ITERS; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(bs + b_off[j]),
                                         (LDS_PTR(void))(smem + A_BYTES + (j * NT + wave * 64) * 16), 16, 0, 0);
    }
    // One loop body for every k-step (a single copy of the MFMA code keeps the
    // accumulators in place). The last step re-issues its own loads into the
    // idle stage, which nobody reads; they are drained before the epilogue.
    for (int t = 0; t < NS; ++t) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      const int tn = (t + 1 < NS) ? t + 1 : t;
      ok = gate(tn);
      if (!ok) break;
      kstep<BM, BN, WM, WN, true>(smem + ((t + 1) & 1) * STAGE, smem + (t & 1) * STAGE, a_src(tn), b_src(tn), a_off,
                                  b_off, wave, ro, acc);
    }
    __builtin_amdgcn_s_waitcnt(0);  // drain the direct loads before storing or leaving
    if (!ok) break;                  // a flag wait timed out: C is left undefined

    // Epilogue: lane holds C[m][n .. n+3] for m = lane % 32 of each 32-row block.
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int64_t m = m0 + wm * TM + fm * 32 + (lane & 31);
      if (m >= M) continue;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        // Keep the accumulator reads of one 32x32 block together.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t n = n0 + wn * TN + fn * 32 + q * 8 + (lane >> 5) * 4;
          if (n >= N) continue;
          if constexpr (OUTF32) {
            float4 v = make_float4(acc[fm][fn][q * 4 + 0], acc[fm][fn][q * 4 + 1], acc[fm][fn][q * 4 + 2],
                                   acc[fm][fn][q * 4 + 3]);
            *reinterpret_cast<float4*>(static_cast<float*>(g.C) + m * N + n) = v;
          } else {
            half4 v;
            v[0] = (_Float16)acc[fm][fn][q * 4 + 0];
            v[1] = (_Float16)acc[fm][fn][q * 4 + 1];
            v[2] = (_Float16)acc[fm][fn][q * 4 + 2];
            v[3] = (_Float16)acc[fm][fn][q * 4 + 3];
            *reinterpret_cast<half4*>(static_cast<_Float16*>(g.C) + m * N + n) = v;
          }
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const GemmArgs& a, bool out_f32, hipStream_t s) {
  const int64_t MB = (a.M + BM - 1) / BM;
  const int64_t NB = (a.N + BN - 1) / BN;
  // Persistent grid of at most one workgroup per CU. A running consumer then
  // always leaves room on its CU (registers, LDS, wave slots) for producer
  // workgroups, so spinning consumers can never lock the producer out.
  const int64_t tiles = MB * NB;
  const int64_t g = tiles < a.num_cus ? tiles : a.num_cus;
  const dim3 grid((unsigned)g);
  const dim3 block(64 * WM * WN);
  const bool gated = a.gate.flags != nullptr;
  if (gated) {
    if (out_f32) hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, WM, WN, true, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, WM, WN, true, false>), grid, block, 0, s, a);
  } else {
    if (out_f32) hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, WM, WN, false, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, WM, WN, false, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mfma(const GemmArgs& a, bool out_f32, hipStream_t s) {
  // Large M: 256 x 256 tiles (one workgroup per CU, 128 KiB of LDS).
  // Smaller M: 128-row tiles so that the grid still covers the 256 CUs.
  if (a.M > 256) return launch_cfg<256, 256, 2, 4>(a, out_f32, s);
  return launch_cfg<128, 128, 2, 2>(a, out_f32, s);
}

}  // namespace agemm
