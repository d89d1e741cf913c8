// Flag-gated shard-decomposed GEMM on gfx950 matrix cores.
//
// Computes C = sum_{s=0}^{W-1} A_s . B[s*KS:(s+1)*KS, :] ("Eliminating
// Multi-GPU Performance Taxes" analysis page, AG+GEMM core identity): each
// workgroup owns a BM x BN tile of C and walks the K dimension shard by shard
// (outer loop over s, inner loop over the shard's k-steps), which is the
// loop order the page gives for the Pull and Push GEMMs. With the gate on
// (Push model), each wave checks, before it issues the loads of the first
// k-step of a (shard, k-tile), that the tile's flag has reached the epoch's
// target: its lanes poll all T flags at once with relaxed agent-scope loads,
// and the wave remembers which tiles it has seen raised, so a launch that
// finds every flag raised pays for one poll per wave.
//
// Data path (per BK-wide k-step, STAGES-deep ring of LDS stages):
//   A_s rows  : global -> LDS with 16-byte direct loads, rows of BK*2 bytes,
//               16-byte chunk index XOR-swizzled so that the 16 rows one
//               16-lane group reads fall in 16 distinct 16-byte slots of
//               the 256-byte bank line;
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

__device__ inline uint64_t wall_clock() { return __builtin_amdgcn_s_memrealtime(); }

// The gfx950 LDS serves a 16-lane group per cycle from 64 banks (256 bytes);
// a read is conflict-free when the group's addresses fall in distinct 4-byte
// banks. Both swizzles below were checked with the LDS bank-conflict counter.
//
// B rows (k) of a stage: the 16-byte chunk index is XORed with swz_b(k), which
// moves the four rows read by one 16-lane transpose read 64 bytes apart.
__device__ inline int swz_b(int k) { return (k & 3) << 2; }

// A rows of BK halves = CPR 16-byte chunks: XOR with swz_a(row) so that the 16
// consecutive rows read by one 16-lane group cover 16 distinct 16-byte slots
// of a 256-byte bank line.
template <int CPR>
__device__ inline int swz_a(int row) {
  return (row / (16 / CPR)) % CPR;
}

template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int BM, int BN, int BK, int WM, int WN>
struct Shape {
  static constexpr int NT = 64 * WM * WN;          // threads
  static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  static constexpr int FM = TM / 32, FN = TN / 32;  // 32x32 MFMA blocks per wave
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int B_BYTES = BK * BN * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int CPR_A = BK / 8;              // 16-byte chunks per A row
  static constexpr int CPR_B = BN / 8;              // 16-byte chunks per B row
  static constexpr int A_ITERS = (BM * BK / 8) / NT;
  static constexpr int B_ITERS = (BK * BN / 8) / NT;
  static constexpr int LOADS = A_ITERS + B_ITERS;   // direct loads per thread per k-step
  static constexpr int KSUB = BK / 16;              // MFMA k-substeps per k-step
  static_assert(FM >= 1 && FN >= 1, "wave tile too small");
  static_assert(A_ITERS * NT == BM * BK / 8 && B_ITERS * NT == BK * BN / 8, "tile/thread mismatch");
  static_assert(CPR_B >= 16, "B row must hold at least 16 chunks for the swizzle");
  static_assert(CPR_A == 4 || CPR_A == 8, "BK must be 32 or 64");
  static_assert(KSUB <= 4, "at most 4 k-substeps");
};

// Per-lane read offsets into one LDS stage (bytes), fixed for the whole launch.
struct ReadOffsets {
  int a[4];   // A fragment of k16-substep ks (fm adds fm * 32 rows)
  int b[4];   // B fragment of 32-column block fn (ks, h add whole rows)
};

// LDS reads are issued with inline assembly: the compiler then neither
// inserts its own (conservative) waits for the direct loads still in flight
// into other stages, nor moves the reads. Waits are explicit: wait_lgkm ties
// the fragment registers so no MFMA can use them before the wait.
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

template <int OFF>
__device__ inline void ds_read_b128(half8& v, uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
}

template <int OFF>
__device__ inline void ds_read_tr(half4& v, uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
}

template <int FM, int FN>
__device__ inline void wait_lgkm(half8 (&af)[FM], half4 (&bl)[FN], half4 (&bh)[FN]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(af[i]));
#pragma unroll
  for (int i = 0; i < FN; ++i) asm volatile("" : "+v"(bl[i]), "+v"(bh[i]));
}

__device__ inline void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Fragment reads of k16-substep KS from the stage at LDS address `cur`.
template <int BM, int BN, int BK, int WM, int WN, int KS>
__device__ __attribute__((always_inline)) inline void read_frags(uint32_t cur, const ReadOffsets& ro,
                                                               half8 (&af)[BM / WM / 32], half4 (&bl)[BN / WN / 32],
                                                               half4 (&bh)[BN / WN / 32]) {
  using S = Shape<BM, BN, BK, WM, WN>;
  constexpr int ROWA = BK * 2, ROWB = BN * 2;
  const uint32_t a_base = cur + ro.a[KS];
#pragma unroll
  for (int fm = 0; fm < S::FM; ++fm) {
    switch (fm) {  // immediate offsets must be compile-time constants
      case 0: ds_read_b128<0 * 32 * ROWA>(af[fm], a_base); break;
      case 1: ds_read_b128<1 * 32 * ROWA>(af[fm], a_base); break;
      case 2: ds_read_b128<2 * 32 * ROWA>(af[fm], a_base); break;
      default: ds_read_b128<3 * 32 * ROWA>(af[fm], a_base); break;
    }
  }
#pragma unroll
  for (int fn = 0; fn < S::FN; ++fn) {
    const uint32_t b_base = cur + S::A_BYTES + ro.b[fn];
    ds_read_tr<KS * 16 * ROWB>(bl[fn], b_base);
    ds_read_tr<KS * 16 * ROWB + 4 * ROWB>(bh[fn], b_base);
  }
}

template <int BM, int BN, int BK, int WM, int WN>
__device__ __attribute__((always_inline)) inline void mfmas(const half8 (&af)[BM / WM / 32],
                                                          const half4 (&bl)[BN / WN / 32],
                                                          const half4 (&bh)[BN / WN / 32],
                                                          f32x16 (&acc)[BM / WM / 32][BN / WN / 32]) {
  using S = Shape<BM, BN, BK, WM, WN>;
#pragma unroll
  for (int fn = 0; fn < S::FN; ++fn) {
    const half8 b = __builtin_shufflevector(bl[fn], bh[fn], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int fm = 0; fm < S::FM; ++fm)
      acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, af[fm], acc[fm][fn], 0, 0, 0);
  }
}

// One k-step: issue the direct loads of a later stage (`nxt`), then run the
// MFMAs of the current stage (`cur`), with the fragment reads of substep
// ks+1 in flight while the MFMAs of substep ks execute.
template <int BM, int BN, int BK, int WM, int WN>
__device__ __attribute__((always_inline)) inline void kstep(
    char* nxt, uint32_t cur, const _Float16* a_src, const _Float16* b_src, const int64_t* a_off,
    const int64_t* b_off, int wave, const ReadOffsets& ro, f32x16 (&acc)[BM / WM / 32][BN / WN / 32]) {
  using S = Shape<BM, BN, BK, WM, WN>;
#pragma unroll
  for (int j = 0; j < S::A_ITERS; ++j)
    __builtin_amdgcn_global_load_lds((const void*)(a_src + a_off[j]),
                                     (LDS_PTR(void))(nxt + (j * S::NT + wave * 64) * 16), 16, 0, 0);
#pragma unroll
  for (int j = 0; j < S::B_ITERS; ++j)
    __builtin_amdgcn_global_load_lds((const void*)(b_src + b_off[j]),
                                     (LDS_PTR(void))(nxt + S::A_BYTES + (j * S::NT + wave * 64) * 16), 16, 0, 0);

  half8 af0[S::FM], af1[S::FM];
  half4 bl0[S::FN], bh0[S::FN], bl1[S::FN], bh1[S::FN];
  read_frags<BM, BN, BK, WM, WN, 0>(cur, ro, af0, bl0, bh0);
  wait_lgkm(af0, bl0, bh0);
  if constexpr (S::KSUB >= 2) read_frags<BM, BN, BK, WM, WN, 1>(cur, ro, af1, bl1, bh1);
  mfmas<BM, BN, BK, WM, WN>(af0, bl0, bh0, acc);
  if constexpr (S::KSUB >= 2) {
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkm(af1, bl1, bh1);
    if constexpr (S::KSUB >= 3) read_frags<BM, BN, BK, WM, WN, 2>(cur, ro, af0, bl0, bh0);
    mfmas<BM, BN, BK, WM, WN>(af1, bl1, bh1, acc);
  }
  if constexpr (S::KSUB >= 3) {
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkm(af0, bl0, bh0);
    if constexpr (S::KSUB >= 4) read_frags<BM, BN, BK, WM, WN, 3>(cur, ro, af1, bl1, bh1);
    mfmas<BM, BN, BK, WM, WN>(af0, bl0, bh0, acc);
  }
  if constexpr (S::KSUB >= 4) {
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkm(af1, bl1, bh1);
    mfmas<BM, BN, BK, WM, WN>(af1, bl1, bh1, acc);
  }
}

template <int BM, int BN, int BK, int STAGES, int WM, int WN, bool GATED, bool OUTF32>
__global__ __launch_bounds__(64 * WM * WN) void gemm_mfma_kernel(GemmArgs g) {
  using S = Shape<BM, BN, BK, WM, WN>;
  constexpr int NT = S::NT, TM = S::TM, TN = S::TN, FM = S::FM, FN = S::FN;
  constexpr int CPR_A = S::CPR_A, CPR_B = S::CPR_B;
  constexpr int ROWA = BK * 2;
  static_assert(STAGES >= 2 && STAGES * S::STAGE <= 160 * 1024 - 64, "LDS budget");

  __shared__ __attribute__((aligned(1024))) char smem[STAGES * S::STAGE];
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
  const int steps_per_tile = SPS / g.gate.kt;  // k-steps per flag tile (BKf / BK)

  // LDS read offsets (tile independent). A: row (wm*TM + fm*32 + lane%32),
  // logical 16-byte chunk (2*ks + lane/32), stored at chunk ^ swz_a(row).
  // B (transpose read, 16-lane groups): lane supplies row
  // k = 16*ks + 8*(g/2) + 4*h + (i/4) and columns n = fn*32 + 16*(g%2) + 4*(i%4)
  // of the wave's range, chunk (n/8) ^ swz_b(k); swz_b(k) does not depend on ks or h.
  ReadOffsets ro;
  {
    const int row = wm * TM + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < S::KSUB; ++ks)
      ro.a[ks] = row * ROWA + (((ks * 2 + (lane >> 5)) ^ swz_a<CPR_A>(row)) * 16);
    const int g16 = lane >> 4, i16 = lane & 15;
    const int k = (g16 >> 1) * 8 + (i16 >> 2);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int n = wn * TN + fn * 32 + (g16 & 1) * 16 + (i16 & 3) * 4;
      ro.b[fn] = k * (BN * 2) + (((n >> 3) ^ swz_b(k)) * 16) + (n & 7) * 2;
    }
  }

  // Flag gate. Every wave polls the flags itself and gates only its own
  // direct loads, so the gate needs no barrier and no LDS broadcast. `ready`
  // (wave-uniform) remembers the tiles this wave has already seen raised, so
  // after the first poll of a launch that finds every flag up no further
  // polls happen. A wave whose wait times out records the error, marks the
  // workgroup aborted and from then on skips waiting but keeps the same
  // barrier sequence; the workgroup drops the tile at its end.
  uint64_t ready = 0;
  bool dead = false;
  if (tid == 0) s_abort = 0;
  __syncthreads();
  auto gate = [&](int t) {
    if constexpr (GATED) {
      const int s = t / SPS;
      const int tile = s * g.gate.kt + (t - s * SPS) / steps_per_tile;
      if (((ready >> tile) & 1ull) || dead) return;
      const uint64_t start = wall_clock();
      uint64_t mask = 0;
      uint32_t seen = 0;
      while (true) {
        bool up = false;
        if (lane < g.gate.t) {
          const uint32_t v = __hip_atomic_load(const_cast<uint32_t*>(g.gate.flags) + lane, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
          up = (int32_t)(v - g.gate.target) >= 0;
          if (lane == tile) seen = v;
        }
        mask = __ballot(up);
        if ((mask >> tile) & 1ull) break;
        if (wall_clock() - start > g.gate.timeout_ticks) {
          dead = true;
          if (lane == tile) {
            __hip_atomic_store(&g.gate.err->tile, (uint32_t)tile, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            __hip_atomic_store(&g.gate.err->target, g.gate.target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            __hip_atomic_store(&g.gate.err->seen, seen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            __hip_atomic_store(&g.gate.err->code, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
            s_abort = 1;
          }
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      // The tiles' inbox lines have not been read in this launch before their
      // flags were seen, so no cache can hold a stale copy; the direct loads
      // that follow are ordered after the flag values by control dependency.
      // The strict mode adds the formal agent-scope acquire (an L2-wide
      // invalidate, costly when many waves issue it).
      if (g.gate.strict) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      asm volatile("" ::: "memory");
      ready = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(mask >> 32)) << 32) |
              (uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)mask);
    }
  };

  // Persistent loop over output tiles. Workgroups are dealt round-robin to
  // the 8 XCDs; each XCD gets a contiguous range of logical tiles, ordered in
  // groups of 8 row-blocks, so tiles running together on one XCD share A and
  // B rows in its L2.
  const int G = gridDim.x;
  const bool xcd_split = (total % 8 == 0) && (G % 8 == 0);
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
    int64_t a_off[S::A_ITERS];
#pragma unroll
    for (int j = 0; j < S::A_ITERS; ++j) {
      const int q = j * NT + wave * 64 + lane;
      const int r = q / CPR_A;
      const int c = (q % CPR_A) ^ swz_a<CPR_A>(r);
      int64_t m = m0 + r;
      if (m > M - 1) m = M - 1;  // rows past M load a valid row; their results are not stored
      a_off[j] = m * g.a.lda + c * 8;
    }
    int64_t b_off[S::B_ITERS];
#pragma unroll
    for (int j = 0; j < S::B_ITERS; ++j) {
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
    auto issue = [&](int t, int stage) {
      const _Float16* as = a_src(t);
      const _Float16* bs = b_src(t);
      char* dst = smem + stage * S::STAGE;
#pragma unroll
      for (int j = 0; j < S::A_ITERS; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(as + a_off[j]),
                                         (LDS_PTR(void))(dst + (j * NT + wave * 64) * 16), 16, 0, 0);
#pragma unroll
      for (int j = 0; j < S::B_ITERS; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(bs + b_off[j]),
                                         (LDS_PTR(void))(dst + S::A_BYTES + (j * NT + wave * 64) * 16), 16, 0, 0);
    };

    __syncthreads();  // the previous tile's last reads of LDS are done
    // Prologue: stages 0 .. STAGES-2 (steps past the end re-load the last step
    // into a stage nobody reads, keeping the count of loads in flight uniform).
#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p) {
      const int tp = p < NS ? p : NS - 1;
      gate(tp);
      issue(tp, p);
    }
    // Steady state: wait for the oldest stage, then issue STAGES-1 steps ahead
    // and compute. One loop body for every k-step (a single copy of the MFMA
    // code keeps the accumulators in place).
    const uint32_t smem_lds = lds_addr(smem);
    for (int t = 0; t < NS; ++t) {
      // This thread's loads of stage t are done once at most STAGES-2 later
      // stages are still in flight; the barrier then publishes every thread's
      // part of stage t and tells all waves that stage t-1 is free again.
      wait_vmcnt<(STAGES - 2) * S::LOADS>();
      barrier();
      const int ahead = t + STAGES - 1;
      const int tn = ahead < NS ? ahead : NS - 1;
      gate(tn);
      kstep<BM, BN, BK, WM, WN>(smem + (ahead % STAGES) * S::STAGE, smem_lds + (t % STAGES) * S::STAGE, a_src(tn),
                                b_src(tn), a_off, b_off, wave, ro, acc);
    }
    __builtin_amdgcn_s_waitcnt(0);  // drain the direct loads before storing or leaving
    if constexpr (GATED) {
      __syncthreads();
      if (__builtin_amdgcn_readfirstlane(s_abort)) break;  // a flag wait timed out: C is left undefined
    }

    // Epilogue: lane holds C[m][n .. n+3] for m = lane % 32 of each 32-row
    // block and n = (fn*32 + q*8) + 4*(lane/32) within the wave's columns.
    // One row pointer per 32-row block; the column offsets are compile-time
    // immediates of the stores. Full tiles skip the bounds checks.
    const int64_t col0 = n0 + wn * TN + (lane >> 5) * 4;
    const bool full = (m0 + BM <= M) && (n0 + BN <= N);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int64_t m = m0 + wm * TM + fm * 32 + (lane & 31);
      if (!full && m >= M) continue;
      if constexpr (OUTF32) {
        float* row = static_cast<float*>(g.C) + m * N + col0;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = fn * 32 + q * 8;
            if (!full && col0 + c >= N) continue;
            float4 v = make_float4(acc[fm][fn][q * 4 + 0], acc[fm][fn][q * 4 + 1], acc[fm][fn][q * 4 + 2],
                                   acc[fm][fn][q * 4 + 3]);
            *reinterpret_cast<float4*>(row + c) = v;
          }
        }
      } else {
        _Float16* row = static_cast<_Float16*>(g.C) + m * N + col0;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = fn * 32 + q * 8;
            if (!full && col0 + c >= N) continue;
            half4 v;
            v[0] = (_Float16)acc[fm][fn][q * 4 + 0];
            v[1] = (_Float16)acc[fm][fn][q * 4 + 1];
            v[2] = (_Float16)acc[fm][fn][q * 4 + 2];
            v[3] = (_Float16)acc[fm][fn][q * 4 + 3];
            *reinterpret_cast<half4*>(row + c) = v;
          }
        }
      }
    }
  }
}

template <int BM, int BN, int BK, int STAGES, int WM, int WN>
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
#define AGEMM_LAUNCH(G_, F_) \
  hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, BK, STAGES, WM, WN, G_, F_>), grid, block, 0, s, a)
  if (gated) {
    if (out_f32) AGEMM_LAUNCH(true, true);
    else AGEMM_LAUNCH(true, false);
  } else {
    if (out_f32) AGEMM_LAUNCH(false, true);
    else AGEMM_LAUNCH(false, false);
  }
#undef AGEMM_LAUNCH
  return hipGetLastError();
}

}  // namespace

int mfma_config_count() { return 4; }

hipError_t launch_gemm_mfma(const GemmArgs& a, bool out_f32, hipStream_t s) {
  int cfg = a.tile_config;
  if (cfg < 0) cfg = a.M > 256 ? 0 : 2;
  switch (cfg) {
    case 0: return launch_cfg<256, 256, 64, 2, 2, 4>(a, out_f32, s);
    case 1: return launch_cfg<256, 256, 32, 4, 2, 4>(a, out_f32, s);
    case 2: return launch_cfg<128, 128, 64, 2, 2, 2>(a, out_f32, s);
    default: return launch_cfg<128, 128, 32, 4, 2, 2>(a, out_f32, s);
  }
}

}  // namespace agemm
