// Flag-gated shard-decomposed GEMM on gfx950 matrix cores.
//
// Computes C = sum_{s=0}^{W-1} A_s . B[s*KS:(s+1)*KS, :] ("Eliminating
// Multi-GPU Performance Taxes" analysis page, AG+GEMM core identity): each
// workgroup owns BM x BN tiles of C (persistent loop over tiles) and walks K
// shard by shard, the loop order the page gives for the Pull and Push GEMMs.
// With the gate on (Push model) each wave checks, when its load cursor enters
// a (shard, k-tile) and before any load of that tile, that the tile's flag
// has reached the epoch's target: its lanes poll all T flags at once with
// relaxed agent-scope loads, and the wave remembers which tiles it has seen
// raised, so a launch that finds every flag raised pays for one poll per
// wave. The check sits in the cursor's tile-crossing branch (taken once per
// k-tile), not in the per-k-step path: a gate test in every k-step, or a
// second gate-free copy of the loop beside a gated one, measurably slowed the
// MFMA issue of the whole kernel.
//
// Data path (BK-wide k-steps, ring of STAGES LDS buffers):
//   A_s, B -> LDS : 16-byte direct loads (global_load_lds). One uniform base
//                   pointer per k-step plus a fixed 32-bit offset per lane. A
//                   comes from a row-major shard or from the k-panel inbox
//                   (32-column panels of M rows, where a tile's k-step is one
//                   contiguous run); A rows (BK*2 bytes) and B rows (BN*2
//                   bytes) are stored with the 16-byte chunk index
//                   XOR-swizzled so that the reads below are free of LDS bank
//                   conflicts;
//   LDS -> regs   : A fragments with 16-byte reads, B fragments with
//                   transpose reads (ds_read_b64_tr_b16), which turn the
//                   N-contiguous B rows into the K-contiguous operand;
//   math          : v_mfma_f32_32x32x16_f16 with the roles swapped (the B^T
//                   block is the first operand), so a lane ends up holding four
//                   consecutive C columns and stores them with one store.
//
// Schedule. The only workgroup barrier of a k-step sits in its last k16
// substep, after that substep's fragments are already in registers: the
// barrier frees the step's LDS buffer and publishes the next one, whose first
// fragments are then read between the last substep's MFMAs. The direct loads
// run on a cursor that is STAGES-1 steps ahead and crosses output-tile
// boundaries (no pipeline drain per tile); each barrier interval issues one
// cursor step's loads, one every few MFMAs, into the buffer the barrier freed,
// so they never arrive in a burst that would stall the fragment reads.
//
// Tile shapes. Three, all of four waves: 256x256 (128x128 wave tiles, 256
// fp32 accumulators per lane held in AGPRs: a third less LDS per MFMA than
// eight waves with 128x64 tiles, which measured slower), 128x128 for M up to
// 128 and 256x128 for M up to 256 (one row block: B is read once). At
// M = 4096 the MFMA pipes are busy about 73 % of the cycles at the 1.6-1.7
// GHz the part holds under this load (a register-only MFMA loop holds 2.4
// GHz). Copies of the kernel without the barrier or without the waits run no
// faster; without the A loads it runs 6.5 % faster whatever memory they read:
// the wave's own issue of loads and fragment reads, and the clock that the
// power of all of it sets, bound the rate.
#include "agemm_internal.h"
#include "mfma_sched.h"

#include <algorithm>

namespace agemm {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
#define LDS_PTR(T) __attribute__((address_space(3))) T*

__device__ inline uint64_t wall_clock() { return __builtin_amdgcn_s_memrealtime(); }
// A 64-lane ballot made wave-uniform. readfirstlane returns a signed int:
// each half goes through uint32_t so that bit 31 is not sign-extended into
// the upper half (which would mark every flag tile from 32 on as raised).
__device__ inline uint64_t uniform_mask(uint64_t mask) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)mask);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(mask >> 32));
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}
using sched::swz_a;
using sched::swz_b;

template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ inline void barrier() { asm volatile("s_barrier" ::: "memory"); }
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

template <int BM, int BN, int BK, int WM, int WN>
struct Shape {
  static constexpr int NT = 64 * WM * WN;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int NMF = FM * FN;               // MFMAs per wave per k16 substep
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int B_BYTES = BK * BN * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int CPR_A = BK / 8;
  static constexpr int CPR_B = BN / 8;
  static constexpr int A_ITERS = (BM * BK / 8) / NT;
  static constexpr int B_ITERS = (BK * BN / 8) / NT;
  static constexpr int LOADS = A_ITERS + B_ITERS;   // direct loads per thread per k-step
  static constexpr int KSUB = BK / 16;
  static constexpr int LPS = LOADS / KSUB;          // direct loads per substep
  static constexpr int NR = FM + 2 * FN;            // fragment reads per substep
  static constexpr bool AGPR = NMF >= 16;           // accumulators pinned in AGPRs
  static_assert(A_ITERS * NT == BM * BK / 8 && B_ITERS * NT == BK * BN / 8, "tile/thread mismatch");
  static_assert(CPR_B >= 16, "B row must hold at least 16 chunks for the swizzle");
  static_assert(CPR_A == 4 || CPR_A == 8, "BK must be 32 or 64");
  static_assert(KSUB == 2 || KSUB == 4, "two or four k-substeps");
  static_assert(LPS * KSUB == LOADS && LPS <= NMF, "loads must spread evenly over the substeps");
  static constexpr int LSTRIDE = (NMF + LPS - 1) / LPS;  // one direct load every LSTRIDE MFMAs
  static_assert((LPS - 1) * LSTRIDE < NMF, "a substep issues all its loads between its MFMAs");
  static_assert(FM <= 4 && FN <= 4, "at most 4x4 MFMA blocks per wave");
};

template <int FM, int FN>
struct Frags {
  half8 a[FM];
  half4 bl[FN], bh[FN];
};

template <int FM, int FN>
__device__ inline void wait_frags(Frags<FM, FN>& f) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(f.a[i]));
#pragma unroll
  for (int i = 0; i < FN; ++i) asm volatile("" : "+v"(f.bl[i]), "+v"(f.bh[i]));
}

// Read r of substep KS: r < FM are the A blocks (one 16-byte read each),
// then two transpose reads per B block.
template <int BM, int BN, int BK, int WM, int WN, int KS>
__device__ __attribute__((always_inline)) inline void read_one(int r, uint32_t stage, int a_off,
                                                             const int (&b_off)[BN / WN / 32],
                                                             Frags<BM / WM / 32, BN / WN / 32>& f) {
  using S = Shape<BM, BN, BK, WM, WN>;
  constexpr int ROWA = BK * 2, ROWB = BN * 2;
  if (r < S::FM) {
    const uint32_t a_base = stage + a_off;
    switch (r) {
      case 0: ds_read_b128<0 * 32 * ROWA>(f.a[0], a_base); break;
      case 1: ds_read_b128<1 * 32 * ROWA>(f.a[1 % S::FM], a_base); break;
      case 2: ds_read_b128<2 * 32 * ROWA>(f.a[2 % S::FM], a_base); break;
      default: ds_read_b128<3 * 32 * ROWA>(f.a[3 % S::FM], a_base); break;
    }
  } else {
    const int fn = (r - S::FM) >> 1, h = (r - S::FM) & 1;
    const uint32_t b_base = stage + S::A_BYTES + b_off[fn];
    if (h == 0) ds_read_tr<KS * 16 * ROWB>(f.bl[fn], b_base);
    else ds_read_tr<KS * 16 * ROWB + 4 * ROWB>(f.bh[fn], b_base);
  }
}

template <int BM, int BN, int BK, int WM, int WN>
__device__ __attribute__((always_inline)) inline void read_one_ks(int ks, int r, uint32_t stage, const int (&ra)[4],
                                                                const int (&b_off)[BN / WN / 32],
                                                                Frags<BM / WM / 32, BN / WN / 32>& f) {
  switch (ks) {
    case 0: read_one<BM, BN, BK, WM, WN, 0>(r, stage, ra[0], b_off, f); break;
    case 1: read_one<BM, BN, BK, WM, WN, 1>(r, stage, ra[1], b_off, f); break;
    case 2: read_one<BM, BN, BK, WM, WN, 2>(r, stage, ra[2], b_off, f); break;
    default: read_one<BM, BN, BK, WM, WN, 3>(r, stage, ra[3], b_off, f); break;
  }
}

// MFMA i of a substep (fn-major). With 256 accumulators per lane they are
// kept in AGPRs through an "a" operand: otherwise the allocator moves them to
// architectural VGPRs for the epilogue's conversions and spills.
template <int FM, int FN, bool AGPR>
__device__ __attribute__((always_inline)) inline void mfma_one(const Frags<FM, FN>& f, f32x16 (&acc)[FM][FN], int i) {
  const int fn = i / FM, fm = i % FM;
  const half8 b = __builtin_shufflevector(f.bl[fn], f.bh[fn], 0, 1, 2, 3, 4, 5, 6, 7);
  if constexpr (AGPR)
    asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc[fm][fn]) : "v"(b), "v"(f.a[fm]));
  else
    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, f.a[fm], acc[fm][fn], 0, 0, 0);
}

// Device-coherent (agent-scope) 8-byte store and load of the split-K partials:
// they bypass the per-XCD L2s, so a partial written on one XCD is read
// correctly on another without an L2-wide fence.
__device__ inline void store_coherent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t load_coherent(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// BNT: B is read by exactly one tile (one row block of C): its direct loads
// are nontemporal (no L2 allocation).
template <int BM, int BN, int BK, int STAGES, int WM, int WN, bool GATED, bool OUTF32, bool SPLIT, bool ARRIVAL,
          bool BNT = false>
__global__ __launch_bounds__(64 * WM * WN) void gemm_mfma_kernel(GemmArgs g) {
  static_assert(!ARRIVAL || (GATED && !SPLIT), "arrival order is a mode of the gated whole-tile consumer");
  using S = Shape<BM, BN, BK, WM, WN>;
  constexpr int NT = S::NT, TM = S::TM, TN = S::TN, FM = S::FM, FN = S::FN, LOADS = S::LOADS;
  constexpr int CPR_A = S::CPR_A, KSUB = S::KSUB, NMF = S::NMF, NR = S::NR, LPS = S::LPS;
  constexpr bool AGPR = S::AGPR;
  constexpr int ROWA = BK * 2;
  static_assert(STAGES >= 2 && STAGES * S::STAGE <= 160 * 1024, "LDS budget");
  static_assert(STAGES * LOADS <= 63, "loads in flight exceed the vmcnt range");
  constexpr int RPM = (NR + NMF / 2 - 1) / (NMF / 2);  // fragment reads after each of the first MFMAs
  constexpr int LSTRIDE = S::LSTRIDE;

  __shared__ __attribute__((aligned(1024))) char smem[STAGES * S::STAGE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave / WN;
  const int wn = wave - wm * WN;

  const int64_t M = g.M, N = g.N;
  const int SPS = (int)(g.KS / BK);
  const int NS = (int)(g.K / BK);
  const int G = gridDim.x;
  const sched::TileGrid tg = sched::tile_grid(M, N, BM, BN, G);
  // Work of this workgroup as segments (a tile and its k-steps), whole tiles
  // or the stream-K split's run of (tile, shard) units: see mfma_sched.h.
  const int Wsh = g.W;
  const sched::Work wk = sched::work_of((int)blockIdx.x, G, tg.total, Wsh, SPS, SPLIT);
  const int bp = wk.bp;
  using Seg = sched::Seg;
  auto seg_first = [&](Seg& q) { sched::seg_first(wk, q); };
  auto seg_next = [&](Seg& q) -> bool { return sched::seg_next(wk, q); };

  // LDS read offsets, fixed for the launch. B (transpose read, 16-lane
  // groups): lane supplies row k = 16*ks + 8*(g/2) + 4*h + (i/4) and columns
  // n = fn*32 + 16*(g%2) + 4*(i%4) of the wave's range, stored at chunk
  // (n/8) ^ swz_b(k); swz_b(k) does not depend on ks or h, which become
  // immediate offsets. A: row wm*TM + fm*32 + lane%32, logical chunk
  // 2*ks + lane/32 stored at chunk ^ swz_a(row); one offset per substep.
  int rb[FN];
  {
    const int g16 = lane >> 4, i16 = lane & 15;
    const int k = (g16 >> 1) * 8 + (i16 >> 2);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int n = wn * TN + fn * 32 + (g16 & 1) * 16 + (i16 & 3) * 4;
      rb[fn] = k * (BN * 2) + (((n >> 3) ^ swz_b(k)) * 16) + (n & 7) * 2;
    }
  }
  int ra_ks[4] = {0, 0, 0, 0};
  {
    const int row = wm * TM + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < KSUB; ++ks) ra_ks[ks] = row * ROWA + (((ks * 2 + (lane >> 5)) ^ swz_a<CPR_A>(row)) * 16);
  }

  // Direct-load cursor: the (tile, k-step) whose loads are issued next. It is
  // advanced with additions only; its flag tile feeds the gate. Past the last
  // tile it keeps re-loading the last step into buffers nobody reads, which
  // keeps the count of loads in flight, and so every wait, uniform.
  Seg cseg;                                  // segment of the cursor
  seg_first(cseg);
  sched::KPos kp{};                          // shard order: position and next event step
  int ct = 0, cfsub = 0;                     // arrival order: k-step in the tile and in its flag tile
  const int spt = SPS / g.gate.kt;
  bool track = GATED;                        // a flag of this launch may still be unseen
  const char* cb = nullptr;
  const char* ca = nullptr;
  int64_t a_row0 = 0;
  uint32_t a_off[S::A_ITERS], b_off[S::B_ITERS];
  const int64_t lda2 = g.a.lda * 2;
  // A's byte step from one k-step to the next: BK columns of a row-major
  // shard, or BK / 32 whole panels of the k-panel layout.
  const bool panels = g.a.panels != 0;
  const int64_t panel_bytes = M * (kPanelK * 2);
  const int64_t a_kstep = panels ? (int64_t)(BK / kPanelK) * panel_bytes : (int64_t)BK * 2;

  // Flag gate of the tile the cursor enters (called from cursor_enter and at
  // each flag-tile crossing of cursor_advance, before any load of the tile).
  // `ready` (wave-uniform) remembers the tiles this wave has seen raised. A wave whose wait times out records the
  // error and stops waiting; the launch still runs to its end with the same
  // barrier sequence, and C is undefined.
  uint64_t ready = 0;
  bool dead = false;
  // Arrival order (ARRIVAL only). The sum over shards may be taken in any
  // order, so at each flag-tile boundary of an output tile wave 0 picks the
  // lowest-numbered flag tile it has seen raised and not yet taken (polling
  // only when there is none) and publishes the choice through LDS; every
  // wave applies it after the next workgroup barrier, so all waves load the
  // same flag tile into each stage. Two alternating slots: a choice is
  // written only after every wave has passed the barrier that follows the
  // read of the choice before it.
  __shared__ int s_choice[2];
  uint64_t taken = 0;
  int wslot = 0, rslot = 0;
  bool pending = false;  // a choice waits to be applied after the next barrier
  int64_t c_n0 = 0;
  const uint64_t tmask = sched::flag_mask(g.gate.t);
  auto gate = [&](const int tile) {
    if constexpr (GATED) {
      // Fast path (tile already seen, or given up) falls through without a
      // taken branch: with one wave per SIMD a taken branch per k-step stalls
      // the MFMA issue measurably.
      if (__builtin_expect(((ready >> tile) & 1ull) || dead, 1)) return;
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
          }
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      // The tiles' inbox lines have not been read in this launch before their
      // flags were seen, so no cache holds a stale copy, and the loads that
      // follow are ordered after the flag values by control dependency. The
      // strict mode adds the formal agent-scope acquire (an L2-wide
      // invalidate, costly when many waves issue it).
      if (g.gate.strict) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      asm volatile("" ::: "memory");
      ready = uniform_mask(mask);
    }
  };
  auto tile_coords = [&](int w, int64_t& m0, int64_t& n0) {
    int mb, nb;
    sched::tile_coords(tg, SPLIT, w, mb, nb);
    m0 = (int64_t)mb * BM;
    n0 = (int64_t)nb * BN;
  };
  // Arrival order: wave 0's choice of the next flag tile (see above). If no
  // untaken tile comes up within the timeout it takes the lowest untaken one,
  // whose gate then reports the timeout.
  auto choose = [&]() {
    if constexpr (ARRIVAL) {
      if (wave == 0) {
        uint64_t c = ready & ~taken & tmask;
        if (c == 0 && !dead) {
          const uint64_t start = wall_clock();
          while (true) {
            bool up = false;
            if (lane < g.gate.t)
              up = (int32_t)(__hip_atomic_load(const_cast<uint32_t*>(g.gate.flags) + lane, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT) - g.gate.target) >= 0;
            ready |= uniform_mask(__ballot(up));
            c = ready & ~taken & tmask;
            if (c != 0 || wall_clock() - start > g.gate.timeout_ticks) break;
            __builtin_amdgcn_s_sleep(2);
          }
        }
        if (lane == 0) s_choice[wslot] = sched::arrival_pick(ready, taken, tmask);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
      wslot ^= 1;
      pending = true;
    }
  };
  // Lane offsets of tile w: the LDS destination of chunk q is byte q*16 of
  // the stage; rows past M and columns past N re-load a valid row/column
  // whose results are never stored. m0 and n0 go into the base pointers.
  auto cursor_enter = [&]() {
    int64_t m0, n0;
    tile_coords(cseg.w, m0, n0);
    const int rmax = (int)(M - 1 - m0);
#pragma unroll
    for (int j = 0; j < S::A_ITERS; ++j) {
      const int q = j * NT + wave * 64 + lane;
      a_off[j] = panels ? sched::a_src_offset_panels<BK>(q, rmax, panel_bytes) : sched::a_src_offset<BK>(q, rmax, lda2);
    }
    const int cmax = (int)(N - 8 - n0);
#pragma unroll
    for (int j = 0; j < S::B_ITERS; ++j) b_off[j] = sched::b_src_offset<BN>(j * NT + wave * 64 + lane, cmax, N);
    a_row0 = panels ? m0 * (kPanelK * 2) : m0 * lda2;
    if constexpr (ARRIVAL) {
      c_n0 = n0;
      ct = 0;
      cfsub = 0;
      taken = 0;
      choose();
      return;
    }
    // A segment starts at a shard border.
    sched::kpos_enter(kp, cseg, SPS, spt, g.gate.kt, track);
    ca = (const char*)g.a.base[kp.cs] + a_row0;
    cb = (const char*)g.B + n0 * 2 + (int64_t)cseg.kb * BK * N * 2;
    gate(kp.cft);
  };
  // Arrival order: applies the published choice (after a barrier): points the
  // cursor at the flag tile's first k-step and gates it. The choice is one of
  // the tile's untaken flag tiles (masked with T), so every k-step of the
  // output tile is loaded exactly once.
  auto arrival_apply = [&]() {
    const int f = __builtin_amdgcn_readfirstlane(s_choice[rslot]);
    rslot ^= 1;
    pending = false;
    taken |= 1ull << f;
    const int fs = f / g.gate.kt;
    const int step = sched::flag_first_step(f, g.gate.kt, SPS, spt);
    ca = (const char*)g.a.base[fs] + a_row0 + (int64_t)(step - fs * SPS) * a_kstep;
    cb = (const char*)g.B + c_n0 * 2 + (int64_t)step * BK * N * 2;
    gate(f);
  };
  // Shard order: the common k-step is two pointer bumps, a counter and one
  // branch that is not taken (with one wave per SIMD a taken branch in every
  // k-step stalls the MFMA issue; the compiler keeps every counter in scalar
  // registers only with the segment end tested apart from the event step);
  // shard, flag-tile and segment borders go through cursor_event. Past the
  // last tile the cursor keeps re-loading the last step into buffers nobody
  // reads, which keeps the count of loads in flight, and so every wait,
  // uniform.
  auto cursor_event = [&]() __attribute__((always_inline)) {
    if (kp.ct == cseg.ke) {
      if (seg_next(cseg)) {
        cursor_enter();
      } else {
        ca -= a_kstep;
        cb -= (int64_t)BK * N * 2;
        kp.ct = cseg.ke - 1;
      }
      return;
    }
    const int ev = sched::kpos_event(kp, cseg.ke, SPS, spt, track);
    if (ev & sched::kEvShard) ca = (const char*)g.a.base[kp.cs] + a_row0;
    if (ev & sched::kEvFlag) {
      gate(kp.cft);
      // every flag seen raised (or the wait given up): no gate from here on
      if (__builtin_amdgcn_readfirstlane((int)(((ready & tmask) == tmask) || dead))) track = false;
    }
  };
  auto cursor_advance = [&]() {
    if constexpr (ARRIVAL) {
      if (++ct == cseg.ke) {
        if (seg_next(cseg)) cursor_enter();
        else ct = cseg.ke - 1;
        return;
      }
      if (++cfsub == spt) {
        cfsub = 0;
        choose();
      } else {
        cb += (int64_t)BK * N * 2;
        ca += a_kstep;
      }
      return;
    }
    ca += a_kstep;
    cb += (int64_t)BK * N * 2;
    if (__builtin_expect(sched::kpos_step(kp, cseg.ke), 0)) cursor_event();
  };

  auto issue_one = [&](int j, int buf) {
    char* dst = smem + buf * S::STAGE;
    if (j < S::A_ITERS)
      __builtin_amdgcn_global_load_lds((const void*)(ca + a_off[j]),
                                       (LDS_PTR(void))(dst + (j * NT + wave * 64) * 16), 16, 0, 0);
    else
      __builtin_amdgcn_global_load_lds((const void*)(cb + b_off[j - S::A_ITERS]),
                                       (LDS_PTR(void))(dst + S::A_BYTES + ((j - S::A_ITERS) * NT + wave * 64) * 16),
                                       16, 0, BNT ? 2 : 0);
  };

  const uint32_t lds0 = lds_addr(smem);
  Frags<FM, FN> F0, F1;

  // First look at the flags with plain loads, which the per-XCD L2 serves
  // after one miss: a device-coherent poll from every wave of the grid would
  // queue a thousand requests on one memory line at launch. A cached flag can
  // only lag the true value (flags only grow within the wrap window), so a
  // flag seen raised here is raised; one seen down is polled coherently by
  // the gate when it is needed.
  if constexpr (GATED) {
    bool up = false;
    if (lane < g.gate.t) up = (int32_t)(g.gate.flags[lane] - g.gate.target) >= 0;
    const uint64_t mask = __ballot(up);
    ready = uniform_mask(mask);
    if (g.gate.strict) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    asm volatile("" ::: "memory");
  }

  // Prologue: steps 0 .. STAGES-2 in full; the interval opened by the
  // prologue barrier then loads step STAGES-1 into the last buffer.
  cursor_enter();
  if constexpr (ARRIVAL) {
    barrier();
    arrival_apply();
  }
#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p) {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) issue_one(j, p);
    cursor_advance();
    if constexpr (ARRIVAL) {
      if (pending) {
        barrier();
        arrival_apply();
      }
    }
  }
  wait_vmcnt<(STAGES - 2) * LOADS>();
  barrier();
  if constexpr (ARRIVAL) {
    if (pending) arrival_apply();
  }
  int dbuf = STAGES - 1;  // buffer the current interval's direct loads go to
#pragma unroll
  for (int j = 0; j < LPS; ++j) issue_one(j, dbuf);
#pragma unroll
  for (int r = 0; r < NR; ++r) read_one_ks<BM, BN, BK, WM, WN>(0, r, lds0, ra_ks, rb, F0);

  // Split-K hand-off (SPLIT only). Owner of unit u: the largest b with
  // floor(b*U/G) <= u. Each workgroup publishes at most two partials, for its
  // first and its last tile, in slots 2*b and 2*b + 1; one ticket counter per
  // tile.
  __shared__ uint32_t s_ticket;
  auto owner = [&](int64_t u) { return sched::owner(wk, u); };
  auto slot_of = [&](int b, int w) { return sched::slot_of(wk, b, w); };
  constexpr int SLOT_U64 = BM * BN / 2;  // one slot in 8-byte words
  // Word h of block (fm, fn) of thread tid: contiguous across the workgroup.
  auto slot_word = [&](int fm, int fn, int h) { return ((fm * FN + fn) * 8 + h) * NT + tid; };

  auto main_loop = [&]() {
    int buf = 0;
    Seg ms;
    seg_first(ms);
    do {
      const int w = ms.w;
      f32x16 acc[FM][FN];
  #pragma unroll
      for (int i = 0; i < FM; ++i)
  #pragma unroll
        for (int j = 0; j < FN; ++j)
  #pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

      // One k-step; the loop below runs two per iteration (one taken branch
      // per two k-steps: measured 0.65 % faster at M = 4096 than one per step).
      auto kstep = [&]() __attribute__((always_inline)) {
        const uint32_t cur = lds0 + buf * S::STAGE;
        const int nbuf = buf + 1 == STAGES ? 0 : buf + 1;
        // Substeps 0 .. KSUB-2: MFMAs of this substep, with the next substep's
        // fragment reads (in the first half) and this interval's direct loads
        // (one every LSTRIDE MFMAs) between them.
  #pragma unroll
        for (int ks = 0; ks < KSUB - 1; ++ks) {
          Frags<FM, FN>& fc = (ks & 1) ? F1 : F0;
          Frags<FM, FN>& fnx = (ks & 1) ? F0 : F1;
          wait_frags(fc);
  #pragma unroll
          for (int i = 0; i < NMF; ++i) {
            mfma_one<FM, FN, AGPR>(fc, acc, i);
  #pragma unroll
            for (int r = i * RPM; r < (i + 1) * RPM && r < NR; ++r)
              read_one_ks<BM, BN, BK, WM, WN>(ks + 1, r, cur, ra_ks, rb, fnx);
            if (i % LSTRIDE == 0) issue_one((ks + 1) * LPS + i / LSTRIDE, dbuf);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        cursor_advance();  // every load of the cursor's step is out
        // Last substep: its fragments are in registers; after the barrier this
        // stage is free (the next interval loads into it) and the next stage is
        // complete (its first fragments are read between the MFMAs).
        Frags<FM, FN>& fl = ((KSUB - 1) & 1) ? F1 : F0;
        Frags<FM, FN>& f0 = ((KSUB - 1) & 1) ? F0 : F1;
        wait_frags(fl);
        wait_vmcnt<(STAGES - 2) * LOADS>();
        barrier();
        if constexpr (ARRIVAL) {
          if (pending) arrival_apply();
        }
        dbuf = buf;
        const uint32_t nxt = lds0 + nbuf * S::STAGE;
  #pragma unroll
        for (int i = 0; i < NMF; ++i) {
          mfma_one<FM, FN, AGPR>(fl, acc, i);
  #pragma unroll
          for (int r = i * RPM; r < (i + 1) * RPM && r < NR; ++r)
            read_one_ks<BM, BN, BK, WM, WN>(0, r, nxt, ra_ks, rb, f0);
          if (i % LSTRIDE == 0) issue_one(i / LSTRIDE, dbuf);
          __builtin_amdgcn_sched_barrier(0);
        }
        buf = nbuf;
      };
      int t = ms.kb;
      for (; t + 1 < ms.ke; t += 2) {
        kstep();
        kstep();
      }
      if constexpr (BK != 32) {  // BK = 32: a segment (whole shards of 64k columns) has an even step count
        if (t < ms.ke) kstep();
      }

      if constexpr (AGPR) {
        // the assembler MFMAs' results are read below: let the last ones retire
        asm volatile("s_nop 15\n s_nop 15\n s_nop 15\n s_nop 15" ::: "memory");
      }
      // A tile whose units fall to several workgroups: each publishes its
      // partial sums (device-coherent stores, which bypass the per-XCD L2s),
      // waits until they have completed, and then counts itself in with one
      // atomic; the workgroup that counts in last already sees every other
      // partial, adds all of them in contributor order (its own from its
      // registers) and writes C. Nobody waits for anybody, and the result
      // does not depend on which workgroup finishes last. (A variant in
      // which only the non-last contributors published, and the last polled
      // a publication counter, failed on MI355X: the poll kept reading a
      // stale count while the others' increments landed.)
      bool reduce = false;
      int gfirst = 0, ncontrib = 1;
      if constexpr (SPLIT) {
        if (ms.kb != 0 || ms.ke != NS) {
          const int64_t uf = (int64_t)w * Wsh;
          gfirst = owner(uf);
          ncontrib = owner(uf + Wsh - 1) - gfirst + 1;
          uint64_t* dst = reinterpret_cast<uint64_t*>(g.split_ws) + (int64_t)slot_of(bp, w) * SLOT_U64;
  #pragma unroll
          for (int fm = 0; fm < FM; ++fm)
  #pragma unroll
            for (int fn = 0; fn < FN; ++fn)
  #pragma unroll
              for (int h = 0; h < 8; ++h) {
                // copy the elements out first: a bit cast applied to a vector
                // element itself was compiled as a read of element 0
                const float lo = acc[fm][fn][2 * h], hi = acc[fm][fn][2 * h + 1];
                store_coherent(dst + slot_word(fm, fn, h), ((uint64_t)__builtin_bit_cast(uint32_t, hi) << 32) |
                                                               __builtin_bit_cast(uint32_t, lo));
              }
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
          uint32_t* cnt = g.split_cnt + w;
          if (tid == 0) s_ticket = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __syncthreads();
          const uint32_t ticket = __builtin_amdgcn_readfirstlane(s_ticket);
          if (ticket + 1 != (uint32_t)ncontrib) continue;
          // every contributor has counted in: clear the counter for the next call
          if (tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          reduce = true;
        }
      }
      // Sum of block (fm, fn) over the contributors in order, this
      // workgroup's own partial taken from its registers.
      auto total_of = [&](int fm, int fn) -> f32x16 {
        f32x16 v = acc[fm][fn];
        if constexpr (SPLIT) {
          if (reduce) {
            const int me = bp - gfirst;
            for (int j = 0; j < ncontrib; ++j) {
              f32x16 p;
              if (j == me) {
                p = acc[fm][fn];
              } else {
                const uint64_t* src =
                    reinterpret_cast<const uint64_t*>(g.split_ws) + (int64_t)slot_of(gfirst + j, w) * SLOT_U64;
  #pragma unroll
                for (int h = 0; h < 8; ++h) {
                  const uint64_t x = load_coherent(src + slot_word(fm, fn, h));
                  p[2 * h] = __builtin_bit_cast(float, (uint32_t)x);
                  p[2 * h + 1] = __builtin_bit_cast(float, (uint32_t)(x >> 32));
                }
              }
              if (j == 0) v = p;
              else v = v + p;
            }
          }
        }
        return v;
      };
      int64_t m0, n0;
      tile_coords(w, m0, n0);
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
            const f32x16 v = total_of(fm, fn);
  #pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int c = fn * 32 + q * 8;
              if (!full && col0 + c >= N) continue;
              *reinterpret_cast<float4*>(row + c) =
                  make_float4(v[q * 4 + 0], v[q * 4 + 1], v[q * 4 + 2], v[q * 4 + 3]);
            }
          }
        } else {
          _Float16* row = static_cast<_Float16*>(g.C) + m * N + col0;
  #pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            __builtin_amdgcn_sched_barrier(0);  // convert one accumulator block at a time
            const f32x16 tv = total_of(fm, fn);
  #pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int c = fn * 32 + q * 8;
              if (!full && col0 + c >= N) continue;
              uint2 v;
              float x0 = tv[q * 4 + 0], x1 = tv[q * 4 + 1];
              float x2 = tv[q * 4 + 2], x3 = tv[q * 4 + 3];
              asm volatile("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(v.x) : "v"(x0), "v"(x1));
              asm volatile("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(v.y) : "v"(x2), "v"(x3));
              *reinterpret_cast<uint2*>(row + c) = v;
            }
          }
        }
      }
    } while (seg_next(ms));
  };
  main_loop();
  __builtin_amdgcn_s_waitcnt(0);
  if constexpr (GATED) {
    // Inbox guard: every load of the workgroup, its inbox reads among them,
    // has completed (each wave's wait above; then the barrier); count the
    // workgroup out of the inbox (no returned value).
    if (g.consumed != nullptr) {
      __syncthreads();
      if (tid == 0)
        __hip_atomic_fetch_add(g.consumed + guard_counter(blockIdx.x) * kGuardStride, 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

inline bool arrival_requested(const GemmArgs& a) { return a.arrival != 0 && a.gate.flags != nullptr; }

template <int BM, int BN, int BK, int STAGES, int WM, int WN>
hipError_t launch_cfg(const GemmArgs& a, const MfmaPlan& p, bool out_f32, hipStream_t s, const LaunchTiming& t) {
  // Persistent grid of at most one workgroup per CU (the LDS ring admits no
  // second one). Every configuration leaves registers free on each SIMD, so
  // producer workgroups can always run beside spinning consumers.
  if (p.bm != BM || p.bn != BN) return hipErrorInvalidValue;
  const dim3 grid((unsigned)p.grid), block(64 * WM * WN);
  const bool gated = a.gate.flags != nullptr;
  // Arrival order needs a tile to span at least the prologue's steps (the
  // cursor publishes a tile's order at a barrier the prologue does not have).
  const bool arrival = arrival_requested(a) && !p.split && a.K / BK >= STAGES;
  const bool bnt = p.bnt && !arrival;
#define L4(G_, F_, S_, A_)                                                                                     \
  do {                                                                                                        \
    if (t.start)                                                                                              \
      hipExtLaunchKernelGGL((gemm_mfma_kernel<BM, BN, BK, STAGES, WM, WN, G_, F_, S_, A_>), grid, block, 0, s,  \
                            t.start, t.stop, 0, a);                                                           \
    else                                                                                                      \
      hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, BK, STAGES, WM, WN, G_, F_, S_, A_>), grid, block, 0, s, a); \
  } while (0)
#define L(G_, F_, S_) L4(G_, F_, S_, false)
#define L5(G_, F_)                                                                                              \
  do {                                                                                                         \
    if (t.start)                                                                                               \
      hipExtLaunchKernelGGL((gemm_mfma_kernel<BM, BN, BK, STAGES, WM, WN, G_, F_, false, false, true>), grid,  \
                            block, 0, s, t.start, t.stop, 0, a);                                               \
    else                                                                                                       \
      hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, BK, STAGES, WM, WN, G_, F_, false, false, true>), grid,     \
                         block, 0, s, a);                                                                      \
  } while (0)
#define L2(S_)                                                     \
  do {                                                             \
    if (gated) { if (out_f32) L(true, true, S_); else L(true, false, S_); }   \
    else { if (out_f32) L(false, true, S_); else L(false, false, S_); }       \
  } while (0)
  if constexpr (BN == 128) {
    if (bnt) {
      if (gated) { if (out_f32) L5(true, true); else L5(true, false); }
      else { if (out_f32) L5(false, true); else L5(false, false); }
      return hipGetLastError();
    }
  }
  if (arrival) {
    if (out_f32) L4(true, true, false, true);
    else L4(true, false, false, true);
  } else if (p.split) {
    L2(true);
  } else {
    L2(false);
  }
#undef L2
#undef L
#undef L4
#undef L5
  return hipGetLastError();
}

}  // namespace

int mfma_config_count() { return 3; }

// Default tile by M. Consumer alone, whole tiles, K = 8192, N = 28672, us
// on MI355X (the stream-K split of the 256x256 tiles measured 202.6 and
// 206.9 us at M = 224 and 256):
//   M      128x128 (1)  256x128 (2)  256x256 (0)
//   128      98.4         131.6        170.0
//   192     164.5         159.8        181.6
//   224     173.7         164.7        184.2
//   256     178.7         169.4        187.6
//   320     209.8         233.2        210.7
//   512     325.2         310.3        226.8
// One row block of 256 covers M up to 256 and reads each element of B once;
// above that the 256x256 tile moves the fewest bytes per FLOP.
int mfma_config_for(int64_t M, int tile_config) {
  if (tile_config >= 0 && tile_config < mfma_config_count()) return tile_config;
  return M <= 128 ? 1 : M <= 256 ? 2 : 0;
}

// A split must save the busiest workgroup at least this many columns of K
// (see mfma_plan).
constexpr int64_t kMinSplitSavedColumns = 4096;

MfmaPlan mfma_plan(int64_t M, int64_t N, int64_t K, int W, int num_cus, int tile_config, int split_mode) {
  MfmaPlan p;
  p.cfg = mfma_config_for(M, tile_config);
  p.bm = p.cfg == 1 ? 128 : 256;
  p.bn = p.cfg == 0 ? 256 : 128;
  p.tiles = ((M + p.bm - 1) / p.bm) * ((N + p.bn - 1) / p.bn);
  // Busiest workgroup's run, in (tile, shard) units: whole tiles dealt to
  // min(tiles, CUs) workgroups, against equal runs of units over min(units, CUs).
  // Every split tile costs its contributors a BM x BN fp32 partial each
  // (written and read back once); measured on MI355X at K = 8192, N = 28672,
  // that hand-off outweighs a 12.5 % shorter run (224 tiles on 256 CUs: 120
  // against 101 us at M = 128, 333 against 245 us at M = 512). The automatic
  // choice therefore splits only when whole tiles would leave at least half
  // of the CUs idle, where the run shrinks by 2x or more, and only when that
  // saves the busiest workgroup at least kMinSplitSavedColumns columns of K:
  // the hand-off costs a fixed 18-30 us with 128-column tiles and about 95 us
  // with 256x256 tiles. Consumer alone, W = 8 (whole against split, us):
  //   M, N        K = 2048      K = 4096      K = 8192
  //   8, 256      18.2 / 20.0   27.8 / 21.3   46.5 / 23.8
  //   128, 4096   20.3 / 33.0   30.1 / 36.2   50.6 / 42.1
  //   300, 1032   45.5 / 104.8  78.7 / 110.0  144.2 / 119.4
  // (columns saved: 7 x K/8, i.e. 1792, 3584, 7168).
  const int64_t g_tiles = std::min<int64_t>(p.tiles, num_cus);
  const int64_t run_tiles = (p.tiles + g_tiles - 1) / g_tiles * W;
  const int64_t units = p.tiles * W;
  // The split kernels of the 256-row tiles hold (nearly) all of a SIMD's 512
  // registers per wave (their hand-off epilogue), so no producer wave fits on
  // a CU that runs one: their grid leaves an eighth of the CUs free for the
  // producer a gated launch waits for.
  const int64_t split_cus = p.cfg == 1 ? num_cus : std::max<int64_t>(1, num_cus - num_cus / 8);
  const int64_t g_units = std::min<int64_t>(units, split_cus);
  const int64_t run_units = (units + g_units - 1) / g_units;
  const int64_t saved_columns = (run_tiles - run_units) * (K / W);
  if (split_mode < 0)
    p.split = W >= 2 && 2 * p.tiles <= num_cus && 2 * run_units <= run_tiles && saved_columns >= kMinSplitSavedColumns;
  else p.split = split_mode > 0 && W >= 2;
  p.grid = p.split ? g_units : g_tiles;
  // One row block: every element of B is read by one tile only, so its loads
  // skip L2 allocation (M = 128, N = 28672, 224 workgroups: 98.7 against
  // 101.4 us). With more row blocks, tiles of one XCD share B panels through
  // the L2; with few workgroups the nontemporal loads streamed slower (32
  // tiles: 73 against 48 us), so at least half of the CUs must be busy.
  // (Arrival-order launches keep the default policy.)
  p.bnt = p.bn == 128 && M <= p.bm && !p.split && 2 * p.grid >= num_cus;
  if (p.split) {
    p.ws_bytes = sizeof(float) * 2 * (size_t)p.grid * (size_t)(p.bm * p.bn);
    p.cnt_bytes = sizeof(uint32_t) * (size_t)p.tiles;
  }
  return p;
}

// Arrival order runs on whole tiles (a split tile's partial ranges stay in shard order).
static MfmaPlan launch_plan(const GemmArgs& a) {
  return mfma_plan(a.M, a.N, a.K, a.W, a.num_cus, a.tile_config, (a.split && !arrival_requested(a)) ? 1 : 0);
}

int64_t mfma_guard_units(const GemmArgs& a) { return launch_plan(a).grid; }

hipError_t launch_gemm_mfma(const GemmArgs& a, bool out_f32, hipStream_t s, const LaunchTiming& t) {
  MfmaPlan p = launch_plan(a);
  if (p.split && (!a.split_ws || !a.split_cnt)) return hipErrorInvalidValue;
  switch (p.cfg) {
    case 0: return launch_cfg<256, 256, 32, 4, 2, 2>(a, p, out_f32, s, t);   // 4 waves, 128x128 per wave
    case 1: return launch_cfg<128, 128, 64, 4, 2, 2>(a, p, out_f32, s, t);   // 4 waves, 64x64 per wave
    default: return launch_cfg<256, 128, 32, 4, 2, 2>(a, p, out_f32, s, t);  // 4 waves, 128x64 per wave
  }
}

}  // namespace agemm
