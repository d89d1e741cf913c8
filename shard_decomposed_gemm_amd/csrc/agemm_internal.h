// Internal interface between the C-ABI host library and the gfx950 kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "guard_units.h"

namespace agemm {

constexpr int kMaxShards = 16;
constexpr int kMaxTiles = 64;   // T = W * KT; one wave polls every flag at once

// Device error word (lives in host-pinned, device-mapped memory).
struct ErrWord {
  uint32_t code;     // 0 = none, 1 = flag wait timed out, 2 = inbox guard wait timed out (producer)
  uint32_t tile;     // tile id (code 1) or guard counter (code 2) that timed out
  uint32_t target;   // value waited for
  uint32_t seen;     // last value observed
};

// Inbox guard: counters, their spacing and the host's totals (guard_units.h).

// Columns of one k-panel of the inbox layout (see ASource).
constexpr int kPanelK = 32;

// Where the GEMM reads its A operand for shard s. Row-major (panels == 0):
// element (m, j) at base[s] + m * lda + j. K-panels (panels == 1): the shard
// is cut into panels of kPanelK columns, each stored as M rows of kPanelK
// contiguous elements, one panel after the other: element (m, j) at
// base[s] + ((j / kPanelK) * M + m) * kPanelK + j % kPanelK. A tile's k-step
// then reads whole contiguous rows of 64 bytes that sit next to each other,
// instead of 64-byte pieces one row apart; the producer and the gather copy
// write this layout into the inbox and the BSP buffer.
struct ASource {
  const _Float16* base[kMaxShards];
  int64_t lda;
  int32_t panels;
};

// The k-panel layout addresses a flag tile's panels with 32-bit byte offsets
// (buffer stores and lane offsets): it is used when BKf / kPanelK panels of
// M rows stay below 2^31 bytes.
inline bool panel_layout_fits(int64_t M, int64_t bkf) {
  return bkf % kPanelK == 0 && (bkf / kPanelK) * M * (kPanelK * 2) < (int64_t{1} << 31);
}

// Flag gate of the consumer. flags == nullptr disables gating.
struct Gate {
  const uint32_t* flags;
  uint32_t target;          // epoch * contributors per tile (wrapping)
  int32_t kt;               // KT
  int32_t t;                // T
  uint64_t timeout_ticks;   // wall-clock ticks (100 MHz on gfx950)
  int32_t strict;           // 1: agent-scope acquire fence after each flag wait
  ErrWord* err;
};

struct GemmArgs {
  ASource a;
  const _Float16* B;  // K x N row-major
  void* C;            // M x N row-major, fp16 or fp32
  int64_t M, N, K, KS;
  int32_t W;
  int32_t num_cus;    // compute units of the device (persistent grid size)
  int32_t tile_config;  // MFMA tile configuration, -1 = chosen from the shape
  Gate gate;
  // Stream-K split of the MFMA consumer (split != 0): the grid's workgroups
  // take equal runs of (output tile, shard) units in tile-major order; a tile
  // whose units fall to several workgroups is summed by the last of them to
  // finish, in contributor order, from partials the others publish.
  int32_t split;
  float* split_ws;      // 2 * grid slots of BM x BN fp32 partials
  uint32_t* split_cnt;  // one ticket counter per output tile, zero between calls
  // Gated launches only: 1 = take each output tile's flag tiles in arrival
  // order (raised ones first), 0 = shard order.
  int32_t arrival;
  // Gated launches with the inbox guard: the inbox's kGuardCounters counters
  // (kGuardStride apart) this launch counts its units into (nullptr: none).
  uint32_t* consumed;
};

// Default flag k-tile BKf for shard width KS and W shards: min(256, KS),
// widened to the next multiple of 64 dividing KS until T = W * KS / BKf <= 64;
// 0 if there is none. (The kernels also use it as a tiling of K when ungated.)
inline int64_t default_flag_ktile(int64_t KS, int W) {
  int64_t bkf = KS < 256 ? KS : 256;
  while ((KS / bkf) * W > kMaxTiles) {
    int64_t next = bkf + 64;
    while (next <= KS && KS % next) next += 64;
    if (next > KS) return 0;
    bkf = next;
  }
  return bkf;
}

// Launch plan of the MFMA consumer for a shape, fixed when a context is
// created: tile configuration, grid, and whether the stream-K split is used.
struct MfmaPlan {
  int cfg = 0;
  int64_t bm = 0, bn = 0;
  int64_t tiles = 0;     // output tiles
  int64_t grid = 0;      // workgroups of the persistent grid
  bool split = false;
  bool bnt = false;      // B's direct loads nontemporal (one row block, whole tiles, shard order)
  size_t ws_bytes = 0;   // split partial slots
  size_t cnt_bytes = 0;  // split counters
};

// Producer: copies item (position p in release order, row chunk q) from A_s to
// dst and optionally raises the tile's flag. The release schedule travels in
// the kernel arguments (T <= 64 entries), so a call needs no allocation.
struct ProduceArgs {
  const _Float16* src[kMaxShards];  // A_s, M x KS
  _Float16* dst;                    // inbox base or gathered A
  int32_t panels;                   // 1: dst in the k-panel layout of ASource (dst_ld unused)
  int64_t dst_shard_stride;         // elements between shard slots (inbox, panels: M*KS; row-major gather: KS)
  int64_t dst_ld;                   // row stride of a row-major dst (inbox: KS; gather: K)
  uint32_t* flags;                  // nullptr in gather mode
  uint64_t* t0;                     // device, 2 words: common start time per launch parity
  uint32_t parity;
  int32_t has_delay;                // 0: release as soon as copied
  int64_t M, KS;
  int32_t bkf, kt, t;
  int32_t rows_per_item;            // rows copied by one workgroup
  int32_t items_per_tile;           // = ceil(M / rows_per_item), contributors per flag
  int32_t order[kMaxTiles];         // tile released p-th
  uint32_t offset_ticks[kMaxTiles]; // its release time after the launch's start, wall-clock ticks
  // Inbox guard (push only; nullptr: none): before its first copy every
  // workgroup waits until counter j of `consumed` has reached guard_target[j]
  // (wrap-aware), the units that the fused launches issued on the inbox
  // count into it.
  const uint32_t* consumed;
  uint32_t guard_target[kGuardCounters];
  uint32_t* go;                     // the inbox's word: workgroup 0 sets it to go_seq once the guard holds
  uint32_t go_seq;                  // producer launches on this inbox so far, this one included (wrapping)
  uint64_t timeout_ticks;           // bound of the guard wait
  ErrWord* err;
};

// Work split of the small-M path, chosen on the host for the device's CU
// count: items are (K-range, column block), a K-range being `ranges`-th of the
// shards and a column block 8 * lanes columns.
struct SmallMPlan {
  int32_t lanes = 0;   // active lanes per streaming wave (8 columns each)
  int32_t ranges = 0;  // K-ranges (divides W)
  int32_t nblk = 0;    // column blocks
  int32_t wg_per_cu = 1;  // cap of the persistent grid, in workgroups per CU
  bool ok = false;     // the small-M kernel takes this shape
};

// Split-K workspace for the small-M path (one partial per K-range).
struct SmallMArgs {
  GemmArgs g;
  SmallMPlan plan;
  float* ws;          // ranges x M x N partial sums
  uint32_t* counters; // one per column block, zero between calls
};
// Units a small-M launch counts into the inbox guard: one per item.
inline int64_t small_m_guard_units(const SmallMPlan& p) { return (int64_t)p.ranges * p.nblk; }
// Units an MFMA launch counts into the inbox guard: one per workgroup of the
// grid launch_gemm_mfma uses for these arguments.
int64_t mfma_guard_units(const GemmArgs& a);


// Optional HIP events attached to a consumer kernel's dispatch (its own start
// and end timestamps); null = plain launch.
struct LaunchTiming {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// max_workgroups > 0: a persistent grid of at most that many workgroups walks
// the items in release order; 0: one workgroup per item.
hipError_t launch_produce(const ProduceArgs& a, int max_workgroups, hipStream_t s);
hipError_t launch_gemm_mfma(const GemmArgs& a, bool out_f32, hipStream_t s, const LaunchTiming& t = {});
int mfma_config_count();
int mfma_config_for(int64_t M, int tile_config);  // configuration launch_gemm_mfma uses
// split_mode: -1 = split when it shortens the busiest workgroup's run enough, 0 = never, 1 = whenever W >= 2.
MfmaPlan mfma_plan(int64_t M, int64_t N, int64_t K, int W, int num_cus, int tile_config, int split_mode);
hipError_t launch_gemm_small_m(const SmallMArgs& a, bool out_f32, hipStream_t s, const LaunchTiming& t = {});
// Overlap probe (probes.hip): times[0..1] = start, end of a kernel that sleeps
// `ticks` on `first`; times[2] = start of a kernel launched after it on `second`.
hipError_t launch_overlap_probe(hipStream_t first, hipStream_t second, uint64_t* times, uint64_t ticks);
int small_m_limit();         // largest M the small-M kernel takes
int small_m_default_max();   // largest M for which it is the default consumer
SmallMPlan small_m_plan(int W, int64_t M, int64_t KS, int64_t N, int num_cus);
// The plan for given lanes / ranges / workgroups per CU, if the kernel takes it.
SmallMPlan small_m_plan_with(int W, int64_t M, int64_t KS, int64_t N, int lanes, int ranges, int wg_per_cu);

}  // namespace agemm
