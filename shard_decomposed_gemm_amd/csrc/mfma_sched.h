// Integer work schedule of the MFMA consumer (gemm_mfma.hip).
//
// Which output tiles and k-steps each workgroup computes, in which order its
// direct loads walk them, where each lane's 16-byte load comes from, and who
// sums a tile that the stream-K split shares between workgroups. The loop
// order follows the AG+GEMM core identity of the "Eliminating Multi-GPU
// Performance Taxes" analysis page: per output tile, shards s = 0..W-1 in
// turn, each shard's k-steps ascending (every k-step of every tile over all
// shards exactly once, as its correctness check #3 asks of the tiled loop).
//
// Plain integer functions with no device-only code, so that the kernel and a
// CPU check (tests/mfma_sched_check.cpp) run exactly the same arithmetic.
#pragma once

#include <stdint.h>

// Always inlined: in the kernel these run on wave-uniform values that must stay
// in scalar registers (a call would put the cursor state in scratch memory).
#if defined(__HIP__)
#define AGEMM_HD __host__ __device__ inline __attribute__((always_inline))
#else
#define AGEMM_HD inline
#endif

namespace agemm {
namespace sched {

// ---------------------------------------------------------------- tile order

// Output tiles of C in BM x BN blocks. With whole tiles and a grid and tile
// count that are multiples of 8, the workgroups (dealt round-robin to the 8
// XCDs) are mapped so that each XCD gets a contiguous range of logical tiles.
struct TileGrid {
  int MB, NB, total;
  bool xcd;
};

AGEMM_HD TileGrid tile_grid(int64_t M, int64_t N, int BM, int BN, int G) {
  TileGrid t;
  t.MB = (int)((M + BM - 1) / BM);
  t.NB = (int)((N + BN - 1) / BN);
  t.total = t.MB * t.NB;
  t.xcd = (t.total % 8 == 0) && (G % 8 == 0);
  return t;
}

// Tile w -> (row block, column block). Logical tiles are ordered in groups of
// 8 row blocks (the last group may be smaller), column-major inside a group,
// so the tiles running together on one XCD share A and B panels in its L2.
// With the split, w is already a logical index (the runs are numbered by XCD).
AGEMM_HD void tile_coords(const TileGrid& tg, bool split, int w, int& mb, int& nb) {
  const int logical = (!split && tg.xcd) ? (w % 8) * (tg.total / 8) + (w / 8) : w;
  constexpr int GM = 8;
  const int group = logical / (GM * tg.NB);
  const int first_m = group * GM;
  const int gsize = (tg.MB - first_m) < GM ? (tg.MB - first_m) : GM;
  const int in_group = logical - group * GM * tg.NB;
  mb = first_m + in_group % gsize;
  nb = in_group / gsize;
}

// ------------------------------------------------------- work of a workgroup

// A workgroup's work as segments: a tile and its k-steps [kb, ke). Without
// the split, tiles b, b + G, b + 2G, ... in full. With it, the units
// [u0, u1) of the workgroup's run (unit = (tile, shard), tile-major; the run
// of run number r is [floor(r*U/G), floor((r+1)*U/G))), cut at tile borders,
// so only the first and last segments can be partial; every segment starts
// and ends at a shard border. Run numbers are assigned so that consecutive
// runs share an XCD (workgroups are dealt round-robin to the 8 XCDs) and work
// on neighbouring tiles.
struct Work {
  int block, G, W, SPS, NS, total;
  bool split;
  int bp;          // run number
  int64_t U, u0, u1;
};

struct Seg {
  int w, kb, ke;
};

AGEMM_HD Work work_of(int block, int G, int total, int W, int SPS, bool split) {
  Work k;
  k.block = block;
  k.G = G;
  k.W = W;
  k.SPS = SPS;
  k.NS = W * SPS;
  k.total = total;
  k.split = split;
  k.bp = (split && G % 8 == 0) ? (block % 8) * (G / 8) + (block / 8) : block;
  k.U = (int64_t)total * W;
  k.u0 = (int64_t)k.bp * k.U / G;
  k.u1 = (int64_t)(k.bp + 1) * k.U / G;
  return k;
}

AGEMM_HD int seg_end(const Work& k, int w) {
  const int64_t e = k.u1 < (int64_t)(w + 1) * k.W ? k.u1 : (int64_t)(w + 1) * k.W;
  return (int)(e - (int64_t)w * k.W) * k.SPS;
}

AGEMM_HD void seg_first(const Work& k, Seg& q) {
  if (k.split) {
    q.w = (int)(k.u0 / k.W);
    q.kb = (int)(k.u0 - (int64_t)q.w * k.W) * k.SPS;
    q.ke = seg_end(k, q.w);
  } else {
    q.w = k.block;
    q.kb = 0;
    q.ke = k.NS;
  }
}

// Advances q to the next segment; false (q unchanged) when there is none.
AGEMM_HD bool seg_next(const Work& k, Seg& q) {
  if (k.split) {
    const int w = q.w + 1;
    if ((int64_t)w * k.W >= k.u1) return false;
    q.w = w;
    q.kb = 0;
    q.ke = seg_end(k, w);
  } else {
    const int w = q.w + k.G;
    if (w >= k.total) return false;
    q.w = w;
  }
  return true;
}

// Split hand-off: the owner of unit u is the largest run r with
// floor(r*U/G) <= u. Each run publishes at most two partials, for its first
// and its last tile, in slots 2r and 2r + 1.
AGEMM_HD int owner(const Work& k, int64_t u) { return (int)(((u + 1) * k.G - 1) / k.U); }
AGEMM_HD int slot_of(const Work& k, int r, int w) {
  const int first_tile = (int)(((int64_t)r * k.U / k.G) / k.W);
  return 2 * r + (first_tile == w ? 0 : 1);
}

// ------------------------------------------------------ the direct-load cursor

// Position of the direct-load cursor inside its segment (shard order). ct is
// the k-step of the tile whose loads are issued next. Moving to the next
// k-step of the same shard is a pointer bump only; everything else happens
// at an "event" step cev (the first k-step of the next shard, where the A
// pointer moves to that shard's buffer, or of the next flag tile, whose gate
// runs while the workgroup still tracks flags) or at the end of the segment.
struct KPos {
  int ct, cev;
  int cs, nshard;   // shard of ct, first k-step of the next shard
  int cft, nflag;   // flag tile of ct (s * KT + kt), first k-step of the next flag tile
};

enum : int { kEvShard = 1, kEvFlag = 2, kEvEnd = 4 };

AGEMM_HD int min3(int a, int b, int c) {
  const int m = a < b ? a : b;
  return m < c ? m : c;
}

// ke: end of the segment; spt: k-steps per flag tile; KT: flag tiles per shard;
// track: the workgroup may still meet a flag it has not seen raised.
AGEMM_HD void kpos_enter(KPos& p, const Seg& q, int SPS, int spt, int KT, bool track) {
  p.ct = q.kb;
  p.cs = q.kb / SPS;
  p.nshard = (p.cs + 1) * SPS;
  p.cft = p.cs * KT;
  p.nflag = q.kb + spt;
  p.cev = min3(q.ke, p.nshard, track ? p.nflag : 0x7fffffff);
}

// One k-step forward; true when the new step is an event step or the end of
// the segment (the caller then handles the end itself, or calls kpos_event).
AGEMM_HD bool kpos_step(KPos& p, int ke) {
  ++p.ct;
  return (p.ct == p.cev) | (p.ct == ke);
}

// At an event step: what happens at this k-step (kEvEnd alone at the end of
// the segment), and the next event step.
AGEMM_HD int kpos_event(KPos& p, int ke, int SPS, int spt, bool track) {
  if (p.ct == ke) return kEvEnd;
  int ev = 0;
  if (p.ct == p.nshard) {
    ++p.cs;
    p.nshard += SPS;
    ev |= kEvShard;
  }
  if (track && p.ct == p.nflag) {
    ++p.cft;
    p.nflag += spt;
    ev |= kEvFlag;
  }
  p.cev = min3(ke, p.nshard, track ? p.nflag : 0x7fffffff);
  return ev;
}

// ------------------------------------------------------------ arrival order

// Arrival order takes an output tile's flag tiles in any order (the core
// identity is a plain sum over shards). The next one is the lowest-numbered
// flag tile seen raised and not yet taken; with none, the lowest untaken one
// (whose gate then waits). Candidates are masked with the T flag tiles, so a
// choice is always a real, untaken tile.
AGEMM_HD uint64_t flag_mask(int T) { return T >= 64 ? ~0ull : ((1ull << T) - 1ull); }
AGEMM_HD int arrival_pick(uint64_t ready, uint64_t taken, uint64_t tmask) {
  uint64_t c = ready & ~taken & tmask;
  if (c == 0) c = ~taken & tmask;
  return __builtin_ctzll(c);
}
// First k-step (of the tile, in BK units) of flag tile f = s * KT + kt.
AGEMM_HD int flag_first_step(int f, int KT, int SPS, int spt) {
  const int fs = f / KT, fk = f - fs * KT;
  return fs * SPS + fk * spt;
}

// ------------------------------------------------------------ lane offsets

// 16-byte chunks are stored in LDS with their index XOR-swizzled so that the
// fragment reads are free of bank conflicts. A rows hold CPR = BK/8 chunks, B
// rows (BN columns) BN/8 chunks.
template <int CPR>
AGEMM_HD int swz_a(int row) {
  return (row / (16 / CPR)) % CPR;
}
AGEMM_HD int swz_b(int k) { return (k & 3) << 2; }

// Chunk q of a stage's A block (BM rows x BK columns): byte offset of its
// source from the tile's first row at the k-step's first column, rows past M
// clamped to the last row (their results are never stored).
template <int BK>
AGEMM_HD uint32_t a_src_offset(int q, int rmax, int64_t lda_bytes) {
  constexpr int CPR = BK / 8;
  int r = q / CPR;
  const int c = (q % CPR) ^ swz_a<CPR>(r);
  r = r < rmax ? r : rmax;
  return (uint32_t)(r * lda_bytes + c * 16);
}

// The same chunk in the k-panel layout (32-column panels of M rows of 64
// bytes, panel_bytes = M * 64 apart): byte offset from the k-step's first
// panel at the tile's first row. BK = 64 spans two panels.
template <int BK>
AGEMM_HD uint32_t a_src_offset_panels(int q, int rmax, int64_t panel_bytes) {
  constexpr int CPR = BK / 8;
  int r = q / CPR;
  const int c = (q % CPR) ^ swz_a<CPR>(r);
  r = r < rmax ? r : rmax;
  return (uint32_t)((c >> 2) * panel_bytes + r * 64 + (c & 3) * 16);
}

// Chunk q of a stage's B block (BK rows x BN columns): byte offset of its
// source from the k-step's first row at the tile's first column, columns past
// N clamped to the last 8 (their results are never stored).
template <int BN>
AGEMM_HD uint32_t b_src_offset(int q, int cmax, int64_t N) {
  constexpr int CPR = BN / 8;
  const int k = q / CPR;
  int c = ((q % CPR) ^ swz_b(k)) * 8;
  c = c < cmax ? c : cmax;
  return (uint32_t)((k * N + c) * 2);
}

}  // namespace sched
}  // namespace agemm
