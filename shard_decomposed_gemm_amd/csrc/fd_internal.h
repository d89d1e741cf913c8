// Internal interface between the Flash-Decode combine's C-ABI host code
// (fdc.cpp) and its gfx950 kernels (fd_combine.hip).
#pragma once

#include "agemm_internal.h"

namespace agemm {

// Flash-Decode combine (fdcombine.h). Inbox(s) holds T/W blocks, one per head
// tile j, each `blk` bytes: the HT x D binary32 outputs of heads
// [j*HT, (j+1)*HT) of rank s, then their HT statistics, padded to a whole
// 128-byte line so that no cache line holds data of two tiles (a line read
// after one tile's flag never carries a stale copy of another tile's data).
struct FdLayout {
  int32_t W, H, D, HT, nht;  // nht = H / HT
  int64_t blk;               // bytes per (rank, head tile) block
};

struct FdProduceArgs {
  FdLayout L;
  const float* o_src[kMaxShards];    // H x D per rank
  const float* lse_src[kMaxShards];  // H per rank
  char* dst;                         // inbox (flags) or gather buffer
  uint32_t* flags;                   // nullptr in gather mode
  uint64_t* t0;                      // 2 words: common start time per launch parity
  uint32_t parity;
  int32_t has_delay;
  int32_t order[kMaxTiles];          // tile released p-th
  uint32_t offset_ticks[kMaxTiles];  // its release time after the launch's start
  // Inbox guard (push only): before writing, every workgroup waits until
  // *consumed has reached consumed_target, the count of head waves of every
  // fused combine issued on this inbox so far (each counts itself in once it
  // has read its last block). Bounded by timeout_ticks; a timeout is
  // recorded in *err with code 2.
  const uint32_t* consumed;
  uint32_t consumed_target;
  uint64_t timeout_ticks;
  ErrWord* err;
};

struct FdCombineArgs {
  FdLayout L;
  const char* src;         // inbox or gather buffer (block layout above)
  void* O;                 // H x D, binary16 or binary32
  const uint32_t* flags;   // nullptr: no gate, ranks in ascending order
  uint32_t target;         // flag value that means "this epoch's tile is in"
  uint64_t timeout_ticks;  // wall-clock ticks
  ErrWord* err;
  uint32_t* consumed;      // gated: the inbox's consumed count, +1 per head wave when it is done reading
};

hipError_t launch_fd_produce(const FdProduceArgs& a, hipStream_t s);
hipError_t launch_fd_combine(const FdCombineArgs& a, bool out_f32, hipStream_t s, const LaunchTiming& t = {});

}  // namespace agemm
