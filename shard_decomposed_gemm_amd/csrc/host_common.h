// Host-side pieces shared by the two C-ABI contexts (agemm.cpp for the
// shard-decomposed GEMM, fdc.cpp for the Flash-Decode combine): status text,
// argument checks, the producer's release schedule, stream ordering between
// calls of one context, and kernel timing with events attached to dispatches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "agemm.h"
#include "agemm_internal.h"

namespace agemm {

// "AGEMM_xxx: message" into *last; returns code.
int set_error(std::string* last, int code, const char* fmt, ...) __attribute__((format(printf, 3, 4)));
int set_hip_error(std::string* last, hipError_t e, const char* what);
const char* status_name(int code);

inline bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Testing hook: when AGEMM_EPOCH_BASE is set, a new context starts both
// inboxes' epoch counts at its value (and sets its flags and counts to
// match), so that a few calls take the 32-bit counters across their wrap.
// Returns 1 and sets *base when it is set to a number in 0..2^32-1, 0 when it
// is unset, -1 when it holds anything else (the context is then refused).
int epoch_base_from_env(uint32_t* base);

// Validates a release schedule for T tiles and converts it for the producer:
// order[p] = tile released p-th, offset_ticks[p] = its release time in
// wall-clock ticks, *has_delay = any offset non-zero. sched == NULL is tile
// order with no delay.
int parse_schedule(const agemm_schedule* sched, int T, double ticks_per_ns, int32_t* order, uint32_t* offset_ticks,
                   int32_t* has_delay, std::string* last);

// Ordering between the calls of one context on different streams. Every
// producer comes after the previous producer, and every consumer call after
// the previous consumer call of the context, of any kind (they share
// workspaces). The inbox guard holds a producer on the device until the
// fused consumers that read its inbox before are done with it; a context may
// also order the producer after the last fused consumer of its inbox with a
// stream dependency (`after_fused` records that consumer's event at once,
// `before_produce` waits for it), so that the producer is not dispatched, and
// does not sit waiting on the CUs, while that consumer runs. A wait is
// skipped when the earlier call ran on the waiting stream (in-stream order
// already holds, and every dependency packet costs command-processor time
// between kernels).
//
// Events of calls on the context's own streams (`owned`, the verified pair)
// are recorded lazily: only when a call on another stream has to wait for
// them, and then on the stream the call ran on, marking everything queued
// there so far (the call and possibly later work: a wait on it is at worst
// longer, never shorter). A record after every call cost the stream about
// 3 us of command-processor time per call (M = 1: 79.3 against 75.9 us per
// fused step). Caller streams, whose lifetime the context does not know, get
// their events when the call is made.
struct StreamOrder {
  hipEvent_t ev_producer = nullptr, ev_consumer = nullptr;
  hipStream_t producer_stream = nullptr, consumer_stream = nullptr;
  bool producer_pending = false, consumer_pending = false;
  bool producer_recorded = true, consumer_recorded = true;
  hipEvent_t ev_fused[2] = {nullptr, nullptr};  // last fused consumer of each inbox (after_fused)
  hipStream_t fused_stream[2] = {nullptr, nullptr};
  bool fused_pending[2] = {false, false};
  hipStream_t owned[2] = {nullptr, nullptr};

  hipError_t create();
  void destroy();
  // After the previous producer; with slot >= 0 also after the last fused
  // consumer of that inbox marked with after_fused.
  hipError_t before_produce(hipStream_t s, int slot = -1);
  hipError_t after_produce(hipStream_t s);
  hipError_t before_consumer(hipStream_t s);
  hipError_t after_consumer(hipStream_t s);
  // Records the event of a fused consumer of inbox `slot` on s at once (for a
  // later before_produce of that inbox).
  hipError_t after_fused(int slot, hipStream_t s);

 private:
  bool is_owned(hipStream_t s) const { return s != nullptr && (s == owned[0] || s == owned[1]); }
  static hipError_t wait_for(hipEvent_t ev, hipStream_t from, bool pending, bool* recorded, hipStream_t s);
  static hipError_t mark(hipEvent_t ev, hipStream_t s, bool lazy, hipStream_t* stream, bool* pending, bool* recorded);
};

// A producer and a consumer stream on which kernels run concurrently: pairs
// of new non-blocking, default-priority streams are probed (a kernel that
// sleeps 100 us on the first, then one on the second that records its start)
// and the first pair whose second kernel started while the first still ran is
// kept in pair[0..1]. probe_times: 3 device words. Synchronises the device.
int find_stream_pair(hipStream_t pair[2], uint64_t* probe_times, double ticks_per_ns, std::string* last);

// Events attached to the dispatch of each consumer kernel launched while
// active (its own start and end stamps), up to cap launches.
struct KernelTimer {
  std::vector<hipEvent_t> events;  // start, stop pairs
  int32_t cap = 0, count = 0;
  bool on = false;

  int begin(int32_t max_launches, std::string* last);
  LaunchTiming next();
  int end(float* us, int32_t max, int32_t* out_count, std::string* last);
  void destroy();
};

}  // namespace agemm
