// Inbox guard bookkeeping shared by the kernels and the host library. No HIP
// dependency: a CPU check compiles it as it is.
//
// Per inbox, kGuardCounters counters into which a fused consumer launch counts
// its units (the small-M kernel's items, the MFMA kernel's workgroups) once
// they are done reading the inbox, unit u into counter guard_counter(u). The
// producer of a later epoch on that inbox waits on the device until every
// counter has reached the total of the launches issued on it, which the host
// keeps with add_guard_units. Spreading the counts keeps each address to a few
// dozen atomics per launch, and one counter per 4 KiB spreads the addresses
// over the memory channels (counters on a couple of lines serialised the
// counts and held up the consumer's stream); one wave polls all of them at
// once.
#pragma once

#include <stdint.h>

namespace agemm {

constexpr int kGuardCounters = 64;
constexpr int kGuardStride = 1024;  // uint32 elements from one counter to the next

// The counter unit u counts into.
constexpr int guard_counter(int64_t u) { return (int)(u % kGuardCounters); }

// Adds what a launch of `units` units counts into each counter to the totals
// (wrapping, as the counters do).
inline void add_guard_units(uint32_t (&target)[kGuardCounters], int64_t units) {
  for (int j = 0; j < kGuardCounters; ++j)
    target[j] += (uint32_t)(units / kGuardCounters + (j < units % kGuardCounters ? 1 : 0));
}

}  // namespace agemm
