// CPU check of the inbox guard's bookkeeping (guard_units.h, compiled as the
// kernels and the host library use it): the totals the host adds for a launch
// of n units equal what the launch's units count into each counter (unit u
// into guard_counter(u)), and totals kept over many launches, started just
// below the 32-bit wrap, stay equal to counters raised one unit at a time.
// PLANT = 1 plants a mistake (the remainder's units go to the last counters)
// that the check must catch.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "guard_units.h"

using namespace agemm;

namespace {

void add_units(uint32_t (&target)[kGuardCounters], int64_t units) {
#if PLANT == 1
  for (int j = 0; j < kGuardCounters; ++j)
    target[j] += (uint32_t)(units / kGuardCounters + (j >= kGuardCounters - units % kGuardCounters ? 1 : 0));
#else
  add_guard_units(target, units);
#endif
}

}  // namespace

int main() {
  std::vector<int64_t> sizes;
  for (int64_t n = 0; n <= 4096; ++n) sizes.push_back(n);
  const int64_t large[] = {448, 1792, 65536, 131072, 1000003, (int64_t)1 << 31};
  for (int64_t n : large) sizes.push_back(n);
  for (int64_t n : sizes) {
    uint32_t target[kGuardCounters] = {};
    add_units(target, n);
    std::vector<uint64_t> hist(kGuardCounters, 0);
    if (n <= 2000000) {
      for (int64_t u = 0; u < n; ++u) hist[guard_counter(u)]++;
    } else {  // closed form for the largest size: every counter takes n / 64
      for (int j = 0; j < kGuardCounters; ++j) hist[j] = (uint64_t)(n / kGuardCounters) + (j < n % kGuardCounters);
    }
    uint64_t sum = 0;
    for (int j = 0; j < kGuardCounters; ++j) {
      sum += target[j];
      if (target[j] != (uint32_t)hist[j]) {
        std::printf("FAIL: %lld units: counter %d total %u, counted %llu\n", (long long)n, j, target[j],
                    (unsigned long long)hist[j]);
        return 1;
      }
    }
    if (n < ((int64_t)1 << 31) && sum != (uint64_t)n) {
      std::printf("FAIL: %lld units: totals sum to %llu\n", (long long)n, (unsigned long long)sum);
      return 1;
    }
  }
  // many launches of changing sizes, from just below the wrap
  const uint32_t base = 4294967293u;
  uint32_t target[kGuardCounters];
  std::vector<uint32_t> counter(kGuardCounters, base);
  for (int j = 0; j < kGuardCounters; ++j) target[j] = base;
  const int64_t launches[] = {448, 32, 256, 224, 1792, 7, 63, 65, 129, 448};
  for (int rep = 0; rep < 50; ++rep)
    for (int64_t n : launches) {
      add_units(target, n);
      for (int64_t u = 0; u < n; ++u) counter[guard_counter(u)] += 1u;
      for (int j = 0; j < kGuardCounters; ++j)
        if (target[j] != counter[j]) {
          std::printf("FAIL: launch of %lld units (round %d): counter %d total %u, counted %u\n", (long long)n, rep,
                      j, target[j], counter[j]);
          return 1;
        }
    }
  std::printf("ok: %zu launch sizes, 500 launches across the wrap\n", sizes.size());
  return 0;
}
