// Host-side pieces shared by the GEMM and Flash-Decode combine contexts.
#include "host_common.h"

#include <cerrno>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>

namespace agemm {

namespace {
const char* kStatusNames[] = {"AGEMM_OK",  "AGEMM_EINVAL",   "AGEMM_ESHAPE", "AGEMM_ENOMEM",
                              "AGEMM_EHIP", "AGEMM_ETIMEOUT", "AGEMM_ESTATE"};
}  // namespace

int epoch_base_from_env(uint32_t* base) {
  const char* env = std::getenv("AGEMM_EPOCH_BASE");
  if (!env) return 0;
  char* end = nullptr;
  errno = 0;
  const unsigned long long v = std::strtoull(env, &end, 0);
  if (!*env || *end || errno || v > 0xffffffffull || env[0] == '-') return -1;
  *base = (uint32_t)v;
  return 1;
}

const char* status_name(int code) {
  if (code < 0 || code > AGEMM_ESTATE) return "AGEMM_UNKNOWN";
  return kStatusNames[code];
}

int set_error(std::string* last, int code, const char* fmt, ...) {
  if (last) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    *last = std::string(status_name(code)) + ": " + buf;
  }
  return code;
}

int set_hip_error(std::string* last, hipError_t e, const char* what) {
  return set_error(last, AGEMM_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int parse_schedule(const agemm_schedule* sched, int T, double ticks_per_ns, int32_t* order, uint32_t* offset_ticks,
                   int32_t* has_delay, std::string* last) {
  *has_delay = 0;
  for (int p = 0; p < T; ++p) {
    order[p] = p;
    offset_ticks[p] = 0;
  }
  if (!sched) return AGEMM_OK;
  if (sched->n != T || !sched->order || !sched->offset_ns)
    return set_error(last, AGEMM_EINVAL, "schedule must have n == T (%d) entries and non-NULL arrays", T);
  bool seen[kMaxTiles] = {};
  int64_t prev = 0;
  for (int p = 0; p < T; ++p) {
    const int32_t tile = sched->order[p];
    if (tile < 0 || tile >= T || seen[tile]) return set_error(last, AGEMM_EINVAL, "schedule order is not a permutation");
    seen[tile] = true;
    const int64_t off = sched->offset_ns[p];
    if (off < 0 || off < prev)
      return set_error(last, AGEMM_EINVAL, "schedule offsets must be non-negative and non-decreasing");
    const double ticks = (double)off * ticks_per_ns;
    if (ticks > 1.0e9) return set_error(last, AGEMM_EINVAL, "schedule offset %lld ns is over 10 s", (long long)off);
    prev = off;
    order[p] = tile;
    offset_ticks[p] = (uint32_t)(ticks + 0.5);
    if (offset_ticks[p]) *has_delay = 1;
  }
  return AGEMM_OK;
}

int find_stream_pair(hipStream_t pair[2], uint64_t* probe_times, double ticks_per_ns, std::string* last) {
  std::vector<hipStream_t> spare;
  const uint64_t ticks = (uint64_t)(100000.0 * ticks_per_ns);
  hipError_t e = hipSuccess;
  for (int attempt = 0; attempt < 8 && e == hipSuccess && !pair[0]; ++attempt) {
    hipStream_t p = nullptr, q = nullptr;
    e = hipStreamCreateWithFlags(&p, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&q, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipMemset(probe_times, 0, 3 * sizeof(uint64_t));
    if (e == hipSuccess) e = launch_overlap_probe(p, q, probe_times, ticks);
    uint64_t t[3] = {0, 0, 0};
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpy(t, probe_times, sizeof t, hipMemcpyDeviceToHost);
    if (e == hipSuccess && t[2] != 0 && t[2] < t[1]) {
      pair[0] = p;
      pair[1] = q;
    } else {
      if (p) spare.push_back(p);
      if (q) spare.push_back(q);
    }
  }
  for (hipStream_t x : spare) (void)hipStreamDestroy(x);
  if (e != hipSuccess) return set_hip_error(last, e, "stream pair probe");
  if (!pair[0]) return set_error(last, AGEMM_EHIP, "no pair of streams ran concurrently in 8 attempts");
  return AGEMM_OK;
}

hipError_t StreamOrder::create() {
  hipError_t e = hipEventCreateWithFlags(&ev_producer, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&ev_consumer, hipEventDisableTiming);
  for (int i = 0; i < 2 && e == hipSuccess; ++i) e = hipEventCreateWithFlags(&ev_fused[i], hipEventDisableTiming);
  return e;
}

void StreamOrder::destroy() {
  if (ev_producer) (void)hipEventDestroy(ev_producer);
  if (ev_consumer) (void)hipEventDestroy(ev_consumer);
  for (int i = 0; i < 2; ++i)
    if (ev_fused[i]) (void)hipEventDestroy(ev_fused[i]);
  ev_producer = ev_consumer = ev_fused[0] = ev_fused[1] = nullptr;
}

// Makes s wait for the last call marked on `from` (recording its event now if
// that was put off).
hipError_t StreamOrder::wait_for(hipEvent_t ev, hipStream_t from, bool pending, bool* recorded, hipStream_t s) {
  if (!pending || from == s) return hipSuccess;
  if (!*recorded) {
    const hipError_t e = hipEventRecord(ev, from);
    if (e != hipSuccess) return e;
    *recorded = true;
  }
  return hipStreamWaitEvent(s, ev, 0);
}

// Marks a call made on s: records its event now, or puts the record off.
hipError_t StreamOrder::mark(hipEvent_t ev, hipStream_t s, bool lazy, hipStream_t* stream, bool* pending,
                             bool* recorded) {
  if (!lazy) {
    const hipError_t e = hipEventRecord(ev, s);
    if (e != hipSuccess) return e;
  }
  *stream = s;
  *pending = true;
  *recorded = !lazy;
  return hipSuccess;
}

hipError_t StreamOrder::before_produce(hipStream_t s, int slot) {
  hipError_t e = hipSuccess;
  if (slot >= 0 && fused_pending[slot] && fused_stream[slot] != s) e = hipStreamWaitEvent(s, ev_fused[slot], 0);
  if (e == hipSuccess) e = wait_for(ev_producer, producer_stream, producer_pending, &producer_recorded, s);
  return e;
}

hipError_t StreamOrder::after_fused(int slot, hipStream_t s) {
  const hipError_t e = hipEventRecord(ev_fused[slot], s);
  if (e == hipSuccess) {
    fused_pending[slot] = true;
    fused_stream[slot] = s;
  }
  return e;
}

hipError_t StreamOrder::after_produce(hipStream_t s) {
  return mark(ev_producer, s, is_owned(s), &producer_stream, &producer_pending, &producer_recorded);
}

hipError_t StreamOrder::before_consumer(hipStream_t s) {
  return wait_for(ev_consumer, consumer_stream, consumer_pending, &consumer_recorded, s);
}

hipError_t StreamOrder::after_consumer(hipStream_t s) {
  return mark(ev_consumer, s, is_owned(s), &consumer_stream, &consumer_pending, &consumer_recorded);
}

int KernelTimer::begin(int32_t max_launches, std::string* last) {
  if (max_launches < 1 || max_launches > 100000)
    return set_error(last, AGEMM_EINVAL, "max_launches must be in 1..100000");
  if (on) return set_error(last, AGEMM_ESTATE, "timing already active");
  while ((int32_t)events.size() < 2 * max_launches) {
    hipEvent_t ev = nullptr;
    const hipError_t e = hipEventCreate(&ev);
    if (e != hipSuccess) return set_hip_error(last, e, "hipEventCreate");
    events.push_back(ev);
  }
  cap = max_launches;
  count = 0;
  on = true;
  return AGEMM_OK;
}

LaunchTiming KernelTimer::next() {
  LaunchTiming t;
  if (on && count < cap) {
    t.start = events[2 * count];
    t.stop = events[2 * count + 1];
    count++;
  }
  return t;
}

int KernelTimer::end(float* us, int32_t max, int32_t* out_count, std::string* last) {
  if (!on) return set_error(last, AGEMM_ESTATE, "timing not active");
  on = false;
  if (out_count) *out_count = count;
  for (int32_t i = 0; i < count; ++i) {
    hipError_t e = hipEventSynchronize(events[2 * i + 1]);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, events[2 * i], events[2 * i + 1]);
    if (e != hipSuccess) return set_hip_error(last, e, "kernel timing events");
    if (us && i < max) us[i] = ms * 1000.f;
  }
  return AGEMM_OK;
}

void KernelTimer::destroy() {
  for (hipEvent_t e : events) (void)hipEventDestroy(e);
  events.clear();
  cap = count = 0;
  on = false;
}

}  // namespace agemm
