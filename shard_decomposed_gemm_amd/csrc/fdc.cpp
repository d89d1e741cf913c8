// C-ABI of the flag-gated Flash-Decode combine (declared in include/fdcombine.h).
//
// Host side only: validation, the context (two inboxes and their flags, the
// gather buffer, the error word), stream ordering between epochs, kernel
// timing. Every step of the arithmetic runs in fd_combine.hip.
#include "fdcombine.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "fd_internal.h"
#include "host_common.h"

using namespace agemm;

struct fdc_ctx {
  FdLayout L{};
  int32_t t = 0;  // W * nht
  agemm_dtype out_dtype = AGEMM_F16;
  int device = 0;
  double ticks_per_ns = 0.1;
  uint64_t timeout_ticks = 0;

  char* inbox[2] = {nullptr, nullptr};  // one allocation, W * nht blocks each
  char* gathered = nullptr;             // baseline's gather buffer, same layout
  uint32_t* ctrl = nullptr;             // flags[2][64] | t0 fused[2] | t0 bsp[2] | probe[3] | consumed[2]
  uint32_t* flags[2] = {nullptr, nullptr};
  // Per inbox: head waves of its fused combines that are done reading it
  // (device), and the combines issued on it so far (host). A producer of an
  // inbox waits on the device for H x issued.
  uint32_t* consumed[2] = {nullptr, nullptr};
  uint32_t fused_issued[2] = {0, 0};
  uint64_t* t0_fused = nullptr;
  uint64_t* t0_bsp = nullptr;
  ErrWord* err_host = nullptr;
  ErrWord* err_dev = nullptr;

  uint32_t epoch = 0;                 // produce calls so far; epoch e uses inbox e & 1
  uint32_t slot_epochs[2] = {0, 0};  // produce calls per inbox
  uint32_t parity_fused = 0, parity_bsp = 0;

  hipStream_t pair[2] = {nullptr, nullptr};  // fdc_streams: producer, consumer (owned)
  uint64_t* probe_times = nullptr;           // 3 words in ctrl for the overlap probe
  StreamOrder so;     // ordering between calls on different streams
  KernelTimer timer;  // fdc_timing_begin/end

  std::string last_error;
};

namespace {

int fail(fdc_ctx* c, int code, const char* fmt, ...) __attribute__((format(printf, 3, 4)));
int fail(fdc_ctx* c, int code, const char* fmt, ...) {
  if (c) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    set_error(&c->last_error, code, "%s", buf);
  }
  return code;
}

int hip_fail(fdc_ctx* c, hipError_t e, const char* what) { return set_hip_error(&c->last_error, e, what); }

int check_parts(fdc_ctx* c, const void* const* o_parts, const void* const* lse_parts) {
  if (!o_parts || !lse_parts) return fail(c, AGEMM_EINVAL, "o_parts and lse_parts must be non-NULL");
  for (int s = 0; s < c->L.W; ++s)
    if (!aligned16(o_parts[s]) || !aligned16(lse_parts[s]))
      return fail(c, AGEMM_EINVAL, "partial %d: NULL or not 16-byte aligned", s);
  return AGEMM_OK;
}

int fill_schedule(fdc_ctx* c, const agemm_schedule* sched, FdProduceArgs& pa) {
  return parse_schedule(sched, c->t, c->ticks_per_ns, pa.order, pa.offset_ticks, &pa.has_delay, &c->last_error);
}

void base_args(fdc_ctx* c, const void* const* o_parts, const void* const* lse_parts, FdProduceArgs& pa) {
  pa.L = c->L;
  for (int s = 0; s < kMaxShards; ++s) {
    pa.o_src[s] = s < c->L.W ? static_cast<const float*>(o_parts[s]) : nullptr;
    pa.lse_src[s] = s < c->L.W ? static_cast<const float*>(lse_parts[s]) : nullptr;
  }
}

int launch_combine(fdc_ctx* c, const char* src, const uint32_t* flags, uint32_t target, uint32_t* consumed, void* O,
                   hipStream_t s) {
  FdCombineArgs a{};
  a.L = c->L;
  a.src = src;
  a.O = O;
  a.flags = flags;
  a.target = target;
  a.consumed = consumed;
  a.timeout_ticks = c->timeout_ticks;
  a.err = c->err_dev;
  const hipError_t e = launch_fd_combine(a, c->out_dtype == AGEMM_F32, s, c->timer.next());
  if (e != hipSuccess) return hip_fail(c, e, "combine launch");
  return AGEMM_OK;
}

void free_all(fdc_ctx* c) {
  c->timer.destroy();
  if (c->inbox[0]) (void)hipFree(c->inbox[0]);
  if (c->gathered) (void)hipFree(c->gathered);
  if (c->ctrl) (void)hipFree(c->ctrl);
  if (c->err_host) (void)hipHostFree(c->err_host);
  c->so.destroy();
  for (int i = 0; i < 2; ++i)
    if (c->pair[i]) (void)hipStreamDestroy(c->pair[i]);
}

}  // namespace

extern "C" {

int fdc_create(fdc_ctx** out, int W, int H, int D, int heads_per_tile, agemm_dtype out_dtype) {
  if (!out) return AGEMM_EINVAL;
  *out = nullptr;
  if (out_dtype != AGEMM_F16 && out_dtype != AGEMM_F32) return AGEMM_EINVAL;
  uint32_t base = 0;
  const int has_base = epoch_base_from_env(&base);
  if (has_base < 0) return AGEMM_EINVAL;
  const int HT = heads_per_tile;
  if (W < 1 || W > kMaxShards || H < 1 || (D != 64 && D != 128 && D != 256)) return AGEMM_ESHAPE;
  if (HT < 4 || HT > 32 || HT % 4 || H % HT) return AGEMM_ESHAPE;
  const int nht = H / HT;
  if ((int64_t)W * nht > kMaxTiles) return AGEMM_ESHAPE;

  fdc_ctx* c = new (std::nothrow) fdc_ctx();
  if (!c) return AGEMM_ENOMEM;
  c->L.W = W;
  c->L.H = H;
  c->L.D = D;
  c->L.HT = HT;
  c->L.nht = nht;
  c->L.blk = (int64_t)HT * D * 4 + 128;  // outputs, then the statistics in a line of their own
  c->t = W * nht;
  c->out_dtype = out_dtype;

  hipError_t e = hipGetDevice(&c->device);
  int wall_khz = 0;
  if (e == hipSuccess) e = hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, c->device);
  if (e != hipSuccess || wall_khz <= 0) {
    delete c;
    return AGEMM_EHIP;
  }
  c->ticks_per_ns = (double)wall_khz / 1.0e6;
  c->timeout_ticks = (uint64_t)(2.0e9 * c->ticks_per_ns);  // 2 s

  const size_t inbox_bytes = (size_t)c->t * (size_t)c->L.blk;
  // flags, then 8 words: t0 fused[2], t0 bsp[2], probe times[3], consumed[2] (two u32)
  const size_t ctrl_bytes = sizeof(uint32_t) * 2 * kMaxTiles + 8 * sizeof(uint64_t);
  bool ok = hipMalloc(&c->inbox[0], 2 * inbox_bytes) == hipSuccess;
  ok = ok && hipMalloc(&c->gathered, inbox_bytes) == hipSuccess;
  ok = ok && hipMalloc(&c->ctrl, ctrl_bytes) == hipSuccess;
  if (!ok) {
    free_all(c);
    delete c;
    return AGEMM_ENOMEM;
  }
  c->inbox[1] = c->inbox[0] + inbox_bytes;
  c->flags[0] = c->ctrl;
  c->flags[1] = c->ctrl + kMaxTiles;
  c->t0_fused = reinterpret_cast<uint64_t*>(c->ctrl + 2 * kMaxTiles);
  c->t0_bsp = c->t0_fused + 2;
  c->probe_times = c->t0_bsp + 2;
  c->consumed[0] = reinterpret_cast<uint32_t*>(c->probe_times + 3);
  c->consumed[1] = c->consumed[0] + 1;
  void* hp = nullptr;
  e = hipMemset(c->ctrl, 0, ctrl_bytes);
  if (e == hipSuccess) e = hipHostMalloc(&hp, sizeof(ErrWord), hipHostMallocMapped | hipHostMallocCoherent);
  if (e == hipSuccess) {
    c->err_host = static_cast<ErrWord*>(hp);
    std::memset(c->err_host, 0, sizeof(ErrWord));
    void* dp = nullptr;
    e = hipHostGetDevicePointer(&dp, hp, 0);
    c->err_dev = static_cast<ErrWord*>(dp);
  }
  if (e == hipSuccess && has_base > 0) {
    // every produce on an inbox adds one to each of its flags; every fused
    // combine on it adds H to its consumed count
    c->slot_epochs[0] = c->slot_epochs[1] = base;
    c->fused_issued[0] = c->fused_issued[1] = base;
    const std::vector<uint32_t> init(2 * kMaxTiles, base);
    e = hipMemcpy(c->ctrl, init.data(), init.size() * sizeof(uint32_t), hipMemcpyHostToDevice);
    const uint32_t counts[2] = {base * (uint32_t)c->L.H, base * (uint32_t)c->L.H};
    if (e == hipSuccess) e = hipMemcpy(c->consumed[0], counts, sizeof counts, hipMemcpyHostToDevice);
  }
  if (e == hipSuccess) e = c->so.create();
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    free_all(c);
    delete c;
    return AGEMM_EHIP;
  }
  *out = c;
  return AGEMM_OK;
}

int fdc_destroy(fdc_ctx* ctx) {
  if (!ctx) return AGEMM_OK;
  (void)hipSetDevice(ctx->device);
  (void)hipDeviceSynchronize();
  free_all(ctx);
  delete ctx;
  return AGEMM_OK;
}

int fdc_tiles(const fdc_ctx* ctx, int32_t* t) {
  if (!ctx) return AGEMM_EINVAL;
  if (t) *t = ctx->t;
  return AGEMM_OK;
}

int fdc_streams(fdc_ctx* ctx, void** producer, void** consumer) {
  if (!ctx || !producer || !consumer) return AGEMM_EINVAL;
  if (!ctx->pair[0]) {
    const int rc = find_stream_pair(ctx->pair, ctx->probe_times, ctx->ticks_per_ns, &ctx->last_error);
    if (rc) return rc;
    ctx->so.owned[0] = ctx->pair[0];  // the context's own streams: their events are recorded lazily
    ctx->so.owned[1] = ctx->pair[1];
  }
  *producer = ctx->pair[0];
  *consumer = ctx->pair[1];
  return AGEMM_OK;
}

int fdc_set_spin_timeout_us(fdc_ctx* ctx, int64_t us) {
  if (!ctx) return AGEMM_EINVAL;
  if (us < 1) return fail(ctx, AGEMM_EINVAL, "timeout must be positive");
  ctx->timeout_ticks = (uint64_t)((double)us * 1000.0 * ctx->ticks_per_ns);
  return AGEMM_OK;
}

int fdc_produce(fdc_ctx* ctx, const void* const* o_parts, const void* const* lse_parts, const agemm_schedule* sched,
                void* stream) {
  if (!ctx) return AGEMM_EINVAL;
  int rc = check_parts(ctx, o_parts, lse_parts);
  if (rc) return rc;
  FdProduceArgs pa{};
  rc = fill_schedule(ctx, sched, pa);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // The inbox of this epoch was last read by the fused combines of earlier
  // epochs on it. The producer waits for them on the device (the inbox
  // guard), not with a stream dependency: an event wait in front of every
  // producer cost about 4 us of command-processor time per epoch (59 against
  // 55 us per step). Producers stay in call order.
  const int slot = (int)((ctx->epoch + 1) & 1u);
  hipError_t e = ctx->so.before_produce(s);
  if (e != hipSuccess) return hip_fail(ctx, e, "hipStreamWaitEvent");
  base_args(ctx, o_parts, lse_parts, pa);
  pa.dst = ctx->inbox[slot];
  pa.flags = ctx->flags[slot];
  pa.consumed = ctx->consumed[slot];
  pa.consumed_target = ctx->fused_issued[slot] * (uint32_t)ctx->L.H;  // wraps with the count
  pa.timeout_ticks = ctx->timeout_ticks;
  pa.err = ctx->err_dev;
  pa.t0 = ctx->t0_fused;
  pa.parity = ctx->parity_fused & 1u;
  e = launch_fd_produce(pa, s);
  if (e != hipSuccess) return hip_fail(ctx, e, "producer launch");
  if (pa.has_delay) ctx->parity_fused++;
  e = ctx->so.after_produce(s);
  if (e != hipSuccess) return hip_fail(ctx, e, "hipEventRecord");
  ctx->epoch++;
  ctx->slot_epochs[slot]++;
  return AGEMM_OK;
}

int fdc_run_fused(fdc_ctx* ctx, void* O, void* stream) {
  if (!ctx) return AGEMM_EINVAL;
  if (!aligned16(O)) return fail(ctx, AGEMM_EINVAL, "O must be non-NULL and 16-byte aligned");
  if (ctx->epoch == 0) return fail(ctx, AGEMM_ESTATE, "run_fused before any produce");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int slot = (int)(ctx->epoch & 1u);
  // After the previous combine of this context, whatever its stream: the
  // producer of a later epoch waits only for the last fused combine of an
  // inbox, so an earlier reader of that inbox must be done by then.
  hipError_t e = ctx->so.before_consumer(s);
  if (e != hipSuccess) return hip_fail(ctx, e, "hipStreamWaitEvent");
  // One increment per tile per epoch on this inbox (wraps with the counters).
  int rc = launch_combine(ctx, ctx->inbox[slot], ctx->flags[slot], ctx->slot_epochs[slot], ctx->consumed[slot], O, s);
  if (rc) return rc;
  ctx->fused_issued[slot]++;
  e = ctx->so.after_consumer(s);
  if (e != hipSuccess) return hip_fail(ctx, e, "hipEventRecord");
  return AGEMM_OK;
}

int fdc_run_bsp(fdc_ctx* ctx, const void* const* o_parts, const void* const* lse_parts, void* O,
                const agemm_schedule* sched, int host_sync, void* stream) {
  if (!ctx) return AGEMM_EINVAL;
  int rc = check_parts(ctx, o_parts, lse_parts);
  if (rc) return rc;
  if (!aligned16(O)) return fail(ctx, AGEMM_EINVAL, "O must be non-NULL and 16-byte aligned");
  FdProduceArgs pa{};
  rc = fill_schedule(ctx, sched, pa);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // After the previous combine of this context (the gather buffer is shared by
  // baseline calls).
  hipError_t e = ctx->so.before_consumer(s);
  if (e != hipSuccess) return hip_fail(ctx, e, "hipStreamWaitEvent");
  // 1) all-gather stand-in: every partial into the gather buffer
  base_args(ctx, o_parts, lse_parts, pa);
  pa.dst = ctx->gathered;
  pa.flags = nullptr;
  pa.t0 = ctx->t0_bsp;
  pa.parity = ctx->parity_bsp & 1u;
  e = launch_fd_produce(pa, s);
  if (e != hipSuccess) return hip_fail(ctx, e, "gather launch");
  if (pa.has_delay) ctx->parity_bsp++;
  // 2) the bulk-synchronous barrier
  if (host_sync) {
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(ctx, e, "hipStreamSynchronize");
  }
  // 3) the same combine with the flags off
  rc = launch_combine(ctx, ctx->gathered, nullptr, 0, nullptr, O, s);
  if (rc) return rc;
  e = ctx->so.after_consumer(s);
  if (e != hipSuccess) return hip_fail(ctx, e, "hipEventRecord");
  return AGEMM_OK;
}

int fdc_timing_begin(fdc_ctx* ctx, int32_t max_launches) {
  if (!ctx) return AGEMM_EINVAL;
  return ctx->timer.begin(max_launches, &ctx->last_error);
}

int fdc_timing_end(fdc_ctx* ctx, float* us, int32_t max, int32_t* count) {
  if (!ctx) return AGEMM_EINVAL;
  return ctx->timer.end(us, max, count, &ctx->last_error);
}

int fdc_check(fdc_ctx* ctx) {
  if (!ctx) return AGEMM_EINVAL;
  volatile ErrWord* w = ctx->err_host;
  if (w->code == 0) return AGEMM_OK;
  const unsigned code = w->code, tile = w->tile, target = w->target, seen = w->seen;
  w->code = 0;
  if (code == 2)
    return fail(ctx, AGEMM_ETIMEOUT,
                "producer of tile %u gave up waiting for the earlier combines of its inbox (%u of %u head waves done)",
                tile, seen, target);
  return fail(ctx, AGEMM_ETIMEOUT, "combine gave up waiting for tile %u (flag %u, target %u)", tile, seen, target);
}

const char* fdc_last_error(fdc_ctx* ctx) { return ctx ? ctx->last_error.c_str() : ""; }

}  // extern "C"
