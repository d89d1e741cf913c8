// C-ABI of the flag-gated shard-decomposed AG+GEMM (declared in include/agemm.h).
//
// Host side only: validation, the context (inbox, flags, epochs, workspaces,
// error word), stream ordering between epochs, and kernel selection. Every
// step of the arithmetic runs in the gfx950 kernels of this directory.
#include "agemm.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "agemm_internal.h"
#include "host_common.h"

using namespace agemm;

struct agemm_ctx {
  int W = 0;
  int64_t M = 0, K = 0, N = 0, KS = 0, bkf = 0;
  int32_t kt = 0, t = 0;
  agemm_dtype c_dtype = AGEMM_F16;
  int device = 0;
  int num_cus = 0;
  int tile_config = -1;  // AGEMM_TILE_CONFIG override of the MFMA tile choice
  int order = AGEMM_ORDER_SHARD;  // flag-tile order of the fused consumer (agemm_set_order)
  int strict_acquire = 0;  // AGEMM_STRICT_ACQUIRE=1: agent-scope acquire fence after flag waits
  double ticks_per_ns = 0.1;  // wall clock (kHz / 1e6)
  uint64_t timeout_ticks = 0;

  // Two inboxes, used by alternate epochs, each with its own flags: the
  // producer of epoch e only has to wait for the consumers of epoch e-2, so it
  // can fill its inbox while the consumer of epoch e-1 is still running.
  _Float16* inbox[2] = {nullptr, nullptr};  // each W slots of M x KS
  uint32_t* ctrl = nullptr;      // flags[2][64] | 8 u64: t0 fused[2], t0 bsp[2], probe[3]
  uint32_t* flags[2] = {nullptr, nullptr};
  uint64_t* t0_fused = nullptr;
  uint64_t* t0_bsp = nullptr;
  _Float16* gathered = nullptr;  // M x K, BSP only
  // Layout of the inbox and of the BSP buffer (see ASource): k-panels for the
  // MFMA consumer where a flag tile's panels stay below 2^31 bytes,
  // row-major otherwise (the small-M kernel streams rows).
  int32_t a_panels = 0;
  SmallMPlan small_plan;         // small-M work split (small_plan.ok: the small-M kernel is used)
  float* ws = nullptr;           // small-M split-K workspace, ranges x M x N
  uint32_t* counters = nullptr;  // small-M column-block counters
  MfmaPlan mplan;                // MFMA consumer plan (when the small-M kernel is not used)
  float* mws = nullptr;          // MFMA stream-K partial slots (mplan.split)
  uint32_t* mcnt = nullptr;      // MFMA stream-K tile counters (mplan.split)
  ErrWord* err_host = nullptr;
  ErrWord* err_dev = nullptr;

  int32_t rows_per_item = 1, items_per_tile = 1;
  int32_t producer_wgs = 0;      // persistent grid of the push producer (0: one workgroup per item)
  uint32_t epoch = 0;            // produce calls so far; epoch e uses inbox e & 1
  uint32_t slot_epochs[2] = {0, 0};  // produce calls per inbox so far
  uint32_t parity_fused = 0, parity_bsp = 0;
  // Inbox guard: per inbox, the counters its fused consumers count their
  // units into (device) and the totals of the launches issued on it so far
  // (host). The producer of an inbox waits for them on the device instead of
  // behind a stream dependency.
  uint32_t* guard_mem = nullptr;  // both inboxes' counters, kGuardStride apart
  uint32_t* consumed[2] = {nullptr, nullptr};
  uint32_t guard_target[2][kGuardCounters] = {};
  uint32_t* go[2] = {nullptr, nullptr};  // each inbox's producer word (its own 4 KiB)
  uint32_t produce_seq[2] = {0, 0};      // producer launches per inbox so far
  // Long consumers (M above kGuardOnlyMaxM): the producer also waits, with a
  // stream dependency, for the last fused consumer of its inbox (see produce).
  bool producer_waits_event = false;

  hipStream_t pair[2] = {nullptr, nullptr};  // agemm_streams: producer, consumer (owned)
  uint64_t* probe_times = nullptr;           // 3 words in ctrl for the overlap probe
  StreamOrder so;      // ordering between calls on different streams
  KernelTimer timer;   // agemm_timing_begin/end

  std::string last_error;
};

namespace {

int fail(agemm_ctx* c, int code, const char* fmt, ...) __attribute__((format(printf, 3, 4)));
int fail(agemm_ctx* c, int code, const char* fmt, ...) {
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

int hip_fail(agemm_ctx* c, hipError_t e, const char* what) { return set_hip_error(&c->last_error, e, what); }

int check_shards(agemm_ctx* c, const void* const* a_shards) {
  if (!a_shards) return fail(c, AGEMM_EINVAL, "a_shards is NULL");
  for (int s = 0; s < c->W; ++s)
    if (!aligned16(a_shards[s])) return fail(c, AGEMM_EINVAL, "a_shards[%d] is NULL or not 16-byte aligned", s);
  return AGEMM_OK;
}

int fill_schedule(agemm_ctx* c, const agemm_schedule* sched, ProduceArgs& pa) {
  return parse_schedule(sched, c->t, c->ticks_per_ns, pa.order, pa.offset_ticks, &pa.has_delay, &c->last_error);
}

void base_produce_args(agemm_ctx* c, const void* const* a_shards, ProduceArgs& pa) {
  for (int s = 0; s < kMaxShards; ++s)
    pa.src[s] = s < c->W ? static_cast<const _Float16*>(a_shards[s]) : nullptr;
  pa.M = c->M;
  pa.KS = c->KS;
  pa.bkf = (int32_t)c->bkf;
  pa.kt = c->kt;
  pa.t = c->t;
  pa.rows_per_item = c->rows_per_item;
  pa.items_per_tile = c->items_per_tile;
  pa.panels = c->a_panels;
}

// Orders a new consumer after the previous consumer call of the context.
int order_after_consumer(agemm_ctx* c, hipStream_t s) {
  const hipError_t e = c->so.before_consumer(s);
  return e == hipSuccess ? AGEMM_OK : hip_fail(c, e, "hipStreamWaitEvent");
}

// Launches the GEMM (a4-a6 of the path) with the given A source and gate. A
// fused launch also gets its inbox's guard counters (`consumed`) and adds the
// units it counts into them to their totals (`target`) once launched.
int launch_gemm(agemm_ctx* c, const ASource& src, const Gate& gate, const void* B, void* C, hipStream_t s,
                uint32_t* consumed = nullptr, uint32_t (*target)[kGuardCounters] = nullptr) {
  GemmArgs g{};
  g.a = src;
  g.B = static_cast<const _Float16*>(B);
  g.C = C;
  g.M = c->M;
  g.N = c->N;
  g.K = c->K;
  g.KS = c->KS;
  g.W = c->W;
  g.num_cus = c->num_cus;
  g.tile_config = c->tile_config;
  g.gate = gate;
  g.split = c->mplan.split ? 1 : 0;
  g.arrival = (gate.flags != nullptr && c->order == AGEMM_ORDER_ARRIVAL) ? 1 : 0;
  g.split_ws = c->mws;
  g.split_cnt = c->mcnt;
  g.consumed = consumed;
  const bool f32 = c->c_dtype == AGEMM_F32;
  const LaunchTiming t = c->timer.next();
  hipError_t e;
  if (c->ws) {
    SmallMArgs sa{};
    sa.g = g;
    sa.plan = c->small_plan;
    sa.ws = c->ws;
    sa.counters = c->counters;
    e = launch_gemm_small_m(sa, f32, s, t);
    if (e == hipSuccess && target) add_guard_units(*target, small_m_guard_units(c->small_plan));
  } else {
    e = launch_gemm_mfma(g, f32, s, t);
    if (e == hipSuccess && target) add_guard_units(*target, mfma_guard_units(g));
  }
  if (e != hipSuccess) return hip_fail(c, e, "kernel launch");
  return AGEMM_OK;
}

Gate no_gate(agemm_ctx* c) {
  Gate g{};
  g.flags = nullptr;
  g.kt = c->kt;
  g.t = c->t;
  g.err = c->err_dev;
  return g;
}

void free_all(agemm_ctx* c) {
  c->timer.destroy();
  if (c->inbox[0]) (void)hipFree(c->inbox[0]);
  if (c->ctrl) (void)hipFree(c->ctrl);
  if (c->gathered) (void)hipFree(c->gathered);
  if (c->ws) (void)hipFree(c->ws);
  if (c->counters) (void)hipFree(c->counters);
  if (c->guard_mem) (void)hipFree(c->guard_mem);
  if (c->mws) (void)hipFree(c->mws);
  if (c->mcnt) (void)hipFree(c->mcnt);
  if (c->err_host) (void)hipHostFree(c->err_host);
  c->so.destroy();
  for (int i = 0; i < 2; ++i)
    if (c->pair[i]) (void)hipStreamDestroy(c->pair[i]);
}

}  // namespace

extern "C" {

const char* agemm_status_string(int status) { return status_name(status); }

const char* agemm_last_error(const agemm_ctx* ctx) {
  if (!ctx) return "no context";
  return ctx->last_error.c_str();
}

// Up to this M the producer of an inbox waits for its earlier fused consumers
// only on the device (the inbox guard), dispatched as soon as the previous
// producer is done. Above it, it also waits for the last of them with a
// stream dependency: a producer dispatched early sits on the CUs through the
// whole of a long consumer launch, which slowed the launches of several
// rounds of tiles, while the dependency costs a few microseconds of
// command-processor time per step. Fused step in us, guard alone against
// guard plus dependency, interleaved on one box each: M = 384 212.4 / 215.2,
// M = 512 224.7 / 228.1, M = 1024 421.0 / 426.1 and 423.8 / 424.9,
// M = 2048 838.6 / 821.7, M = 4096 1528.9 / 1514.2.
constexpr int64_t kGuardOnlyMaxM = 1024;

int agemm_create(agemm_ctx** out, int W, int64_t M, int64_t K, int64_t N, agemm_dtype c_dtype, int64_t flag_ktile) {
  if (!out) return AGEMM_EINVAL;
  *out = nullptr;
  if (c_dtype != AGEMM_F16 && c_dtype != AGEMM_F32) return AGEMM_EINVAL;
  uint32_t base = 0;
  const int has_base = epoch_base_from_env(&base);
  if (has_base < 0) return AGEMM_EINVAL;
  if (W < 1 || W > kMaxShards || M < 1 || M > INT32_MAX || K < 1 || N < 8) return AGEMM_ESHAPE;
  if (K % W) return AGEMM_ESHAPE;
  const int64_t KS = K / W;
  if (KS % 64 || N % 8) return AGEMM_ESHAPE;
  if (K > (int64_t{1} << 22) || N > (int64_t{1} << 24)) return AGEMM_ESHAPE;  // 32-bit lane offsets
  int64_t bkf = flag_ktile;
  if (bkf == 0) {
    bkf = default_flag_ktile(KS, W);
    if (bkf == 0) return AGEMM_ESHAPE;
  }
  if (bkf < 64 || bkf % 64 || KS % bkf) return AGEMM_ESHAPE;
  if ((KS / bkf) * W > kMaxTiles) return AGEMM_ESHAPE;

  agemm_ctx* c = new (std::nothrow) agemm_ctx();
  if (!c) return AGEMM_ENOMEM;
  c->W = W;
  c->M = M;
  c->K = K;
  c->N = N;
  c->KS = KS;
  c->bkf = bkf;
  c->kt = (int32_t)(KS / bkf);
  c->t = c->kt * W;
  c->c_dtype = c_dtype;
  // Each producer workgroup copies about 16 KiB of one tile. Small items let
  // the first tiles in release order complete within a few microseconds (their
  // workgroups are dispatched first and share the copy), instead of every tile
  // completing together at the end of the copy; each item costs one flag
  // increment. Measured: 8-16 KiB items cut the fused step by 4 % at M = 128
  // and M = 512 against 256 KiB items. AGEMM_PRODUCER_ITEM_KIB overrides.
  int64_t item_bytes = 16384;
  if (const char* env = std::getenv("AGEMM_PRODUCER_ITEM_KIB")) {
    const long long kib = std::atoll(env);
    if (kib >= 1 && kib <= 1024) item_bytes = kib * 1024;
  }
  c->rows_per_item = (int32_t)std::max<int64_t>(1, item_bytes / (bkf * 2));
  c->items_per_tile = (int32_t)((M + c->rows_per_item - 1) / c->rows_per_item);

  hipError_t e = hipGetDevice(&c->device);
  int wall_khz = 0;
  if (e == hipSuccess) e = hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, c->device);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&c->num_cus, hipDeviceAttributeMultiprocessorCount, c->device);
  if (e != hipSuccess || wall_khz <= 0 || c->num_cus <= 0) {
    delete c;
    return AGEMM_EHIP;
  }
  c->ticks_per_ns = (double)wall_khz / 1.0e6;
  int64_t timeout_us = 2000000;
  if (const char* env = std::getenv("AGEMM_SPIN_TIMEOUT_MS")) {
    const long long ms = std::atoll(env);
    if (ms > 0) timeout_us = ms * 1000;
  }
  c->timeout_ticks = (uint64_t)((double)timeout_us * 1000.0 * c->ticks_per_ns);
  if (const char* env = std::getenv("AGEMM_STRICT_ACQUIRE")) c->strict_acquire = std::atoi(env) != 0;
  // The push producer runs beside the consumer: a persistent grid of half as
  // many workgroups as CUs copies the items in release order instead of one
  // workgroup per item flooding every CU. AGEMM_PRODUCER_WGS overrides, up to
  // one workgroup per CU: the workgroups that wait in the inbox guard must
  // leave room on the CUs for the consumers they wait for (one producer
  // workgroup fits beside a CU's consumer workgroups).
  c->producer_wgs = c->num_cus / 2;
  if (const char* env = std::getenv("AGEMM_PRODUCER_WGS")) {
    const int v = std::atoi(env);
    if (v >= 1) c->producer_wgs = std::min(v, c->num_cus);
  }
  if (const char* env = std::getenv("AGEMM_TILE_CONFIG")) {
    const int v = std::atoi(env);
    if (v >= 0 && v < mfma_config_count()) c->tile_config = v;
  }

  // Everything the context owns is allocated (and zeroed) here, so no call
  // on the hot path allocates or relies on an unordered memset.
  const size_t inbox_bytes = sizeof(_Float16) * (size_t)W * (size_t)M * (size_t)KS;
  const size_t gathered_bytes = sizeof(_Float16) * (size_t)M * (size_t)K;
  const size_t ctrl_bytes = sizeof(uint32_t) * 2 * kMaxTiles + 8 * sizeof(uint64_t);  // + probe times
  const size_t guard_bytes = sizeof(uint32_t) * 2 * (kGuardCounters + 1) * kGuardStride;  // + the two words
  int small_max = small_m_default_max();
  if (const char* env = std::getenv("AGEMM_SMALL_M_MAX")) {
    const int v = std::atoi(env);
    if (v >= 0 && v <= small_m_limit()) small_max = v;
  }
  if (M <= small_max) c->small_plan = small_m_plan(W, M, KS, N, c->num_cus);
  if (const char* env = std::getenv("AGEMM_SMALL_M_PLAN")) {  // "lanes,ranges,wg_per_cu" override
    int l = 0, r = 0, wpc = 0;
    if (std::sscanf(env, "%d,%d,%d", &l, &r, &wpc) == 3 && c->small_plan.ok) {
      const SmallMPlan p = small_m_plan_with(W, M, KS, N, l, r, wpc);
      if (p.ok) c->small_plan = p;
    }
  }
  const bool small = c->small_plan.ok;
  c->a_panels = !small && panel_layout_fits(M, bkf) ? 1 : 0;
  if (!small) {
    int split_mode = -1;
    if (const char* env = std::getenv("AGEMM_SPLIT")) split_mode = std::atoi(env) != 0 ? 1 : 0;
    c->mplan = mfma_plan(M, N, K, W, c->num_cus, c->tile_config, split_mode);
  }
  const size_t ws_bytes = small ? sizeof(float) * (size_t)c->small_plan.ranges * (size_t)M * (size_t)N : 0;
  const size_t cnt_bytes = small ? sizeof(uint32_t) * (size_t)c->small_plan.nblk : 0;
  bool ok = hipMalloc(&c->inbox[0], 2 * inbox_bytes) == hipSuccess;
  ok = ok && hipMalloc(&c->gathered, gathered_bytes) == hipSuccess;
  ok = ok && hipMalloc(&c->ctrl, ctrl_bytes) == hipSuccess;
  ok = ok && hipMalloc(&c->guard_mem, guard_bytes) == hipSuccess;
  ok = ok && hipMemset(c->guard_mem, 0, guard_bytes) == hipSuccess;
  if (ok && small) {
    ok = hipMalloc(&c->ws, ws_bytes) == hipSuccess;
    ok = ok && hipMalloc(&c->counters, cnt_bytes) == hipSuccess;
    ok = ok && hipMemset(c->counters, 0, cnt_bytes) == hipSuccess;
  }
  if (ok && c->mplan.split) {
    ok = hipMalloc(&c->mws, c->mplan.ws_bytes) == hipSuccess;
    ok = ok && hipMalloc(&c->mcnt, c->mplan.cnt_bytes) == hipSuccess;
    ok = ok && hipMemset(c->mcnt, 0, c->mplan.cnt_bytes) == hipSuccess;
  }
  if (!ok) {
    free_all(c);
    delete c;
    return AGEMM_ENOMEM;
  }
  c->inbox[1] = c->inbox[0] + inbox_bytes / sizeof(_Float16);
  c->flags[0] = c->ctrl;
  c->flags[1] = c->ctrl + kMaxTiles;
  c->t0_fused = reinterpret_cast<uint64_t*>(c->ctrl + 2 * kMaxTiles);
  c->t0_bsp = c->t0_fused + 2;
  c->probe_times = c->t0_bsp + 2;
  c->consumed[0] = c->guard_mem;
  c->consumed[1] = c->guard_mem + kGuardCounters * kGuardStride;
  c->go[0] = c->guard_mem + 2 * kGuardCounters * kGuardStride;
  c->go[1] = c->go[0] + kGuardStride;
  // Also where the consumer leaves no room beside it for producer waves (the
  // split kernels of the 256-row tiles): a producer dispatched early could
  // then hold CUs that the consumer it waits for still needs.
  c->producer_waits_event = M > kGuardOnlyMaxM || (!small && c->mplan.split && c->mplan.cfg != 1);
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
    // every produce on an inbox adds items_per_tile to each of its flags
    c->slot_epochs[0] = c->slot_epochs[1] = base;
    const std::vector<uint32_t> init(2 * kMaxTiles, base * (uint32_t)c->items_per_tile);
    e = hipMemcpy(c->ctrl, init.data(), init.size() * sizeof(uint32_t), hipMemcpyHostToDevice);
    if (e == hipSuccess) {
      // the inbox guard's counters and their totals start there too
      std::vector<uint32_t> counts(guard_bytes / sizeof(uint32_t), 0u);
      for (int j = 0; j < 2 * kGuardCounters; ++j) {
        counts[(size_t)j * kGuardStride] = base;
        c->guard_target[j / kGuardCounters][j % kGuardCounters] = base;
      }
      for (int i = 0; i < 2; ++i) {
        counts[(size_t)(2 * kGuardCounters + i) * kGuardStride] = base;
        c->produce_seq[i] = base;
      }
      e = hipMemcpy(c->guard_mem, counts.data(), guard_bytes, hipMemcpyHostToDevice);
    }
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

int agemm_destroy(agemm_ctx* ctx) {
  if (!ctx) return AGEMM_OK;
  (void)hipSetDevice(ctx->device);
  (void)hipDeviceSynchronize();  // a destroy cannot fail: release what was allocated
  free_all(ctx);
  delete ctx;
  return AGEMM_OK;
}

int agemm_tiles(const agemm_ctx* ctx, int64_t* bkf, int32_t* kt, int32_t* t) {
  if (!ctx) return AGEMM_EINVAL;
  if (bkf) *bkf = ctx->bkf;
  if (kt) *kt = ctx->kt;
  if (t) *t = ctx->t;
  return AGEMM_OK;
}

int agemm_consumer_kernel(const agemm_ctx* ctx, int32_t* kind, int32_t* tile_config) {
  if (!ctx) return AGEMM_EINVAL;
  const bool small = ctx->ws != nullptr;
  if (kind) *kind = small ? 1 : 0;
  if (tile_config) *tile_config = small ? -1 : mfma_config_for(ctx->M, ctx->tile_config);
  return AGEMM_OK;
}

int agemm_consumer_grid(const agemm_ctx* ctx, int32_t* grid, int32_t* split) {
  if (!ctx) return AGEMM_EINVAL;
  const bool small = ctx->ws != nullptr;
  if (grid) *grid = small ? -1 : (int32_t)ctx->mplan.grid;
  if (split) *split = small ? 0 : (ctx->mplan.split ? 1 : 0);
  return AGEMM_OK;
}

int agemm_consumer_info(const agemm_ctx* ctx, agemm_consumer_desc* out) {
  if (!ctx || !out) return AGEMM_EINVAL;
  agemm_consumer_desc d{};
  if (ctx->ws) {
    const SmallMPlan& p = ctx->small_plan;
    const int64_t items = (int64_t)p.ranges * p.nblk;
    d.kind = 1;
    d.tile_config = -1;
    d.tiles = (int32_t)items;
    d.grid = (int32_t)std::min<int64_t>(items, (int64_t)p.wg_per_cu * ctx->num_cus);
    d.tiles_per_wg = (int32_t)((items + d.grid - 1) / d.grid);
    d.ranges = p.ranges;
  } else {
    const MfmaPlan& p = ctx->mplan;
    // arrival order runs whole tiles with the default B policy
    const bool arrival = ctx->order == AGEMM_ORDER_ARRIVAL;
    const MfmaPlan q =
        arrival && p.split ? mfma_plan(ctx->M, ctx->N, ctx->K, ctx->W, ctx->num_cus, ctx->tile_config, 0) : p;
    d.kind = 0;
    d.tile_config = q.cfg;
    d.block_m = (int32_t)q.bm;
    d.block_n = (int32_t)q.bn;
    d.tiles = (int32_t)q.tiles;
    d.grid = (int32_t)q.grid;
    d.split = q.split ? 1 : 0;
    d.b_nontemporal = q.bnt && !arrival ? 1 : 0;
    d.tiles_per_wg = q.split ? 1 : (int32_t)((q.tiles + q.grid - 1) / q.grid);
    d.a_panels = ctx->a_panels;
  }
  *out = d;
  return AGEMM_OK;
}

int agemm_mfma_plan(int64_t M, int64_t N, int64_t K, int W, int num_cus, int tile_config, int split_mode, int32_t* cfg,
                    int32_t* grid, int32_t* split) {
  if (M < 1 || N < 8 || W < 1 || W > kMaxShards || K < W || K % W || num_cus < 1 || tile_config < -1 ||
      tile_config >= mfma_config_count() || split_mode < -1 || split_mode > 1)
    return AGEMM_EINVAL;
  const MfmaPlan p = mfma_plan(M, N, K, W, num_cus, tile_config, split_mode);
  if (cfg) *cfg = p.cfg;
  if (grid) *grid = (int32_t)p.grid;
  if (split) *split = p.split ? 1 : 0;
  return AGEMM_OK;
}

int agemm_set_order(agemm_ctx* ctx, int order) {
  if (!ctx) return AGEMM_EINVAL;
  if (order != AGEMM_ORDER_SHARD && order != AGEMM_ORDER_ARRIVAL) return fail(ctx, AGEMM_EINVAL, "unknown order %d", order);
  ctx->order = order;
  return AGEMM_OK;
}

int agemm_streams(agemm_ctx* ctx, void** producer, void** consumer) {
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

int agemm_set_strict_acquire(agemm_ctx* ctx, int strict) {
  if (!ctx) return AGEMM_EINVAL;
  if (strict != 0 && strict != 1) return fail(ctx, AGEMM_EINVAL, "strict must be 0 or 1, got %d", strict);
  ctx->strict_acquire = strict;
  return AGEMM_OK;
}

int agemm_set_spin_timeout_us(agemm_ctx* ctx, int64_t us) {
  if (!ctx) return AGEMM_EINVAL;
  if (us < 1) return fail(ctx, AGEMM_EINVAL, "timeout must be positive");
  ctx->timeout_ticks = (uint64_t)((double)us * 1000.0 * ctx->ticks_per_ns);
  return AGEMM_OK;
}

int agemm_produce(agemm_ctx* ctx, const void* const* a_shards, const agemm_schedule* sched, void* stream) {
  if (!ctx) return AGEMM_EINVAL;
  int rc = check_shards(ctx, a_shards);
  if (rc) return rc;
  ProduceArgs pa{};
  rc = fill_schedule(ctx, sched, pa);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // This epoch's inbox may be overwritten only once the fused consumers that
  // read it before (two epochs ago, and earlier) are done with it: the
  // producer waits for them on the device (the inbox guard), and behind a
  // stream dependency too where producer_waits_event. Producers run in call
  // order.
  const int slot = (int)((ctx->epoch + 1) & 1u);
  hipError_t e = ctx->so.before_produce(s, ctx->producer_waits_event ? slot : -1);
  if (e != hipSuccess) return hip_fail(ctx, e, "hipStreamWaitEvent");
  base_produce_args(ctx, a_shards, pa);
  pa.consumed = ctx->consumed[slot];
  std::memcpy(pa.guard_target, ctx->guard_target[slot], sizeof pa.guard_target);  // wrap with the counters
  pa.go = ctx->go[slot];
  pa.go_seq = ctx->produce_seq[slot] + 1u;
  pa.timeout_ticks = ctx->timeout_ticks;
  pa.err = ctx->err_dev;
  pa.dst = ctx->inbox[slot];
  pa.dst_shard_stride = ctx->M * ctx->KS;
  pa.dst_ld = ctx->KS;
  pa.flags = ctx->flags[slot];
  pa.t0 = ctx->t0_fused;
  pa.parity = ctx->parity_fused & 1u;
  e = launch_produce(pa, ctx->producer_wgs, s);
  if (e != hipSuccess) return hip_fail(ctx, e, "producer launch");
  if (pa.has_delay) ctx->parity_fused++;
  e = ctx->so.after_produce(s);
  if (e != hipSuccess) return hip_fail(ctx, e, "hipEventRecord");
  ctx->epoch++;
  ctx->slot_epochs[slot]++;
  ctx->produce_seq[slot]++;
  return AGEMM_OK;
}

int agemm_run_fused(agemm_ctx* ctx, const void* B, void* C, void* stream) {
  if (!ctx) return AGEMM_EINVAL;
  if (!aligned16(B) || !aligned16(C)) return fail(ctx, AGEMM_EINVAL, "B and C must be non-NULL and 16-byte aligned");
  if (ctx->epoch == 0) return fail(ctx, AGEMM_ESTATE, "run_fused before any produce");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc = order_after_consumer(ctx, s);
  if (rc) return rc;
  const int slot = (int)(ctx->epoch & 1u);
  ASource src{};
  for (int i = 0; i < kMaxShards; ++i)
    src.base[i] = i < ctx->W ? ctx->inbox[slot] + (int64_t)i * ctx->M * ctx->KS : nullptr;
  src.lda = ctx->KS;
  src.panels = ctx->a_panels;
  Gate gate = no_gate(ctx);
  gate.flags = ctx->flags[slot];
  gate.target = ctx->slot_epochs[slot] * (uint32_t)ctx->items_per_tile;  // wraps with the counters
  gate.timeout_ticks = ctx->timeout_ticks;
  gate.strict = ctx->strict_acquire;
  rc = launch_gemm(ctx, src, gate, B, C, s, ctx->consumed[slot], &ctx->guard_target[slot]);
  if (rc) return rc;
  hipError_t e = ctx->producer_waits_event ? ctx->so.after_fused(slot, s) : hipSuccess;
  if (e == hipSuccess) e = ctx->so.after_consumer(s);
  if (e != hipSuccess) return hip_fail(ctx, e, "hipEventRecord");
  return AGEMM_OK;
}

int agemm_run_bsp(agemm_ctx* ctx, const void* const* a_shards, const void* B, void* C, const agemm_schedule* sched,
                  int host_sync, void* stream) {
  if (!ctx) return AGEMM_EINVAL;
  int rc = check_shards(ctx, a_shards);
  if (rc) return rc;
  if (!aligned16(B) || !aligned16(C)) return fail(ctx, AGEMM_EINVAL, "B and C must be non-NULL and 16-byte aligned");
  ProduceArgs pa{};
  rc = fill_schedule(ctx, sched, pa);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = order_after_consumer(ctx, s);
  if (rc) return rc;
  // 1) all-gather stand-in: copy the shards into one M x K buffer
  // ([A_0 | ... | A_{W-1}] row-major, or shard after shard in k-panels)
  base_produce_args(ctx, a_shards, pa);
  pa.dst = ctx->gathered;
  pa.dst_shard_stride = ctx->a_panels ? ctx->M * ctx->KS : ctx->KS;
  pa.dst_ld = ctx->K;
  pa.flags = nullptr;
  pa.t0 = ctx->t0_bsp;
  pa.parity = ctx->parity_bsp & 1u;
  hipError_t e = launch_produce(pa, 0, s);
  if (e != hipSuccess) return hip_fail(ctx, e, "gather launch");
  if (pa.has_delay) ctx->parity_bsp++;
  // 2) the bulk-synchronous barrier
  if (host_sync) {
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(ctx, e, "hipStreamSynchronize");
  }
  // 3) the same GEMM with the flags off, reading the gathered A
  ASource src{};
  for (int i = 0; i < kMaxShards; ++i) src.base[i] = i < ctx->W ? ctx->gathered + (int64_t)i * pa.dst_shard_stride : nullptr;
  src.lda = ctx->K;
  src.panels = ctx->a_panels;
  rc = launch_gemm(ctx, src, no_gate(ctx), B, C, s);
  if (rc) return rc;
  const hipError_t eo = ctx->so.after_consumer(s);
  return eo == hipSuccess ? AGEMM_OK : hip_fail(ctx, eo, "hipEventRecord");
}

int agemm_run_pull(agemm_ctx* ctx, const void* const* a_shards, const void* B, void* C, void* stream) {
  if (!ctx) return AGEMM_EINVAL;
  int rc = check_shards(ctx, a_shards);
  if (rc) return rc;
  if (!aligned16(B) || !aligned16(C)) return fail(ctx, AGEMM_EINVAL, "B and C must be non-NULL and 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = order_after_consumer(ctx, s);
  if (rc) return rc;
  ASource src{};
  for (int i = 0; i < kMaxShards; ++i) src.base[i] = i < ctx->W ? static_cast<const _Float16*>(a_shards[i]) : nullptr;
  src.lda = ctx->KS;
  rc = launch_gemm(ctx, src, no_gate(ctx), B, C, s);
  if (rc) return rc;
  const hipError_t eo = ctx->so.after_consumer(s);
  return eo == hipSuccess ? AGEMM_OK : hip_fail(ctx, eo, "hipEventRecord");
}

int agemm_timing_begin(agemm_ctx* ctx, int32_t max_launches) {
  if (!ctx) return AGEMM_EINVAL;
  return ctx->timer.begin(max_launches, &ctx->last_error);
}

int agemm_timing_end(agemm_ctx* ctx, float* us, int32_t max, int32_t* count) {
  if (!ctx) return AGEMM_EINVAL;
  return ctx->timer.end(us, max, count, &ctx->last_error);
}

int agemm_check(agemm_ctx* ctx) {
  if (!ctx) return AGEMM_EINVAL;
  volatile ErrWord* w = ctx->err_host;
  if (w->code == 0) return AGEMM_OK;
  const unsigned code = w->code, tile = w->tile, target = w->target, seen = w->seen;
  w->code = 0;
  // A timed-out launch can leave split-K counters part-way; clear them.
  hipError_t e = hipSuccess;
  if (ctx->counters) e = hipMemset(ctx->counters, 0, sizeof(uint32_t) * (size_t)ctx->small_plan.nblk);
  if (e == hipSuccess && ctx->mcnt) e = hipMemset(ctx->mcnt, 0, ctx->mplan.cnt_bytes);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(ctx, e, "hipMemset(counters)");
  if (code == 2)
    return fail(ctx, AGEMM_ETIMEOUT,
                "producer gave up waiting for the consumers of its inbox (guard counter %u at %u, target %u)", tile,
                seen, target);
  return fail(ctx, AGEMM_ETIMEOUT, "consumer gave up waiting for tile %u (flag %u, target %u)", tile, seen, target);
}

}  // extern "C"
