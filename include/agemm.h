/*
 * agemm.h — flag-gated, shard-decomposed AG+GEMM on one MI355X (gfx950).
 *
 * The operation (source: "Eliminating Multi-GPU Performance Taxes", detailed
 * analysis page — symbol table and the AG+GEMM core identity):
 *
 *     C = A . B = [A_0 | A_1 | ... | A_{W-1}] . B
 *       = sum_{s=0}^{W-1} A_s . B[s*K/W : (s+1)*K/W, :]
 *
 * A (M x K) is split along K into W shards A_s (M x K/W); B (K x N) and C
 * (M x N) are whole. In the page's Push model a producer stores every shard
 * into a receive buffer Inbox(s, k) and then raises a ready counter
 * Flags(s, k) per tile; the GEMM waits on each tile's flag and consumes that
 * K-slice at once instead of waiting for the whole all-gather. The page's
 * ordering requirement (its correctness check #4) is that a consumer which
 * sees the flag raised also sees the data. Here all W inbox slots live in the
 * HBM of one GPU. The producer writes a tile with device-coherent stores
 * (written through to the coherence point), waits until they have completed,
 * and only then increments the flag (relaxed, agent scope). The consumer
 * polls the flags with relaxed agent-scope loads and reads no line of a tile
 * before it has seen that tile's flag raised; its loads follow the flag value
 * by control dependency. AGEMM_STRICT_ACQUIRE=1 in the environment at create
 * time adds an agent-scope acquire fence after each wait.
 *
 * Layouts: every matrix is row-major fp16 (IEEE binary16) unless stated.
 *   A_s   M x KS, KS = K/W, row stride KS elements (one buffer per shard)
 *   B     K x N,  row stride N (N contiguous); shard s uses rows [s*KS, (s+1)*KS)
 *   C     M x N,  row stride N; fp16 (rounded to nearest even from the fp32
 *         accumulator) or fp32, chosen at create time; overwritten (no beta)
 * A k-tile is BKf consecutive columns of one shard over all M rows;
 * tile id = s*KT + kt with KT = KS/BKf, T = W*KT tiles in all.
 *
 * Shapes accepted: 1 <= W <= 16, K % W == 0, KS % 64 == 0, N % 8 == 0,
 * 8 <= N <= 2^24, K <= 2^22, 1 <= M <= 2^31-1, BKf a multiple of 64 that
 * divides KS, T <= 64. (The K and N bounds keep every per-lane load offset
 * of the GEMM within 32 bits.)
 * Pointers: device pointers, 16-byte aligned. Streams are hipStream_t passed
 * as void* (NULL = the null stream).
 *
 * Errors: every call returns an agemm_status and never aborts. Arguments are
 * validated before anything is launched; a rejected call changes no state.
 * Calls are asynchronous on the given stream. A consumer that waits longer
 * than the spin timeout for a flag stops, records the tile in a device error
 * word and leaves C undefined; a producer that waits longer than the spin
 * timeout for the consumers of its inbox (the inbox guard, agemm_produce)
 * records that and copies anyway (that epoch's results are then undefined).
 * agemm_check() reports either after the caller has synchronised.
 *
 * Ordering between calls on different streams: every producer comes after
 * the previous producer of the context, every consumer call (run_fused,
 * run_bsp, run_pull) after the previous consumer call. On the context's own
 * streams (agemm_streams) the event a later call on another stream waits for
 * is recorded only when that call is made, on the stream of the earlier call,
 * so the later call may also wait for work queued there in between; on
 * caller streams it is recorded right after each call. Destroying a caller
 * stream is safe at any time; the context's streams live until
 * agemm_destroy.
 *
 * Ownership: the context owns two inboxes (each W x M x KS fp16, used by
 * alternate epochs) with their flags (T uint32 counters each), the
 * gathered-A buffer of the BSP path, the split-K workspaces and the error
 * word, and the inbox guard's counters (64 per inbox, 4 KiB apart). The
 * caller owns A_s, B, C and the streams it passes. Everything is allocated at
 * create time; no other call allocates.
 *
 * Work split of the GEMM (fixed at create time). With few output tiles (at
 * most half as many as the GPU's compute units) whole tiles would leave most
 * units idle; the GEMM then deals equal runs of (output tile, shard) units to
 * one workgroup per compute unit (stream-K; with the 256-row tiles on 7/8 of
 * the units, leaving the rest to the producer, since those split kernels
 * hold a whole SIMD's registers per wave). A tile whose shards
 * fall to several workgroups is summed by the last of them to finish, in a
 * fixed order (contributors' shard ranges ascending), from fp32 partials the
 * others leave in the context's workspace; the result does not depend on
 * timing, and the fused, BSP and pull paths of one context give identical C.
 * Consumer calls of one context are ordered after each other (device side)
 * because they share this workspace.
 * A context is not thread-safe; use one per host thread.
 */
#ifndef AGEMM_H
#define AGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct agemm_ctx agemm_ctx;

typedef enum {
  AGEMM_OK = 0,
  AGEMM_EINVAL = 1,   /* null or misaligned pointer, bad enum, bad schedule */
  AGEMM_ESHAPE = 2,   /* shape outside the accepted set above */
  AGEMM_ENOMEM = 3,   /* device or host allocation failed */
  AGEMM_EHIP = 4,     /* a HIP runtime call failed; see agemm_last_error */
  AGEMM_ETIMEOUT = 5, /* a flag wait or an inbox guard wait timed out (reported by agemm_check) */
  AGEMM_ESTATE = 6    /* call out of order, e.g. run_fused before any produce */
} agemm_status;

typedef enum { AGEMM_F16 = 0, AGEMM_F32 = 1 } agemm_dtype;

/* Order in which the fused consumer takes an output tile's flag tiles. */
typedef enum {
  AGEMM_ORDER_SHARD = 0,   /* s = 0..W-1, k-tiles ascending (the core identity's loop order) */
  AGEMM_ORDER_ARRIVAL = 1  /* raised ones first, see agemm_set_order */
} agemm_order;

/* Release schedule of the producer (host arrays, read during the call only).
 * order[p] is the tile id released p-th; offset_ns[p] is its release time in
 * nanoseconds after the producer starts, non-decreasing in p. n must equal T
 * and order must be a permutation of 0..T-1. */
typedef struct {
  int32_t n;
  const int32_t* order;
  const int64_t* offset_ns;
} agemm_schedule;

/* Creates a context for one shape. flag_ktile = BKf in elements; 0 picks
 * min(256, KS), widened until T <= 64. Allocates the inbox and the flags
 * (zeroed) on the current device. Tuning knobs read from the environment at
 * this call (all optional; invalid values are ignored):
 *   AGEMM_SPIN_TIMEOUT_MS    flag-wait and inbox-guard timeout (default 2000 ms)
 *   AGEMM_STRICT_ACQUIRE=1   agent-scope acquire fence after each flag wait
 *   AGEMM_TILE_CONFIG=0..2   MFMA tile configuration, BM x BN (four waves, BK): 0
 *                            256x256 (BK 32), 1 128x128 (BK 64), 2 256x128 (BK 32).
 *                            Default: 1 for M <= 128, 2 for M <= 256, else 0
 *   AGEMM_SPLIT=0|1          MFMA work split: 0 whole tiles only, 1 the stream-K
 *                            split whenever W >= 2 (default: the split when whole
 *                            tiles would leave at least half of the CUs idle and
 *                            it saves the busiest workgroup 4096 columns of K)
 *   AGEMM_SMALL_M_MAX=0..8   largest M for which the small-M kernel is used
 *                            (default 1; 0: never)
 *   AGEMM_SMALL_M_PLAN=l,r,w small-M work split: lanes, K-ranges, workgroups per CU
 *   AGEMM_PRODUCER_ITEM_KIB  bytes of one tile copied by one producer workgroup
 *                            (1..1024, default 16)
 *   AGEMM_PRODUCER_WGS=n     workgroups of the persistent producer grid (default
 *                            half the CUs; at most one per CU)
 *   AGEMM_EPOCH_BASE=n       testing: both inboxes' epoch counts start at n (flags,
 *                            inbox guard counters and words set to match), so that
 *                            a few calls take the 32-bit counters across their wrap
 *                            (n = 2^32 - 3 wraps on the third call per inbox); anything but a number
 *                            in 0..2^32-1 makes agemm_create return EINVAL */
int agemm_create(agemm_ctx** out, int W, int64_t M, int64_t K, int64_t N, agemm_dtype c_dtype,
                 int64_t flag_ktile);

/* Frees everything the context owns. Synchronises the device first. NULL is accepted. */
int agemm_destroy(agemm_ctx* ctx);

/* Shape queries: BKf, KT = KS/BKf and T = W*KT (any output pointer may be NULL). */
int agemm_tiles(const agemm_ctx* ctx, int64_t* bkf, int32_t* kt, int32_t* t);

/* Consumer kernel the context's GEMM calls launch: *kind = 0 for the MFMA
 * tile kernel (then *tile_config is its tile configuration, 0..2), 1 for the
 * small-M split-K streaming kernel (M = 1 by default, M <= 8 through
 * AGEMM_SMALL_M_MAX; *tile_config = -1). Either output pointer may be NULL. */
int agemm_consumer_kernel(const agemm_ctx* ctx, int32_t* kind, int32_t* tile_config);

/* The MFMA consumer's work plan for a shape on a GPU with num_cus compute
 * units, computed on the host without a device (the choice agemm_create
 * makes): *cfg = tile configuration 0..2, *grid = workgroups of the
 * persistent grid, *split = 1 for the stream-K split. tile_config -1 and
 * split_mode -1 are the automatic choices (AGEMM_TILE_CONFIG / AGEMM_SPLIT
 * give the others); the automatic split needs whole tiles to leave half of
 * the CUs idle and the split to save the busiest workgroup at least 4096
 * columns of K. Applies to the MFMA consumer only (a context with M = 1 uses
 * the small-M kernel by default). EINVAL for M < 1, N < 8, W outside 1..16,
 * K not a positive multiple of W, num_cus < 1 or an out-of-range tile_config
 * / split_mode. Output pointers may be NULL. */
int agemm_mfma_plan(int64_t M, int64_t N, int64_t K, int W, int num_cus, int tile_config, int split_mode,
                    int32_t* cfg, int32_t* grid, int32_t* split);

/* Everything the context's consumer launches are built from (fixed at create
 * time, except where the order set by agemm_set_order changes it, as noted).
 *   kind           0: MFMA tile kernel, 1: small-M split-K streaming kernel
 *   tile_config    MFMA tile configuration 0..2 (-1 for small-M)
 *   block_m/_n     output tile of one MFMA workgroup (0 for small-M)
 *   tiles          output tiles (MFMA) or work items (small-M: K-ranges x column blocks)
 *   grid           workgroups of the launch (a persistent grid: at most one MFMA
 *                  workgroup, or two small-M workgroups, per compute unit)
 *   split          1: the stream-K split over (output tile, shard) units
 *   b_nontemporal  1: B's loads skip L2 allocation (one row block of whole tiles;
 *                  not in arrival order)
 *   tiles_per_wg   most output tiles one workgroup runs (whole tiles), 1 with the split
 *   ranges         small-M K-ranges (0 for MFMA)
 *   a_panels       1: the inbox and the BSP buffer hold A in 32-column k-panels
 *                  (each panel M rows of 32 contiguous elements; the MFMA
 *                  consumer then reads 64-byte rows that lie side by side),
 *                  0: row-major (small-M, or a flag tile's panels of 2^31 bytes
 *                  or more) */
typedef struct {
  int32_t kind, tile_config, block_m, block_n;
  int32_t tiles, grid, split, b_nontemporal;
  int32_t tiles_per_wg, ranges, a_panels;
} agemm_consumer_desc;
int agemm_consumer_info(const agemm_ctx* ctx, agemm_consumer_desc* out);

/* Launch shape of the MFMA consumer: *grid = its workgroups, *split = 1 when
 * it runs the stream-K split described above, else 0. For the small-M kernel
 * *grid = -1 and *split = 0. Either output pointer may be NULL. */
int agemm_consumer_grid(const agemm_ctx* ctx, int32_t* grid, int32_t* split);

/* Producer (Push model): copies tile (s, kt) of A_s into Inbox(s) and then
 * raises Flags(s, kt), for every tile, in the schedule's order and at its
 * times (sched == NULL: shard order, no delay). a_shards: host array of W
 * device pointers, each M x KS fp16. Starts a new epoch: the next run_fused
 * waits for this call's flags. Epochs alternate between the two inboxes.
 * Before it overwrites its inbox the producer waits on the device (the inbox
 * guard) until every run_fused issued on that inbox so far has counted
 * itself out of it, so a producer may fill its inbox while the previous
 * epoch's consumer runs. That run_fused must be able to run meanwhile: on a
 * stream the caller holds up for longer than the spin timeout, the producer
 * gives up waiting (AGEMM_ETIMEOUT from agemm_check). For M above 1024, and
 * for the stream-K split of the 256-row tiles (which leaves no room for
 * producer waves beside it), the producer's stream also waits for the last
 * run_fused on its inbox (an event recorded after each run_fused), so that
 * the producer is not dispatched while that consumer runs. */
int agemm_produce(agemm_ctx* ctx, const void* const* a_shards, const agemm_schedule* sched, void* stream);

/* Flag-gated consumer: C = sum_s Inbox(s) . B_s, waiting on Flags(s, kt)
 * before reading each k-tile. Meant to run concurrently with agemm_produce
 * on another stream. B: K x N fp16; C: M x N in the context's dtype.
 * HIP maps streams onto a few hardware queues (4 by default); two streams
 * on one queue run their work in submission order, so the consumer then
 * starts only after the whole producer (still correct, no overlap):
 * agemm_streams gives a pair verified to run concurrently. */
int agemm_run_fused(agemm_ctx* ctx, const void* B, void* C, void* stream);

/* Bulk-synchronous baseline on the same GPU: a gather kernel copies the
 * shards into one contiguous M x K buffer (honouring the same schedule),
 * then, if host_sync != 0, the host waits for the stream (the barrier), then
 * the same GEMM kernel runs with the flags disabled. */
int agemm_run_bsp(agemm_ctx* ctx, const void* const* a_shards, const void* B, void* C,
                  const agemm_schedule* sched, int host_sync, void* stream);

/* Pull model on one GPU: the GEMM reads every K-slice straight from the W
 * shard buffers; no inbox, no flags, one kernel. */
int agemm_run_pull(agemm_ctx* ctx, const void* const* a_shards, const void* B, void* C, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the Pull
 * GEMM of agemm_run_pull with no context. C = sum_s A_s . B[s*KS:(s+1)*KS, :]
 * with the same shapes, layouts, pointer rules and kernels as a context of
 * this shape (the MFMA kernel on whole tiles only, never the stream-K split).
 * It allocates nothing: the small-M kernel's split-K workspace is a
 * file-scope device array of the library (8 MiB of fp32 partials, i.e.
 * ranges x M x N <= 2,097,152 with up to 8 K-ranges, the kernel running at
 * M = 1 here, and 64 KiB of column counters), held on each device until the process ends. Every call
 * on one GPU shares that array: calls that overlap on one GPU (concurrent
 * streams) race and give undefined C; calls in one stream order are fine.
 * Returns AGEMM_ESHAPE for a shape outside the accepted set or whose
 * workspace exceeds the array, AGEMM_EINVAL for a bad dtype or pointer,
 * AGEMM_EHIP for a runtime failure (also on the first call on a device, which
 * looks up the array's device address). Asynchronous on `stream`. */
int agemm_pull_noalloc(int W, int64_t M, int64_t K, int64_t N, agemm_dtype c_dtype, const void* const* a_shards,
                       const void* B, void* C, void* stream);

/* Flag-tile order of later agemm_run_fused calls (default AGEMM_ORDER_SHARD).
 * The AG+GEMM core identity is a plain sum over shards, so the shards' k-tiles
 * may be added in any order. With AGEMM_ORDER_ARRIVAL each output tile takes
 * first, in ascending id, the flag tiles already raised when the consumer
 * reaches it, then the rest in ascending id (each still waited for), so a late
 * shard delays only the work that needs it. Exact-arithmetic results are
 * unchanged; fp32 rounding may differ from shard order. Runs on whole tiles
 * (the stream-K split, if the context chose it, is not used for these calls)
 * and on the MFMA consumer only; the small-M consumer keeps every K-range
 * resident at once and needs no reordering. EINVAL for an unknown order. */
int agemm_set_order(agemm_ctx* ctx, int order);

/* A producer stream and a consumer stream, owned by the context (destroyed by
 * agemm_destroy), on which kernels run concurrently. HIP maps streams onto a
 * few hardware queues (4 by default); on two streams that share a queue the
 * fused consumer starts only after the whole producer (correct, but without
 * the overlap the Push model is for). The first call creates pairs of
 * non-blocking, default-priority streams and keeps the first pair on which a
 * probe kernel launched second started while the first (sleeping 100 us)
 * still ran; later calls return the same pair. Synchronises the device on
 * the first call (set-up, not hot path). EHIP if no pair overlapped in 8
 * attempts. */
int agemm_streams(agemm_ctx* ctx, void** producer, void** consumer);

/* Flag-wait mode of later run_fused calls: 0 = the consumer reads a tile's
 * data after seeing its flag with no fence (no line of the tile was read in
 * the launch before, so no cache holds a stale copy; loads follow the flag by
 * control dependency), 1 = an agent-scope acquire fence after every wait (and
 * after the launch's first look at the flags). Default: the
 * AGEMM_STRICT_ACQUIRE environment variable at create time, else 0. EINVAL
 * for other values. */
int agemm_set_strict_acquire(agemm_ctx* ctx, int strict);

/* Sets the consumer's spin timeout in microseconds (default 2,000,000, or
 * the AGEMM_SPIN_TIMEOUT_MS environment variable at create time). */
int agemm_set_spin_timeout_us(agemm_ctx* ctx, int64_t us);

/* Kernel timing. agemm_timing_begin allocates (or reuses) max_launches
 * pairs of HIP events; every consumer kernel launched by run_fused, run_bsp
 * or run_pull after it (up to max_launches) carries a pair attached to its
 * own dispatch, so the interval is that kernel's execution on the device
 * (the stamps a kernel-trace profiler reports), not the surrounding stream
 * activity. agemm_timing_end synchronises on those events and writes the
 * durations in microseconds, in launch order, to us[0 .. min(count, max)-1]
 * (us may be NULL); *count receives the number of timed launches.
 * ESTATE if begin is called twice or end without begin. */
int agemm_timing_begin(agemm_ctx* ctx, int32_t max_launches);
int agemm_timing_end(agemm_ctx* ctx, float* us, int32_t max, int32_t* count);

/* Ceilings of the current device, secondary references beside the published
 * peaks the rooflines are quoted against (the measurement of the AG+GEMM
 * analysis page's roofline discussion: compute-bound at large M, B streaming
 * at M = 1). No context needed; calibration calls, not hot-path ones.
 *
 * agemm_device_info: compute units, shader clock and memory clock in kHz and
 * memory bus width in bits, as the HIP device properties report them.
 * EINVAL for a NULL output, EHIP if the runtime cannot answer.
 *
 * agemm_probe_mfma: dense fp16 MFMA throughput from registers only
 * (v_mfma_f32_32x32x16_f16, four independent accumulators per wave, two
 * workgroups of four waves per CU, no memory traffic). Runs `warmup` launches,
 * then times `launches` back-to-back launches (about 1.8 ms each at 2.5 PF)
 * with HIP events on `stream` and waits for them; *tflops = 2 x
 * multiply-adds / average launch time. `out` is a caller-owned device buffer
 * of at least 65536 bytes, 4-byte aligned, that receives one word per
 * workgroup (contents meaningless). EINVAL for NULL pointers, warmup < 0 or
 * launches < 1; EHIP on a runtime failure.
 *
 * agemm_probe_read: streaming read of the caller's device buffer `buf`
 * (`bytes` >= 16, a multiple of 16, 16-byte aligned; make it larger than the
 * 256 MB last-level cache so that HBM serves it) with 16-byte nontemporal
 * loads, eight in flight per thread, eight workgroups per CU, each reading
 * one contiguous chunk. Same timing and
 * `out` contract as agemm_probe_mfma; *gbs = bytes / average launch time,
 * in GB/s (1e9 bytes). The buffer is only read. */
int agemm_device_info(int32_t* cus, int32_t* clock_khz, int32_t* mem_clock_khz, int32_t* bus_bits);
int agemm_probe_mfma(int32_t warmup, int32_t launches, void* out, void* stream, double* tflops);
int agemm_probe_read(const void* buf, int64_t bytes, int32_t warmup, int32_t launches, void* out, void* stream,
                     double* gbs);

/* After the caller has synchronised: AGEMM_ETIMEOUT if a consumer's flag wait
 * or a producer's inbox guard timed out since the last check (the error word
 * is then cleared; agemm_last_error says which), else AGEMM_OK. */
int agemm_check(agemm_ctx* ctx);

/* Text of the last error on this context (never NULL). */
const char* agemm_last_error(const agemm_ctx* ctx);

/* Name of a status code (never NULL). */
const char* agemm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* AGEMM_H */
