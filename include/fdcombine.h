/*
 * C-ABI of the flag-gated Flash-Decode combine on one GPU (gfx950).
 *
 * Source: "Eliminating Multi-GPU Performance Taxes" analysis page, the Flash
 * Decode global reduction and correctness check #5, and the page's
 * Flash-Decode ablation (the fine-grained-waits step): each of W ranks
 * computes a partial attention output O_r^partial over its own KV shard; the
 * final output is the online-softmax combine of the W partials, which may be
 * taken in any order, so a consumer that waits per partial (not for all of
 * them) can fold each one in as it arrives.
 *
 * As for the AG+GEMM path (agemm.h), all W inbox slots live in this GPU's
 * memory and a producer kernel fills them: fdc_produce copies each rank's
 * partial into Inbox(s) one head tile at a time and raises Flags(s, tile);
 * fdc_run_fused combines, each wave folding a rank's partial into its running
 * (maximum, scaled sum, scaled output) as soon as that rank's flag for its
 * head tile is raised, in whatever order they come. fdc_run_bsp is the
 * bulk-synchronous baseline: gather copy, host barrier, then the combine
 * with no flags.
 *
 * Partial layout (caller-owned, device memory, read during the call's
 * kernels only):
 *   o_parts[s]   H x D binary32, row-major: the normalised partial output of
 *                rank s (its attention output over its own KV shard), head h
 *                in row h;
 *   lse_parts[s] H binary32: log of the softmax denominator of rank s per
 *                head (log-sum-exp of its scores). Must be finite.
 * Output O: H x D row-major, binary16 (round to nearest even) or binary32:
 *   O[h] = sum_s exp(lse_s[h] - m) o_s[h] / sum_s exp(lse_s[h] - m),
 *   m = max_s lse_s[h].
 *
 * Shapes: 1 <= W <= 16; D in {64, 128, 256}; heads_per_tile (HT) a multiple
 * of 4 in 4..32 dividing H; T = W * H / HT flag tiles, T <= 64. Tile id of
 * (rank s, head tile j) is s * (H / HT) + j; a schedule (agemm_schedule from
 * agemm.h) orders those T ids. All pointers 16-byte aligned.
 *
 * Every call returns an agemm_status, validates before launching (a failed
 * call launches nothing and changes no state), and is asynchronous on the
 * given stream (a hipStream_t passed as void*; NULL = the null stream).
 * Device-side flag waits time out after the spin timeout; fdc_check then
 * reports AGEMM_ETIMEOUT and that call's O is undefined. A context is not
 * thread-safe; use one per host thread. Calls on different streams are
 * ordered as in agemm.h (producer after producer, combine after combine; on
 * the context's own streams the event a later call waits for is recorded
 * when that call is made).
 */
#ifndef FDCOMBINE_H_
#define FDCOMBINE_H_

#include <stdint.h>

#include "agemm.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fdc_ctx fdc_ctx;

/* Creates a context for one shape on the current device: two inboxes (used by
 * alternate epochs) of W x T/W blocks, their flags (zeroed), the gather
 * buffer of the baseline and the error word. out_dtype: output dtype.
 * AGEMM_EPOCH_BASE=n in the environment (testing) starts both inboxes' epoch
 * and consumed counts at n, with the flags to match, so that a few calls take
 * the 32-bit counters across their wrap (anything but a number in 0..2^32-1:
 * EINVAL). */
int fdc_create(fdc_ctx** out, int W, int H, int D, int heads_per_tile, agemm_dtype out_dtype);

/* Frees everything the context owns after synchronising the device. NULL is accepted. */
int fdc_destroy(fdc_ctx* ctx);

/* Number of flag tiles T = W * H / heads_per_tile. */
int fdc_tiles(const fdc_ctx* ctx, int32_t* t);

/* Producer: for every tile in the schedule's order and at its times
 * (sched == NULL: tile order, no delay), copies rank s's rows of head tile j
 * (outputs and statistics) into Inbox(s, j) with device-coherent stores,
 * then raises Flags(s, j). o_parts and lse_parts: host arrays of W device
 * pointers. Starts a new epoch. Its kernel first waits on the device until
 * every fused combine issued so far on the same inbox (the epochs two, four,
 * ... before) has finished reading it: each head wave of a combine counts
 * itself in after its last read (the inbox guard; no stream dependency on
 * the combines). Producer calls stay ordered among themselves. */
int fdc_produce(fdc_ctx* ctx, const void* const* o_parts, const void* const* lse_parts,
                const agemm_schedule* sched, void* stream);

/* Flag-gated combine of the latest produced epoch into O (H x D, the
 * context's dtype). Meant to run concurrently with fdc_produce on another
 * stream. ESTATE before any produce. */
int fdc_run_fused(fdc_ctx* ctx, void* O, void* stream);

/* Bulk-synchronous baseline: the producer kernel in gather mode copies every
 * partial (same schedule) into the context's gather buffer, then, if
 * host_sync != 0, the host waits for the stream, then the same combine runs
 * with the flags off, taking the ranks in ascending order. */
int fdc_run_bsp(fdc_ctx* ctx, const void* const* o_parts, const void* const* lse_parts, void* O,
                const agemm_schedule* sched, int host_sync, void* stream);

/* Spin timeout of the flag waits and of the producer's inbox guard, in
 * microseconds (default 2,000,000). */
int fdc_set_spin_timeout_us(fdc_ctx* ctx, int64_t us);

/* A producer and a consumer stream, owned by the context, on which kernels
 * run concurrently (as agemm_streams: verified with a probe kernel pair on
 * the first call, which synchronises the device; EHIP if no pair of new
 * streams overlapped in 8 attempts). */
int fdc_streams(fdc_ctx* ctx, void** producer, void** consumer);

/* Kernel timing, as agemm_timing_begin/end: HIP events attached to the
 * dispatch of each combine kernel launched while active (up to
 * max_launches); end synchronises and returns the durations in microseconds. */
int fdc_timing_begin(fdc_ctx* ctx, int32_t max_launches);
int fdc_timing_end(fdc_ctx* ctx, float* us, int32_t max, int32_t* count);

/* AGEMM_ETIMEOUT if a combine gave up waiting for a flag, or a producer for
 * its inbox guard, since the last check (the error word is then cleared),
 * else AGEMM_OK. Reads host-mapped memory: synchronise both streams first. */
int fdc_check(fdc_ctx* ctx);

/* Message of the last failed call on this context ("" if none). */
const char* fdc_last_error(fdc_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* FDCOMBINE_H_ */
