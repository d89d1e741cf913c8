// Producer of the Push model on one GPU.
//
// "Eliminating Multi-GPU Performance Taxes" analysis page, Push model and
// correctness check #4: a push kernel stores each tile of shard A_s into the
// receive buffer Inbox(s, k) and only afterwards increments the tile's ready
// counter Flags(s, k), so that a consumer that sees the increment also sees
// the data. Here the inbox is in local HBM. The inbox stores are
// device-coherent (agent-scope atomic stores, which go past the per-XCD L2 to
// the coherence point), every thread waits until they have completed, the
// workgroup meets, and one relaxed increment per workgroup raises the flag.
// An agent-scope release increment would instead write back the whole L2 of
// the producer's XCD, including the consumer's dirty C lines, once per
// workgroup. The same kernel with flags == nullptr is the gather copy of the
// bulk-synchronous baseline (the all-gather that concatenates
// [A_0 | ... | A_{W-1}] along K), with plain stores: the kernel boundary
// publishes them.
//
// Work item = rows [q*R, (q+1)*R) of tile (s, kt), items numbered in release
// order p. The gather copy runs one workgroup per item (it runs alone and
// wants the whole GPU). The push runs beside the consumer GEMM: a bounded,
// persistent grid walks the items in release order (workgroup b takes items
// b, b + G, ...), so it occupies a few waves per CU instead of flooding every
// CU with thousands of copy workgroups while the consumer works. A release
// schedule makes an item wait until offset_ticks[p] after a start time
// shared by all workgroups of the launch; offsets do not decrease with p, so
// a workgroup never holds a later item behind an earlier one's delay.
//
// The inbox is guarded on the device: before its first copy, every workgroup
// waits until the fused consumers that read this inbox in earlier epochs have
// counted themselves out of it. Workgroup 0's first wave polls the
// kGuardCounters counters, one lane each, sleeping long between looks, then
// raises the launch's word, which the other workgroups watch. A consumer
// counts a unit out only after that unit's inbox reads have returned, so the
// stores below cannot overtake them. The wait replaces a stream dependency,
// whose command-processor work sat between consecutive consumer launches
// (with the record after each consumer that it waits for, about 3 us per
// step at M = 1).
#include "agemm_internal.h"

namespace agemm {

namespace {

constexpr int kProducerThreads = 256;

__device__ inline uint64_t wall_clock() { return __builtin_amdgcn_s_memrealtime(); }

// 16-byte device-coherent stores: a raw buffer store with cache policy sc1
// (device scope: written through the XCD's L2 to the coherence point), the
// policy the compiler gives an agent-scope relaxed atomic store, which it only
// emits up to 8 bytes. The compiler tracks these stores in its wait counts.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kPolicyDeviceScope = 16;  // sc1 = 1, sc0 = 0
constexpr int kRsrcWord3 = 0x00020000;   // raw 32-bit buffer, gfx9 family

template <bool FLAGS>
__global__ __launch_bounds__(kProducerThreads) void produce_kernel(ProduceArgs a) {
  const int items = a.t * a.items_per_tile;
  if constexpr (FLAGS) {
    if (a.consumed != nullptr && blockIdx.x == 0) {
      if (threadIdx.x < kGuardCounters) {
        const int j = threadIdx.x;
        const uint32_t target = a.guard_target[j];  // wraps with the counter
        const uint64_t start = wall_clock();
        while (true) {
          const uint32_t v = __hip_atomic_load(const_cast<uint32_t*>(a.consumed) + j * kGuardStride,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const uint64_t behind = __ballot((int32_t)(v - target) < 0);
          if (behind == 0) break;
          if (wall_clock() - start > a.timeout_ticks) {
            if (j == __builtin_ctzll(behind)) {
              __hip_atomic_store(&a.err->tile, (uint32_t)j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
              __hip_atomic_store(&a.err->target, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
              __hip_atomic_store(&a.err->seen, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
              __hip_atomic_store(&a.err->code, 2u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
            }
            break;
          }
          // about 4 us between looks: the consumers it waits for run for tens
          // of microseconds or more
          __builtin_amdgcn_s_sleep(127);
        }
        // lets the launch's other workgroups go (after a timeout too)
        if (j == 0) __hip_atomic_store(a.go, a.go_seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
    } else if (a.consumed != nullptr) {
      // The other workgroups wait for workgroup 0's word: one line per look
      // instead of every workgroup reading all the counters.
      if (threadIdx.x == 0) {
        const uint64_t start = wall_clock();
        while (true) {
          const uint32_t v = __hip_atomic_load(a.go, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if ((int32_t)(v - a.go_seq) >= 0) break;
          if (wall_clock() - start > 2 * a.timeout_ticks) {  // workgroup 0 gives up first
            __hip_atomic_store(&a.err->tile, (uint32_t)kGuardCounters, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            __hip_atomic_store(&a.err->target, a.go_seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            __hip_atomic_store(&a.err->seen, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            __hip_atomic_store(&a.err->code, 2u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
            break;
          }
          __builtin_amdgcn_s_sleep(127);
        }
      }
      __syncthreads();
    }
  }
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int p = item / a.items_per_tile;
    const int q = item - p * a.items_per_tile;
    const int tile = a.order[p];
    const int s = tile / a.kt;
    const int kt = tile - s * a.kt;

    if (a.has_delay) {
      // Launches with a schedule alternate between two start-time slots; each
      // clears the other one for the next scheduled launch (stream-ordered).
      if (threadIdx.x == 0) {
        const uint64_t now = wall_clock();
        unsigned long long expected = 0;
        // The first workgroup to arrive fixes the launch's start time.
        __hip_atomic_compare_exchange_strong(reinterpret_cast<unsigned long long*>(a.t0 + a.parity), &expected,
                                             (unsigned long long)now, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t base = expected ? (uint64_t)expected : now;
        const uint64_t due = base + (uint64_t)a.offset_ticks[p];
        while (wall_clock() < due) __builtin_amdgcn_s_sleep(8);
        if (item == 0)
          __hip_atomic_store(reinterpret_cast<unsigned long long*>(a.t0 + (a.parity ^ 1u)), 0ull, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
    }

    const int64_t r0 = (int64_t)q * a.rows_per_item;
    int64_t r1 = r0 + a.rows_per_item;
    if (r1 > a.M) r1 = a.M;
    const int cpr = a.bkf >> 3;  // 16-byte chunks per row segment
    const int64_t total = (r1 - r0) * cpr;
    const _Float16* __restrict__ src = a.src[s] + (int64_t)kt * a.bkf;
    // Row-major dst: the item's rows of the tile's columns. K-panel dst: the
    // item's rows of each of the tile's bkf / 32 panels (panel_ld = M * 32
    // elements apart), chunks taken panel by panel so that a wave's stores
    // are contiguous.
    const int64_t panel_ld = a.M * kPanelK;
    const int rows = (int)(r1 - r0);
    _Float16* __restrict__ dst =
        a.panels ? a.dst + (int64_t)s * a.dst_shard_stride + (int64_t)kt * (a.bkf / kPanelK) * panel_ld + r0 * kPanelK
                 : a.dst + (int64_t)s * a.dst_shard_stride + (int64_t)kt * a.bkf + r0 * a.dst_ld;
    // Push: the byte range the item's stores fall in, under 2^31 (row-major:
    // an item holds at most 1 MiB of a tile and KS / bkf <= 64; k-panels: the
    // context uses them only where a tile's panels span less). The gather
    // copy stores plainly and leaves the descriptor empty.
    const int span = !FLAGS ? 0
                     : a.panels ? (int)(((a.bkf / kPanelK - 1) * panel_ld + rows * kPanelK) * 2)
                                : (int)(((r1 - r0 - 1) * a.dst_ld + a.bkf) * 2);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(dst, 0, span, kRsrcWord3);

    // Four 16-byte chunks in flight per thread (plain registers, no arrays).
    // Chunk cc: row-major (row cc / cpr, chunk cc % cpr); k-panels (panel
    // cc / (4 rows), row, chunk cc % 4 of the panel row).
    auto src_at = [&](int64_t cc) {
      if (a.panels) {
        const int ci = (int)cc, per_panel = rows * 4;
        const int p = ci / per_panel, rem = ci - p * per_panel;
        return reinterpret_cast<const uint4*>(src + (r0 + (rem >> 2)) * a.KS + p * kPanelK + (rem & 3) * 8);
      }
      return reinterpret_cast<const uint4*>(src + (r0 + cc / cpr) * a.KS + (cc % cpr) * 8);
    };
    auto dst_off = [&](int64_t cc) -> int64_t {  // elements
      if (a.panels) {
        const int ci = (int)cc, per_panel = rows * 4;
        const int p = ci / per_panel, rem = ci - p * per_panel;
        return p * panel_ld + rem * 8;
      }
      return (cc / cpr) * a.dst_ld + (cc % cpr) * 8;
    };
    auto put = [&](int64_t cc, const uint4& v) {
      if constexpr (FLAGS) {
        const u32x4 x = {v.x, v.y, v.z, v.w};
        __builtin_amdgcn_raw_buffer_store_b128(x, rsrc, (int)(dst_off(cc) * 2), 0, kPolicyDeviceScope);
      } else {
        *reinterpret_cast<uint4*>(dst + dst_off(cc)) = v;
      }
    };
    constexpr int P = kProducerThreads;
    int64_t c = threadIdx.x;
    for (; c + 3 * P < total; c += 4 * P) {
      const uint4 v0 = *src_at(c);
      const uint4 v1 = *src_at(c + P);
      const uint4 v2 = *src_at(c + 2 * P);
      const uint4 v3 = *src_at(c + 3 * P);
      put(c, v0);
      put(c + P, v1);
      put(c + 2 * P, v2);
      put(c + 3 * P, v3);
    }
    for (; c < total; c += P) put(c, *src_at(c));

    if constexpr (FLAGS) {
      // Every thread's device-coherent stores have completed before the
      // workgroup meets; then one increment publishes the item's part of the
      // tile. The barrier also keeps the next item's delay wait (thread 0)
      // behind this item's stores.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (threadIdx.x == 0) __hip_atomic_fetch_add(a.flags + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (a.has_delay) {
      __syncthreads();  // thread 0's next delay wait starts after this item
    }
  }
}

}  // namespace

hipError_t launch_produce(const ProduceArgs& a, int max_workgroups, hipStream_t s) {
  const unsigned items = (unsigned)a.t * (unsigned)a.items_per_tile;
  const unsigned grid = max_workgroups > 0 && (unsigned)max_workgroups < items ? (unsigned)max_workgroups : items;
  if (a.flags) hipLaunchKernelGGL(produce_kernel<true>, dim3(grid), dim3(kProducerThreads), 0, s, a);
  else hipLaunchKernelGGL(produce_kernel<false>, dim3(grid), dim3(kProducerThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace agemm
