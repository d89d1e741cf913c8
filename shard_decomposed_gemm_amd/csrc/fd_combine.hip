// Flash-Decode combine with fine-grained waits, on gfx950.
//
// "Eliminating Multi-GPU Performance Taxes" analysis page, Flash Decode
// global reduction and correctness check #5: the final output is the
// online-softmax combine of the W ranks' partial outputs, in any order. The
// page's ablation credits most of the Flash-Decode gain to fine-grained waits:
// the combining consumer waits per partial tile instead of for the whole
// all-gather.
//
// Producer (one workgroup per (rank s, head tile j), in release order): copies
// the tile's HT x D partial outputs and HT statistics of rank s into its
// inbox block with device-coherent stores, waits for them, then raises
// Flags(s, j) with one relaxed increment (the same protocol as the AG+GEMM
// producer: a consumer that sees the flag finds the data at the coherence
// point, and no line of the block was read in this launch before).
//
// Combine (one wave per head h, lane l holding d = l, l+64, ...): the wave
// polls the W flags of its head tile, and folds every newly raised rank into
// its running state, lowest rank first among those raised together:
//   m' = max(m, lse_s),  l' = l e^(m-m') + e^(lse_s-m'),
//   acc' = acc e^(m-m') + e^(lse_s-m') o_s,
// then writes acc / l. Waves own disjoint heads, so each takes the ranks in
// its own arrival order with no coordination; rounding depends on that order,
// the exact value does not. Without flags (the baseline) the ranks go in
// ascending order.
#include "fd_internal.h"

namespace agemm {
namespace {

constexpr int kFdThreads = 256;

__device__ inline uint64_t fd_clock() { return __builtin_amdgcn_s_memrealtime(); }

template <bool FLAGS>
__global__ __launch_bounds__(kFdThreads) void fd_produce_kernel(FdProduceArgs a) {
  const int p = blockIdx.x;
  const int tile = a.order[p];
  const int s = tile / a.L.nht;
  const int j = tile - s * a.L.nht;

  if constexpr (FLAGS) {
    // Inbox guard: the fused combines that read this inbox before must be
    // done with it. Their head waves count themselves in after their last
    // read; the stores below cannot overtake those reads, which had
    // returned before the count was raised.
    if (threadIdx.x == 0) {
      const uint64_t start = fd_clock();
      while (true) {
        const uint32_t v = __hip_atomic_load(const_cast<uint32_t*>(a.consumed), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        if ((int32_t)(v - a.consumed_target) >= 0) break;
        if (fd_clock() - start > a.timeout_ticks) {
          __hip_atomic_store(&a.err->tile, (uint32_t)tile, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          __hip_atomic_store(&a.err->target, a.consumed_target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          __hip_atomic_store(&a.err->seen, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          __hip_atomic_store(&a.err->code, 2u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
          break;
        }
        __builtin_amdgcn_s_sleep(4);
      }
    }
    __syncthreads();
  }

  if (a.has_delay) {
    // The first workgroup of the launch fixes its start time; launches with a
    // schedule alternate between two start slots, each clearing the other.
    if (threadIdx.x == 0) {
      const uint64_t now = fd_clock();
      unsigned long long expected = 0;
      __hip_atomic_compare_exchange_strong(reinterpret_cast<unsigned long long*>(a.t0 + a.parity), &expected,
                                           (unsigned long long)now, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t base = expected ? (uint64_t)expected : now;
      const uint64_t due = base + (uint64_t)a.offset_ticks[p];
      while (fd_clock() < due) __builtin_amdgcn_s_sleep(8);
      if (p == 0)
        __hip_atomic_store(reinterpret_cast<unsigned long long*>(a.t0 + (a.parity ^ 1u)), 0ull, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
  }

  const int64_t n_o = (int64_t)a.L.HT * a.L.D / 4;  // 16-byte chunks of outputs
  const int64_t n_all = n_o + a.L.HT / 4;           // plus the statistics
  const uint4* so = reinterpret_cast<const uint4*>(a.o_src[s] + (int64_t)j * a.L.HT * a.L.D);
  const uint4* sl = reinterpret_cast<const uint4*>(a.lse_src[s] + (int64_t)j * a.L.HT);
  char* blk = a.dst + ((int64_t)s * a.L.nht + j) * a.L.blk;
  uint4* dst = reinterpret_cast<uint4*>(blk);  // statistics follow the outputs contiguously
  for (int64_t c = threadIdx.x; c < n_all; c += kFdThreads) {
    const uint4 v = c < n_o ? so[c] : sl[c - n_o];
    if constexpr (FLAGS) {
      uint64_t* d = reinterpret_cast<uint64_t*>(dst + c);
      __hip_atomic_store(d, ((uint64_t)v.y << 32) | v.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(d + 1, ((uint64_t)v.w << 32) | v.z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      dst[c] = v;
    }
  }
  if constexpr (FLAGS) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(a.flags + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <bool GATED, bool OUTF32, int DPL>
__global__ __launch_bounds__(kFdThreads) void fd_combine_kernel(FdCombineArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.x * (kFdThreads / 64) + wave;
  if (h >= a.L.H) return;  // the kernel has no barrier: a spare wave just ends
  const int j = h / a.L.HT;
  const int hr = h - j * a.L.HT;
  const int W = a.L.W;

  float m = -__builtin_inff();
  float l = 0.f;
  float acc[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) acc[k] = 0.f;

  // Folds rank s's partial for head h into the running state.
  auto take = [&](int s) {
    const char* blk = a.src + ((int64_t)s * a.L.nht + j) * a.L.blk;
    const float lse = reinterpret_cast<const float*>(blk + (int64_t)a.L.HT * a.L.D * 4)[hr];
    const float* o = reinterpret_cast<const float*>(blk) + (int64_t)hr * a.L.D;
    float v[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) v[k] = o[lane + 64 * k];
    const float mn = fmaxf(m, lse);
    const float sa = expf(m - mn);   // 0 for the first rank (m = -inf)
    const float sb = expf(lse - mn);
    l = l * sa + sb;
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] = acc[k] * sa + sb * v[k];
    m = mn;
  };

  if constexpr (GATED) {
    const uint32_t all = W >= 32 ? ~0u : ((1u << W) - 1u);
    uint32_t done = 0;
    const uint64_t start = fd_clock();
    while (done != all) {
      bool up = false;
      uint32_t seen = 0;
      if (lane < W) {
        seen = __hip_atomic_load(const_cast<uint32_t*>(a.flags) + lane * a.L.nht + j, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        up = (int32_t)(seen - a.target) >= 0;
      }
      uint32_t ready = __builtin_amdgcn_readfirstlane((uint32_t)__ballot(up)) & ~done;
      if (ready == 0) {
        if (fd_clock() - start > a.timeout_ticks) {
          const int first = __builtin_ctz(all & ~done);
          if (lane == first) {
            __hip_atomic_store(&a.err->tile, (uint32_t)(first * a.L.nht + j), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_SYSTEM);
            __hip_atomic_store(&a.err->target, a.target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            __hip_atomic_store(&a.err->seen, seen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            __hip_atomic_store(&a.err->code, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
          }
          break;  // the output of this head is undefined
        }
        __builtin_amdgcn_s_sleep(2);
        continue;
      }
      // The raised ranks' blocks were not read in this launch before their
      // flags were seen, and the loads below follow the flag values by
      // control dependency.
      asm volatile("" ::: "memory");
      done |= ready;
      while (ready) {
        const int s = __builtin_ctz(ready);
        ready &= ready - 1u;
        take(s);
      }
    }
  } else {
    for (int s = 0; s < W; ++s) take(s);
  }

  const float inv = 1.f / l;
  if constexpr (OUTF32) {
    float* out = static_cast<float*>(a.O) + (int64_t)h * a.L.D;
#pragma unroll
    for (int k = 0; k < DPL; ++k) out[lane + 64 * k] = acc[k] * inv;
  } else {
    _Float16* out = static_cast<_Float16*>(a.O) + (int64_t)h * a.L.D;
#pragma unroll
    for (int k = 0; k < DPL; ++k) out[lane + 64 * k] = (_Float16)(acc[k] * inv);
  }
  if constexpr (GATED) {
    // This head's reads of the inbox have all returned: count it in, so that
    // a later producer of this inbox may overwrite it.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0) __hip_atomic_fetch_add(a.consumed, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <bool GATED, bool OUTF32>
hipError_t launch_combine_dpl(const FdCombineArgs& a, hipStream_t s, const LaunchTiming& t) {
  const dim3 grid((unsigned)((a.L.H + kFdThreads / 64 - 1) / (kFdThreads / 64))), block(kFdThreads);
#define L(D_)                                                                                                    \
  do {                                                                                                           \
    if (t.start)                                                                                                 \
      hipExtLaunchKernelGGL((fd_combine_kernel<GATED, OUTF32, D_>), grid, block, 0, s, t.start, t.stop, 0, a);   \
    else                                                                                                         \
      hipLaunchKernelGGL((fd_combine_kernel<GATED, OUTF32, D_>), grid, block, 0, s, a);                           \
  } while (0)
  switch (a.L.D) {
    case 64: L(1); break;
    case 128: L(2); break;
    case 256: L(4); break;
    default: return hipErrorInvalidValue;
  }
#undef L
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fd_produce(const FdProduceArgs& a, hipStream_t s) {
  const unsigned items = (unsigned)(a.L.W * a.L.nht);
  if (a.flags) hipLaunchKernelGGL(fd_produce_kernel<true>, dim3(items), dim3(kFdThreads), 0, s, a);
  else hipLaunchKernelGGL(fd_produce_kernel<false>, dim3(items), dim3(kFdThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fd_combine(const FdCombineArgs& a, bool out_f32, hipStream_t s, const LaunchTiming& t) {
  const bool gated = a.flags != nullptr;
  if (gated) return out_f32 ? launch_combine_dpl<true, true>(a, s, t) : launch_combine_dpl<true, false>(a, s, t);
  return out_f32 ? launch_combine_dpl<false, true>(a, s, t) : launch_combine_dpl<false, false>(a, s, t);
}

}  // namespace agemm
