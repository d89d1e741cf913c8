// agemm_pull_noalloc: the Pull GEMM of agemm_run_pull with no context and no
// device allocation, for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The only device memory the Pull kernels need beyond the caller's inputs and
// output is the small-M kernel's split-K workspace (per-K-range fp32 partials
// and one counter per column block). Here it is a file-scope device array,
// `scratch`, of fixed size. Its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is
// ever passed to kernels. The MFMA kernel runs whole tiles (no stream-K
// split), which needs no workspace.
#include <mutex>

#include "agemm.h"
#include "agemm_internal.h"

namespace agemm {
namespace {

constexpr size_t kScratchPartialBytes = size_t{8} << 20;  // small-M partials: ranges x M x N fp32
constexpr size_t kScratchCounterBytes = size_t{64} << 10;  // small-M column-block counters
constexpr size_t kScratchBytes = kScratchPartialBytes + kScratchCounterBytes;

static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_setup_mu;
char* g_scratch[kMaxDevices];  // device address of `scratch` on each device (null until set up)
int g_cus[kMaxDevices];

__global__ void clear_words(uint32_t* p, int n) {
  for (int i = (int)(blockIdx.x * blockDim.x + threadIdx.x); i < n; i += (int)(gridDim.x * blockDim.x)) p[i] = 0u;
}

// Once per device, with the device current: the device address of `scratch`
// (the array's name is a host-side stand-in in host code) and the CU count.
int setup(int dev, char** ptr, int* cus) {
  std::lock_guard<std::mutex> lock(g_setup_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return AGEMM_EHIP;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return AGEMM_EHIP;
    g_cus[dev] = n;
    g_scratch[dev] = static_cast<char*>(p);
  }
  *ptr = g_scratch[dev];
  *cus = g_cus[dev];
  return AGEMM_OK;
}

bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace agemm

using namespace agemm;

extern "C" int agemm_pull_noalloc(int W, int64_t M, int64_t K, int64_t N, agemm_dtype c_dtype,
                                  const void* const* a_shards, const void* B, void* C, void* stream) {
  if (c_dtype != AGEMM_F16 && c_dtype != AGEMM_F32) return AGEMM_EINVAL;
  if (W < 1 || W > kMaxShards || M < 1 || M > INT32_MAX || K < 1 || N < 8 || K % W) return AGEMM_ESHAPE;
  const int64_t KS = K / W;
  if (KS % 64 || N % 8 || K > (int64_t{1} << 22) || N > (int64_t{1} << 24)) return AGEMM_ESHAPE;
  // The kernels tile K by the flag k-tile even without flags: the one a
  // context of this shape picks by default.
  const int64_t bkf = default_flag_ktile(KS, W);
  if (bkf == 0) return AGEMM_ESHAPE;
  if (!a_shards || !aligned16(B) || !aligned16(C)) return AGEMM_EINVAL;
  for (int s = 0; s < W; ++s)
    if (!aligned16(a_shards[s])) return AGEMM_EINVAL;

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return AGEMM_EHIP;
  char* ws = nullptr;
  int cus = 0;
  int rc = setup(dev, &ws, &cus);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);

  GemmArgs g{};
  for (int i = 0; i < kMaxShards; ++i) g.a.base[i] = i < W ? static_cast<const _Float16*>(a_shards[i]) : nullptr;
  g.a.lda = KS;
  g.B = static_cast<const _Float16*>(B);
  g.C = C;
  g.M = M;
  g.N = N;
  g.K = K;
  g.KS = KS;
  g.W = W;
  g.num_cus = cus;
  g.tile_config = -1;
  g.gate.flags = nullptr;  // Pull: no flags, no error word
  g.gate.kt = (int32_t)(KS / bkf);
  g.gate.t = W * g.gate.kt;
  g.split = 0;             // whole tiles: no workspace
  const bool f32 = c_dtype == AGEMM_F32;

  const SmallMPlan plan = M <= small_m_default_max() ? small_m_plan(W, M, KS, N, cus) : SmallMPlan{};
  hipError_t e;
  if (plan.ok) {
    const size_t ws_bytes = sizeof(float) * (size_t)plan.ranges * (size_t)M * (size_t)N;
    const size_t cnt_bytes = sizeof(uint32_t) * (size_t)plan.nblk;
    if (ws_bytes > kScratchPartialBytes || cnt_bytes > kScratchCounterBytes) return AGEMM_ESHAPE;
    SmallMArgs sa{};
    sa.g = g;
    sa.plan = plan;
    sa.ws = reinterpret_cast<float*>(ws);
    sa.counters = reinterpret_cast<uint32_t*>(ws + kScratchPartialBytes);
    // The counters must start at zero (every call of this device shares them;
    // a completed launch leaves them at zero, this makes it certain).
    hipLaunchKernelGGL(clear_words, dim3(1), dim3(256), 0, s, sa.counters, plan.nblk);
    e = hipGetLastError();
    if (e == hipSuccess) e = launch_gemm_small_m(sa, f32, s);
  } else {
    e = launch_gemm_mfma(g, f32, s);
  }
  return e == hipSuccess ? AGEMM_OK : AGEMM_EHIP;
}
