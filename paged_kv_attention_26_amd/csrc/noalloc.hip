// pa_decode_noalloc: paged decode for callers that cannot allocate device
// memory (code under HIP graph capture, serving loops that forbid
// allocation).  The split-K partials and arrival counters that pa_decode
// keeps in a caller's workspace live here in one file-scope device array
// instead.  Each GPU holds its own copy of the array, at its own address,
// until the process ends; host code never passes the array's name to a
// kernel (in host code it is only a stand-in for the device symbol), but the
// per-device address hipGetSymbolAddress returns.
#include <mutex>

#include "../../include/pa.h"
#include "pa_internal.h"

namespace {

// The largest workspace pa_decode ever needs: head_dim 128, groups of up to 8
// query heads, two partials per wave for at most kDecodeMaxWaves waves, and
// the arrival counters (34.1 MB).
constexpr size_t kArrivalsBytes = size_t(pa::kDecodeMaxWaves) * sizeof(int32_t);
constexpr size_t kScratchBytes = 34095104;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Zero-fills the arrival counters: a kernel, not hipMemsetAsync, so that the
// set-up may also be captured into a graph.
__global__ void __launch_bounds__(256) zero_words(int32_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Address of the current device's scratch, looked up once per device with
// that device current; the first call also clears its arrival counters on
// the caller's stream.  Returns PA_OK or a PA_ERR_* code.
int device_scratch(hipStream_t s, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return pa::set_error(PA_ERR_HIP, "pa_decode_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return pa::set_error(PA_ERR_UNSUPPORTED, "pa_decode_noalloc: device %d beyond the %d this library tracks", dev,
                         kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return pa::set_error(PA_ERR_HIP, "pa_decode_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    const int n = int(kArrivalsBytes / sizeof(int32_t));
    hipLaunchKernelGGL(zero_words, dim3((n + 255) / 256), dim3(256), 0, s, static_cast<int32_t*>(p), n);
    e = hipGetLastError();
    if (e != hipSuccess)
      return pa::set_error(PA_ERR_HIP, "pa_decode_noalloc: clearing the counters: %s", hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return PA_OK;
}

}  // namespace

extern "C" int pa_decode_noalloc(const pa_kv_cache* cache, const void* q, int32_t q_dtype, void* out,
                                 int32_t out_dtype, int32_t num_seqs, int32_t num_q_heads, float scale,
                                 const int32_t* block_table, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t max_context_len, int32_t partition_tokens,
                                 void* hip_stream) {
  if (!cache) return pa::set_error(PA_ERR_NULL, "cache descriptor is NULL");
  const size_t need = pa::decode_workspace_layout(cache->head_dim).total;
  if (need > kScratchBytes)
    return pa::set_error(PA_ERR_WORKSPACE, "pa_decode_noalloc: head_dim %d needs %zu bytes of scratch, above its %zu",
                         cache->head_dim, need, kScratchBytes);
  void* ws = nullptr;
  const int rc = device_scratch(static_cast<hipStream_t>(hip_stream), &ws);
  if (rc) return rc;
  return pa_decode(cache, q, q_dtype, out, out_dtype, num_seqs, num_q_heads, scale, block_table, max_blocks_per_seq,
                   context_lens, max_context_len, partition_tokens, ws, kScratchBytes, hip_stream);
}
