// Decode kernels for the bf16 KV cache (one translation unit per cache dtype
// keeps the build parallel).
#include "decode_kernel.h"

namespace pa {

hipError_t launch_decode_bf16(const DecodeArgs& a, int head_dim, int block_size, int group, int64_t upper_items,
                              hipStream_t s, const LaunchEvents& ev) {
  return launch_decode_kv<KV_BF16>(a, head_dim, block_size, group, upper_items, s, ev);
}

}  // namespace pa
