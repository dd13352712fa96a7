// Decode kernels for the f32 KV cache (one translation unit per cache dtype
// keeps the build parallel).
#include "decode_kernel.h"

namespace pa {

hipError_t launch_decode_f32(const DecodeArgs& a, int head_dim, int block_size, int group, int64_t upper_items,
                             hipStream_t s, const LaunchEvents& ev) {
  return launch_decode_kv<KV_F32>(a, head_dim, block_size, group, upper_items, s, ev);
}

}  // namespace pa
