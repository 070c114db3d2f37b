// Decode-attention kernels instantiated for head_dim 128 (kernels and their
// description are in decode_kernels.h).
#include "decode_kernels.h"

namespace iq {

hipError_t launch_decode_128(int bits, const DecodeArgs &a, hipStream_t s) {
  if (a.rope == kDecodeRope) return partial_dispatch_bits<128, kDecodeRope>(bits, a, s);
  return partial_dispatch_bits<128>(bits, a, s);
}

hipError_t launch_merge_128(int variant, const MergeArgs &a, hipStream_t s) {
  return merge_dispatch<128>(variant, a, s);
}

int decode_groups_per_cu_128(int bits, int rope) {
  return rope == kDecodeRope ? partial_groups_per_cu<128, kDecodeRope>(bits) : partial_groups_per_cu<128>(bits);
}

}  // namespace iq
