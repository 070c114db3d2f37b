// Decode-attention kernels instantiated for head_dim 256 (kernels and their
// description are in decode_kernels.h).
#include "decode_kernels.h"

namespace iq {

hipError_t launch_decode_256(int bits, const DecodeArgs &a, hipStream_t s) {
  if (a.rope == kDecodeRope) return partial_dispatch_bits<256, kDecodeRope>(bits, a, s);
  return partial_dispatch_bits<256>(bits, a, s);
}

hipError_t launch_merge_256(int variant, const MergeArgs &a, hipStream_t s) {
  return merge_dispatch<256>(variant, a, s);
}

int decode_groups_per_cu_256(int bits, int rope) {
  return rope == kDecodeRope ? partial_groups_per_cu<256, kDecodeRope>(bits) : partial_groups_per_cu<256>(bits);
}

}  // namespace iq
