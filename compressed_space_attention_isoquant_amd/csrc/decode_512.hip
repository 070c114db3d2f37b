// Decode-attention kernels instantiated for head_dim 512 (kernels and their
// description are in decode_kernels.h).
#include "decode_kernels.h"

namespace iq {

hipError_t launch_decode_512(int bits, const DecodeArgs &a, hipStream_t s) {
  if (a.rope == kDecodeRope) return partial_dispatch_bits<512, kDecodeRope>(bits, a, s);
  return partial_dispatch_bits<512>(bits, a, s);
}

hipError_t launch_merge_512(int variant, const MergeArgs &a, hipStream_t s) {
  return merge_dispatch<512>(variant, a, s);
}

int decode_groups_per_cu_512(int bits, int rope) {
  return rope == kDecodeRope ? partial_groups_per_cu<512, kDecodeRope>(bits) : partial_groups_per_cu<512>(bits);
}

}  // namespace iq
