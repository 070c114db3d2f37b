// Head-dim dispatch of the decode-attention kernels (decode_kernels.h).
#include "iq_internal.h"

namespace iq {

hipError_t launch_decode_128(int bits, const DecodeArgs &a, hipStream_t s);
hipError_t launch_decode_256(int bits, const DecodeArgs &a, hipStream_t s);
hipError_t launch_decode_512(int bits, const DecodeArgs &a, hipStream_t s);
hipError_t launch_merge_128(int variant, const MergeArgs &a, hipStream_t s);
hipError_t launch_merge_256(int variant, const MergeArgs &a, hipStream_t s);
hipError_t launch_merge_512(int variant, const MergeArgs &a, hipStream_t s);
int decode_groups_per_cu_128(int bits, int rope);
int decode_groups_per_cu_256(int bits, int rope);
int decode_groups_per_cu_512(int bits, int rope);

hipError_t launch_decode(int d, int bits, const DecodeArgs &a, hipStream_t s) {
  switch (d) {
    case 128: return launch_decode_128(bits, a, s);
    case 256: return launch_decode_256(bits, a, s);
    case 512: return launch_decode_512(bits, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_merge(int d, int variant, const MergeArgs &a, hipStream_t s) {
  switch (d) {
    case 128: return launch_merge_128(variant, a, s);
    case 256: return launch_merge_256(variant, a, s);
    case 512: return launch_merge_512(variant, a, s);
  }
  return hipErrorInvalidValue;
}

int decode_groups_per_cu(int d, int bits, int rope) {
  switch (d) {
    case 128: return decode_groups_per_cu_128(bits, rope);
    case 256: return decode_groups_per_cu_256(bits, rope);
    case 512: return decode_groups_per_cu_512(bits, rope);
  }
  return 1;
}

}  // namespace iq
