// Head-dim dispatch of the decode-attention kernels (decode_kernels.h).
#include "iq_internal.h"

namespace iq {

hipError_t launch_decode_128(int bits, const DecodeArgs &a, hipStream_t s);
hipError_t launch_decode_256(int bits, const DecodeArgs &a, hipStream_t s);
hipError_t launch_decode_512(int bits, const DecodeArgs &a, hipStream_t s);
hipError_t launch_merge_128(int variant, const MergeArgs &a, hipStream_t s);
hipError_t launch_merge_256(int variant, const MergeArgs &a, hipStream_t s);
hipError_t launch_merge_512(int variant, const MergeArgs &a, hipStream_t s);

namespace {

constexpr int kOrderThreads = 1024;

// Longest-first order of the (sequence, split) pairs by token count
// (min(chunk, kv_len - split * chunk), at least 0), ties in (split, sequence)
// order: one workgroup.  The 64-bit keys (distinct) are ranked by counting
// up to kOrderThreads pairs (one pass, one barrier), else sorted with a
// bitonic network in LDS.
__global__ __launch_bounds__(kOrderThreads) void order_kernel(const int32_t *kv_len, int batch, int n_split,
                                                              int chunk, int2 *order) {
  __shared__ unsigned long long key[kMaxOrderedPairs];
  const int n = batch * n_split;
  int npad = 1;
  while (npad < n) npad <<= 1;
  for (int i = threadIdx.x; i < npad; i += kOrderThreads) {
    unsigned long long k = ~0ull;
    if (i < n) {
      const int sp = i / batch, b = i - sp * batch;
      long long tok = (long long)kv_len[b] - (long long)sp * chunk;
      tok = tok < 0 ? 0 : (tok > chunk ? chunk : tok);
      k = ((unsigned long long)(chunk - tok) << 32) | (unsigned)i;
    }
    key[i] = k;
  }
  __syncthreads();
  if (n <= kOrderThreads) {
    const int i = threadIdx.x;
    if (i < n) {
      const unsigned long long k = key[i];
      int r = 0;
      for (int m = 0; m < n; ++m) r += key[m] < k ? 1 : 0;
      const int sp = i / batch, b = i - sp * batch;
      order[r] = make_int2((sp << 16) | b, kv_len[b]);
    }
    return;
  }
  for (int size = 2; size <= npad; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < npad; i += kOrderThreads) {
        const int j = i ^ stride;
        if (j > i) {
          const unsigned long long x = key[i], y = key[j];
          if ((x > y) == ((i & size) == 0)) {
            key[i] = y;
            key[j] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int r = threadIdx.x; r < n; r += kOrderThreads) {
    const int i = (int)(key[r] & 0xffffffffu);
    const int sp = i / batch, b = i - sp * batch;
    order[r] = make_int2((sp << 16) | b, kv_len[b]);
  }
}

}  // namespace

hipError_t launch_decode(int d, int bits, const DecodeArgs &a, hipStream_t s) {
  if (a.order) {
    hipLaunchKernelGGL(order_kernel, dim3(1), dim3(kOrderThreads), 0, s, a.kv_len, a.batch, a.n_split, a.chunk,
                       a.order);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
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

}  // namespace iq
