// Stage-1 kernels: fused normalise + WHT + SO(4) + Lloyd-Max + bit-pack +
// append (RotaryQuant §3.2 Algorithm 1), and the inverse (dequantize).
//
// Work split: one head vector of d elements is held by d/32 lanes, 32
// consecutive elements per lane, in registers.  The Walsh-Hadamard butterflies
// with stride < 32 run inside a lane; the log2(d/32) strides >= 32 are
// lane-xor exchanges.  Each SO(4) block (4 consecutive elements) is in one
// lane, and the 32 codes of a lane form exactly b whole dwords of the packed
// row (32 * b bits), so packing needs no cross-lane traffic.
#include "iq_device.h"
#include "iq_internal.h"

namespace iq {
namespace {

constexpr int kThreads = 256;

template <typename T>
struct IO;

template <>
struct IO<float> {
  // 32 consecutive elements starting at p (16-byte aligned).
  __device__ static void load32(const float *p, float (&r)[32]) {
    const float4 *p4 = reinterpret_cast<const float4 *>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float4 v = p4[i];
      r[4 * i + 0] = v.x;
      r[4 * i + 1] = v.y;
      r[4 * i + 2] = v.z;
      r[4 * i + 3] = v.w;
    }
  }
  __device__ static void store32(float *p, const float (&r)[32]) {
    float4 *p4 = reinterpret_cast<float4 *>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) p4[i] = make_float4(r[4 * i], r[4 * i + 1], r[4 * i + 2], r[4 * i + 3]);
  }
};

template <>
struct IO<_Float16> {
  __device__ static void load32(const _Float16 *p, float (&r)[32]) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const h8 *p8 = reinterpret_cast<const h8 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h8 v = p8[i];
#pragma unroll
      for (int k = 0; k < 8; ++k) r[8 * i + k] = static_cast<float>(v[k]);
    }
  }
  __device__ static void store32(_Float16 *p, const float (&r)[32]) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    h8 *p8 = reinterpret_cast<h8 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h8 v;
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = static_cast<_Float16>(r[8 * i + k]);
      p8[i] = v;
    }
  }
};

// Unnormalised Walsh-Hadamard butterflies over d = 32 * LPV elements held as
// r[0..31] in each of LPV consecutive lanes (lane j holds elements 32j..32j+31).
template <int LPV>
__device__ __forceinline__ void wht_butterflies(float (&r)[32], int j) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      if ((k & h) == 0) {
        float a = r[k], b = r[k + h];
        r[k] = a + b;
        r[k + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int hl = 1; hl < LPV; hl <<= 1) {
    const bool upper = (j & hl) != 0;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      float o = shfl_xor(r[k], hl);
      r[k] = upper ? (o - r[k]) : (r[k] + o);
    }
  }
}

template <int D, int BITS, int VARIANT, typename TIn>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantArgs a) {
  constexpr int LPV = D / 32;            // lanes per vector
  constexpr int VPW = 64 / LPV;          // vectors per wave
  constexpr int VPB = VPW * (kThreads / 64);
  constexpr int NLEV = 1 << BITS;
  constexpr int ROWB = D * BITS / 8;     // packed row bytes
  const int h = blockIdx.y;

  __shared__ float4 qs[D / 4][2];        // (q_L, q_R) of this head's blocks
  for (int i = threadIdx.x; i < D / 2; i += kThreads)
    qs[i >> 1][i & 1] = reinterpret_cast<const float4 *>(a.quats + (size_t)h * D * 2)[i];
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane % LPV;
  const long long nvec = (long long)a.batch * a.n;
  const long long v = (long long)blockIdx.x * VPB + wave * VPW + lane / LPV;
  const bool valid = v < nvec;
  const long long vv = valid ? v : 0;    // inactive lanes still join the exchanges

  float r[32];
  const TIn *src = static_cast<const TIn *>(a.x) + ((size_t)vv * a.hkv + h) * D + 32 * j;
  IO<TIn>::load32(src, r);

  // s = ||x||_2 (fp32 sum of squares, tree over the vector's lanes)
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < 32; ++k) ss = fmaf(r[k], r[k], ss);
#pragma unroll
  for (int m = 1; m < LPV; m <<= 1) ss += shfl_xor(ss, m);
  const float s = sqrtf(ss);
  // x^ = x / s folded with the 1/sqrt(d) of the normalised transform
  const float inv = s > 0.f ? 1.0f / (s * sqrtf((float)D)) : 0.f;
#pragma unroll
  for (int k = 0; k < 32; ++k) r[k] *= inv;

  wht_butterflies<LPV>(r, j);

#pragma unroll
  for (int blk = 0; blk < 8; ++blk) {
    const int gb = 8 * j + blk;
    float4 t = so4_fwd<VARIANT>(make_float4(r[4 * blk], r[4 * blk + 1], r[4 * blk + 2], r[4 * blk + 3]),
                                qs[gb][0], qs[gb][1]);
    r[4 * blk] = t.x;
    r[4 * blk + 1] = t.y;
    r[4 * blk + 2] = t.z;
    r[4 * blk + 3] = t.w;
  }

  // Lloyd-Max code = number of thresholds strictly below the value; packed
  // LSB-first: code k of this lane occupies bits BITS*k .. BITS*k+BITS-1.
  uint32_t w[BITS];
#pragma unroll
  for (int i = 0; i < BITS; ++i) w[i] = 0u;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    uint32_t code = 0;
#pragma unroll
    for (int t = 0; t < NLEV - 1; ++t) code += (r[k] > a.tab.thr[t]) ? 1u : 0u;
    const int bit = BITS * k;
    w[bit >> 5] |= code << (bit & 31);
    if ((bit & 31) + BITS > 32) w[(bit >> 5) + 1] |= code >> (32 - (bit & 31));
  }

  if (valid) {
    const int b = (int)(v / a.n);
    const int t = (int)(v % a.n);
    const long long row = ((long long)b * a.hkv + h) * a.capacity + a.start_pos[b] + t;
    uint32_t *dst = reinterpret_cast<uint32_t *>(a.codes + row * ROWB + 4 * BITS * j);
    if constexpr (BITS == 4) {
      *reinterpret_cast<uint4 *>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    } else if constexpr (BITS == 2) {
      *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[1]);
    } else {
#pragma unroll
      for (int i = 0; i < BITS; ++i) dst[i] = w[i];
    }
    if (j == 0) a.norms[row] = float_to_half_bits(s);
  }
}

template <int D, int BITS, int VARIANT, typename TOut>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(DequantArgs a) {
  constexpr int LPV = D / 32;
  constexpr int VPW = 64 / LPV;
  constexpr int VPB = VPW * (kThreads / 64);
  constexpr int NLEV = 1 << BITS;
  constexpr int ROWB = D * BITS / 8;
  const int h = blockIdx.y;

  __shared__ float4 qs[D / 4][2];
  __shared__ float cent[NLEV];
  for (int i = threadIdx.x; i < D / 2; i += kThreads)
    qs[i >> 1][i & 1] = reinterpret_cast<const float4 *>(a.quats + (size_t)h * D * 2)[i];
  if (threadIdx.x < NLEV) cent[threadIdx.x] = a.tab.cent[threadIdx.x];
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane % LPV;
  const long long nvec = (long long)a.batch * a.n;
  const long long v = (long long)blockIdx.x * VPB + wave * VPW + lane / LPV;
  const bool valid = v < nvec;
  const int b = valid ? (int)(v / a.n) : 0;
  const int t = valid ? (int)(v % a.n) : 0;
  const long long row = ((long long)b * a.hkv + h) * a.capacity + a.start_pos[b] + t;

  uint32_t w[BITS];
  const uint32_t *src = reinterpret_cast<const uint32_t *>(a.codes + row * ROWB + 4 * BITS * j);
#pragma unroll
  for (int i = 0; i < BITS; ++i) w[i] = src[i];
  const float s16 = half_bits_to_float(a.norms[row]);

  float r[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int bit = BITS * k;
    uint32_t code = w[bit >> 5] >> (bit & 31);
    if ((bit & 31) + BITS > 32) code |= w[(bit >> 5) + 1] << (32 - (bit & 31));
    r[k] = cent[code & (NLEV - 1)];
  }

#pragma unroll
  for (int blk = 0; blk < 8; ++blk) {
    const int gb = 8 * j + blk;
    float4 u = so4_inv<VARIANT>(make_float4(r[4 * blk], r[4 * blk + 1], r[4 * blk + 2], r[4 * blk + 3]),
                                qs[gb][0], qs[gb][1]);
    r[4 * blk] = u.x;
    r[4 * blk + 1] = u.y;
    r[4 * blk + 2] = u.z;
    r[4 * blk + 3] = u.w;
  }

  wht_butterflies<LPV>(r, j);

  const float scale = s16 / sqrtf((float)D);
#pragma unroll
  for (int k = 0; k < 32; ++k) r[k] *= scale;

  if (valid) {
    TOut *dst = static_cast<TOut *>(a.out) + ((size_t)v * a.hkv + h) * D + 32 * j;
    IO<TOut>::store32(dst, r);
  }
}

template <int D, int BITS, int VARIANT>
hipError_t quantize_dispatch_io(int in_f16, const QuantArgs &a, hipStream_t s) {
  constexpr int VPB = (64 / (D / 32)) * (kThreads / 64);
  const long long nvec = (long long)a.batch * a.n;
  dim3 grid((unsigned)((nvec + VPB - 1) / VPB), (unsigned)a.hkv);
  if (in_f16)
    hipLaunchKernelGGL((quantize_kernel<D, BITS, VARIANT, _Float16>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((quantize_kernel<D, BITS, VARIANT, float>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D, int BITS, int VARIANT>
hipError_t dequantize_dispatch_io(int out_f16, const DequantArgs &a, hipStream_t s) {
  constexpr int VPB = (64 / (D / 32)) * (kThreads / 64);
  const long long nvec = (long long)a.batch * a.n;
  dim3 grid((unsigned)((nvec + VPB - 1) / VPB), (unsigned)a.hkv);
  if (out_f16)
    hipLaunchKernelGGL((dequantize_kernel<D, BITS, VARIANT, _Float16>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((dequantize_kernel<D, BITS, VARIANT, float>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D, int BITS>
hipError_t quantize_dispatch_variant(int variant, int in_f16, const QuantArgs &a, hipStream_t s) {
  return variant == 0 ? quantize_dispatch_io<D, BITS, 0>(in_f16, a, s)
                      : quantize_dispatch_io<D, BITS, 1>(in_f16, a, s);
}

template <int D, int BITS>
hipError_t dequantize_dispatch_variant(int variant, int out_f16, const DequantArgs &a, hipStream_t s) {
  return variant == 0 ? dequantize_dispatch_io<D, BITS, 0>(out_f16, a, s)
                      : dequantize_dispatch_io<D, BITS, 1>(out_f16, a, s);
}

template <int D>
hipError_t quantize_dispatch_bits(int bits, int variant, int in_f16, const QuantArgs &a, hipStream_t s) {
  switch (bits) {
    case 2: return quantize_dispatch_variant<D, 2>(variant, in_f16, a, s);
    case 3: return quantize_dispatch_variant<D, 3>(variant, in_f16, a, s);
    case 4: return quantize_dispatch_variant<D, 4>(variant, in_f16, a, s);
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t dequantize_dispatch_bits(int bits, int variant, int out_f16, const DequantArgs &a, hipStream_t s) {
  switch (bits) {
    case 2: return dequantize_dispatch_variant<D, 2>(variant, out_f16, a, s);
    case 3: return dequantize_dispatch_variant<D, 3>(variant, out_f16, a, s);
    case 4: return dequantize_dispatch_variant<D, 4>(variant, out_f16, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_quantize(int d, int bits, int variant, int in_f16, const QuantArgs &a, hipStream_t s) {
  switch (d) {
    case 128: return quantize_dispatch_bits<128>(bits, variant, in_f16, a, s);
    case 256: return quantize_dispatch_bits<256>(bits, variant, in_f16, a, s);
    case 512: return quantize_dispatch_bits<512>(bits, variant, in_f16, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_dequantize(int d, int bits, int variant, int out_f16, const DequantArgs &a, hipStream_t s) {
  switch (d) {
    case 128: return dequantize_dispatch_bits<128>(bits, variant, out_f16, a, s);
    case 256: return dequantize_dispatch_bits<256>(bits, variant, out_f16, a, s);
    case 512: return dequantize_dispatch_bits<512>(bits, variant, out_f16, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace iq
