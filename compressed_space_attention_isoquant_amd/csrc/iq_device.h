// Device-side helpers for the IsoQuant kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iq {

// Hamilton product p q, components (w, x, y, z), rule i j = k.
__device__ __forceinline__ float4 hamilton(float4 p, float4 q) {
  float4 r;
  r.x = p.x * q.x - p.y * q.y - p.z * q.z - p.w * q.w;
  r.y = p.x * q.y + p.y * q.x + p.z * q.w - p.w * q.z;
  r.z = p.x * q.z - p.y * q.w + p.z * q.x + p.w * q.y;
  r.w = p.x * q.w + p.y * q.z - p.z * q.y + p.w * q.x;
  return r;
}

__device__ __forceinline__ float4 qconj(float4 q) { return make_float4(q.x, -q.y, -q.z, -q.w); }

// Forward block rotation (IsoQuant abstract): Full v -> q_L v conj(q_R),
// Fast v -> q_L v.
template <int VARIANT>
__device__ __forceinline__ float4 so4_fwd(float4 v, float4 qL, float4 qR) {
  float4 t = hamilton(qL, v);
  if (VARIANT == 0) t = hamilton(t, qconj(qR));
  return t;
}

// Inverse block rotation: Full w -> conj(q_L) w q_R, Fast w -> conj(q_L) w.
template <int VARIANT>
__device__ __forceinline__ float4 so4_inv(float4 w, float4 qL, float4 qR) {
  float4 t = hamilton(qconj(qL), w);
  if (VARIANT == 0) t = hamilton(t, qR);
  return t;
}

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

}  // namespace iq
