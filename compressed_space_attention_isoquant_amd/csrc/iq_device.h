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

// 2-D special case (IsoQuant abstract): the pairs (v.x, v.y) and (v.z, v.w)
// of a 4-D block, read as complex numbers, times z0 = (z.x, z.y) and
// z1 = (z.z, z.w), each stored as (cos, sin).
__device__ __forceinline__ float4 planar_fwd(float4 v, float4 z) {
  return make_float4(z.x * v.x - z.y * v.y, z.y * v.x + z.x * v.y, z.z * v.z - z.w * v.w,
                     z.w * v.z + z.z * v.w);
}

// Inverse: times the conjugates.
__device__ __forceinline__ float4 planar_inv(float4 w, float4 z) {
  return make_float4(z.x * w.x + z.y * w.y, z.x * w.y - z.y * w.x, z.z * w.z + z.w * w.w,
                     z.z * w.w - z.w * w.z);
}

constexpr int kPlanar = 2;

// Floats of rotation parameters per 4-D block: a quaternion pair (Full,
// Fast) or two unit complex numbers (Planar).
__host__ __device__ constexpr int block_param_floats(int variant) { return variant == kPlanar ? 4 : 8; }

// Block rotation of 4-D block blk of a head whose parameters start at p.
template <int VARIANT>
__device__ __forceinline__ float4 block_fwd(float4 v, const float *p, int blk) {
  const float4 *q = reinterpret_cast<const float4 *>(p);
  if constexpr (VARIANT == kPlanar) return planar_fwd(v, q[blk]);
  else return so4_fwd<VARIANT>(v, q[2 * blk], q[2 * blk + 1]);
}

template <int VARIANT>
__device__ __forceinline__ float4 block_inv(float4 w, const float *p, int blk) {
  const float4 *q = reinterpret_cast<const float4 *>(p);
  if constexpr (VARIANT == kPlanar) return planar_inv(w, q[blk]);
  else return so4_inv<VARIANT>(w, q[2 * blk], q[2 * blk + 1]);
}

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

}  // namespace iq
