// Stage-1 kernels: fused normalise + WHT + SO(4) + Lloyd-Max + bit-pack +
// append (RotaryQuant §3.2 Algorithm 1), and the inverse (dequantize).
//
// Work split: one head vector of d elements is held by d/32 lanes, 32
// consecutive elements per lane, in registers.  The Walsh-Hadamard butterflies
// with stride < 32 run inside a lane; the log2(d/32) strides >= 32 are
// lane-xor exchanges.  Each SO(4) block (4 consecutive elements) is in one
// lane, and the 32 codes of a lane form exactly b whole dwords of the packed
// row (32 * b bits), so packing needs no cross-lane traffic.
#include <type_traits>

#include "iq_device.h"
#include "iq_internal.h"

namespace iq {
namespace {

constexpr int kThreads = 256;

// f(std::integral_constant<int, m>) for m = 1, 2, 4, ... < N.
template <int N, int M = 1, class F>
__device__ __forceinline__ void static_for_pow2(F &&f) {
  if constexpr (M < N) {
    f(std::integral_constant<int, M>{});
    static_for_pow2<N, 2 * M>(f);
  }
}

// Position (batch b, row t) of vector v = b * n + t of a [batch][n] set of
// vectors, stepped by a fixed stride (= sq * n + sr, 0 <= sr < n) without a
// division per step.
struct VecPos {
  int b, t;
  __device__ void init(int v, int n) {
    b = v / n;
    t = v - b * n;
  }
  __device__ void advance(int sq, int sr, int n) {
    t += sr;
    const bool wrap = t >= n;
    t = wrap ? t - n : t;
    b += sq + (wrap ? 1 : 0);
  }
};

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
  __device__ static void load32(const _Float16 *p, _Float16 (&r)[32]) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const h8 *p8 = reinterpret_cast<const h8 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h8 v = p8[i];
#pragma unroll
      for (int k = 0; k < 8; ++k) r[8 * i + k] = v[k];
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

// Value of lane (lane ^ M) within groups of 32 lanes for M = 4 and 16, which
// no DPP pattern of one row reaches: ds_swizzle (bit-mask mode) goes through
// the LDS crossbar, which costs no vector-ALU slot but has LDS latency.
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  static_assert(M == 4 || M == 16, "swizzle exchange");
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), (M << 10) | 0x1F));
}

// Unnormalised Walsh-Hadamard butterflies over d = 32 * LPV elements held as
// r[0..31] in each of LPV consecutive lanes (lane j holds elements 32j..32j+31).
// Across lanes the pair (a, b) of lanes (j, j ^ hl) becomes (a + b, a - b).
// Lane j keeps its values multiplied by a sign sigma(j): the upper lane of a
// pair stores b' = -(a - b) = b - a, so every lane does r += s(j) * other
// with s(j) = -1 on upper lanes, one multiply-add per value.  The signs only
// depend on the lane bits already exchanged, so partners always carry equal
// signs, and after all stages lane j holds sigma(j) * (H x) with
// sigma(j) = (-1)^popcount(j) (lane_sign); the caller multiplies by sigma(j)
// after the transform.
template <int LPV>
__device__ __forceinline__ float lane_sign(int j) {
  return (__builtin_popcount(j & (LPV - 1)) & 1) ? -1.f : 1.f;
}

// r[k] += sign * r[k] of lane (lane ^ M), k = K0 .. K0+7, for M = 1, 2, 8:
// one v_fmac_f32 per value whose first operand is read through DPP, so the
// exchange costs no instruction of its own (the compiler keeps a separate
// DPP move here).  The leading s_nop gives the two wait states a DPP read
// needs after a VALU write of the same register; the same fused multiply-add
// as fmaf, so results are unchanged.
#define IQ_DPP_FMAC8(CTRL)                                                                        \
  asm volatile("s_nop 1\n"                                                                       \
               "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                \
               "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                \
               "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                \
               "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                \
               "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                \
               "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                \
               "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                \
               "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf"                   \
               : "+v"(r[K0]), "+v"(r[K0 + 1]), "+v"(r[K0 + 2]), "+v"(r[K0 + 3]), "+v"(r[K0 + 4]), \
                 "+v"(r[K0 + 5]), "+v"(r[K0 + 6]), "+v"(r[K0 + 7])                               \
               : "v"(sign))

template <int M, int K0>
__device__ __forceinline__ void dpp_fmac8(float (&r)[32], float sign) {
  static_assert(M == 1 || M == 2 || M == 8, "DPP exchange");
  if constexpr (M == 1)
    IQ_DPP_FMAC8("quad_perm:[1,0,3,2]");
  else if constexpr (M == 2)
    IQ_DPP_FMAC8("quad_perm:[2,3,0,1]");
  else
    IQ_DPP_FMAC8("row_ror:8");
}
#undef IQ_DPP_FMAC8

// In-lane strides below 2^F of the transform are applied inside the block
// matrices (F = 2 for Full and Fast: the 4-point transform of each block; 1 for
// Planar, whose 2x2 blocks absorb the stride-1 butterflies and stay 2x2):
// the butterflies of every stride commute, so x -> M H4 (rest of H) x is the
// same map, and the block's 16 multiply-adds replace two butterfly stages.
__host__ __device__ constexpr int fold_stages(int variant) { return variant == kPlanar ? 1 : 2; }

// Lane distances 1, 2 and 8 ride on the multiply-add (DPP operand), 4 and 16
// go through the swizzle.  In-lane strides start at H0.
template <int LPV, int H0>
__device__ __forceinline__ void wht_butterflies(float (&r)[32], int j) {
#pragma unroll
  for (int h = H0; h < 32; h <<= 1) {
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      if ((k & h) == 0) {
        float a = r[k], b = r[k + h];
        r[k] = a + b;
        r[k + h] = a - b;
      }
    }
  }
  static_for_pow2<LPV>([&](auto hl_c) {
    constexpr int hl = decltype(hl_c)::value;
    const float sign = (j & hl) ? -1.f : 1.f;
    if constexpr (hl == 1 || hl == 2 || hl == 8) {
      dpp_fmac8<hl, 0>(r, sign);
      dpp_fmac8<hl, 8>(r, sign);
      dpp_fmac8<hl, 16>(r, sign);
      dpp_fmac8<hl, 24>(r, sign);
    } else {
#pragma unroll
      for (int k = 0; k < 32; ++k) r[k] = fmaf(lane_xor<hl>(r[k]), sign, r[k]);
    }
    // Finish the stage before the next: left to itself the scheduler runs
    // each value through all stages in turn, one exchange latency at a time.
    __builtin_amdgcn_sched_barrier(0);
  });
}

// Columns of the 4x4 matrices M H_F of the forward block rotations M after
// the folded butterflies H_F (the 2^F-point transform on each 2^F-element
// sub-block): column c of block gb = 8 j + blk (held by lane j of a vector)
// is block_fwd(H_F e_c), times lane_sign(j) when SIGNED, stored at
// qm[blk][c][j] so that the lanes of a vector read consecutive 16-byte words
// (no LDS bank conflicts).  The inverse is the transpose of the unsigned
// matrix: (M H_F)^T = H_F M^T, the inverse block rotation followed by the
// folded butterflies.
template <int LPV>
using BlockMatrices = float4[8][4][LPV];

template <int D, int VARIANT, bool SIGNED>
__device__ __forceinline__ void load_block_matrices(BlockMatrices<D / 32> &qm, const float *params) {
  constexpr int F = fold_stages(VARIANT), SUB = (1 << F) - 1;
  for (int i = threadIdx.x; i < D; i += blockDim.x) {
    const int gb = i >> 2, c = i & 3;
    // column c of H_F: (-1)^popcount(k & c) inside c's sub-block, 0 outside
    auto hf = [&](int k) {
      return (k & ~SUB) == (c & ~SUB) ? ((__builtin_popcount(k & c & SUB) & 1) ? -1.f : 1.f) : 0.f;
    };
    const float4 e = make_float4(hf(0), hf(1), hf(2), hf(3));
    float4 col = block_fwd<VARIANT>(e, params, gb);
    if (SIGNED && lane_sign<D / 32>(gb >> 3) < 0.f) col = make_float4(-col.x, -col.y, -col.z, -col.w);
    qm[gb & 7][c][gb >> 3] = col;
  }
}

// m0..m3: the columns
template <int VARIANT>
__device__ __forceinline__ float4 mat_vec(float4 m0, float4 m1, float4 m2, float4 m3, float4 v) {
  float4 t;
  if constexpr (VARIANT == kPlanar) {   // two 2x2 diagonal blocks
    t.x = fmaf(m1.x, v.y, m0.x * v.x);
    t.y = fmaf(m1.y, v.y, m0.y * v.x);
    t.z = fmaf(m3.z, v.w, m2.z * v.z);
    t.w = fmaf(m3.w, v.w, m2.w * v.z);
    return t;
  }
  t.x = fmaf(m3.x, v.w, fmaf(m2.x, v.z, fmaf(m1.x, v.y, m0.x * v.x)));
  t.y = fmaf(m3.y, v.w, fmaf(m2.y, v.z, fmaf(m1.y, v.y, m0.y * v.x)));
  t.z = fmaf(m3.z, v.w, fmaf(m2.z, v.z, fmaf(m1.z, v.y, m0.z * v.x)));
  t.w = fmaf(m3.w, v.w, fmaf(m2.w, v.z, fmaf(m1.w, v.y, m0.w * v.x)));
  return t;
}

__device__ __forceinline__ float dot4(float4 a, float4 b) {
  return fmaf(a.w, b.w, fmaf(a.z, b.z, fmaf(a.y, b.y, a.x * b.x)));
}

// transpose of the matrix with columns m0..m3, times v
template <int VARIANT>
__device__ __forceinline__ float4 mat_t_vec(float4 m0, float4 m1, float4 m2, float4 m3, float4 v) {
  if constexpr (VARIANT == kPlanar)
    return make_float4(fmaf(m0.y, v.y, m0.x * v.x), fmaf(m1.y, v.y, m1.x * v.x), fmaf(m2.w, v.w, m2.z * v.z),
                       fmaf(m3.w, v.w, m3.z * v.z));
  return make_float4(dot4(m0, v), dot4(m1, v), dot4(m2, v), dot4(m3, v));
}

template <int D, int BITS, int VARIANT, typename TIn>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantArgs a) {
  constexpr int LPV = D / 32;            // lanes per vector
  constexpr int VPW = 64 / LPV;          // vectors per wave
  constexpr int VPB = VPW * (kThreads / 64);
  constexpr int NLEV = 1 << BITS;
  constexpr int ROWB = D * BITS / 8;     // packed row bytes
  const int h = blockIdx.y;
  const AppendTensor &T = a.t[blockIdx.z];

  __shared__ BlockMatrices<LPV> qm;      // block rotation matrices of this head
  __shared__ uint2 cells[kMaxCells];
  load_block_matrices<D, VARIANT, true>(qm, T.quats + (size_t)h * (D / 4) * block_param_floats(VARIANT));
  static_assert(kMaxCells <= kThreads, "one cell per thread");
  if ((int)threadIdx.x < a.cells.n) cells[threadIdx.x] = a.cells.e[threadIdx.x];
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane % LPV;
  const long long nvec = (long long)a.batch * a.n;   // < 2^31 (checked by the host)
  const int n = a.n;
  const int stride = (int)gridDim.x * VPB;
  const int sq = stride / n, sr = stride - sq * n;
  // Lanes past the last vector (b >= batch) work on vector 0 instead and store
  // what its own lanes store, so that every memory access is unconditional.
  auto clamp = [&](const VecPos &p, int &b, int &t) {
    const bool ok = p.b < a.batch;
    b = ok ? p.b : 0;
    t = ok ? p.t : 0;
  };
  // input and append position of the vector at p
  auto fetch = [&](const VecPos &p, TIn (&x)[32], int &sp) {
    int b, t;
    clamp(p, b, t);
    IO<TIn>::load32(static_cast<const TIn *>(T.x) + ((size_t)(b * n + t) * a.hkv + h) * a.x_stride + 32 * j, x);
    sp = a.start_pos[b];
  };
  // Workgroups stride over the vectors of one head, so the tables above are
  // built once per workgroup.  The next vector's loads are issued before this
  // one's stores (a load issued after a store cannot be waited for alone), and
  // no branch skips a store or a load, so that the waits stay exact.
  VecPos cur, nxt;
  cur.init((int)blockIdx.x * VPB + wave * VPW + lane / LPV, n);
  nxt = cur;
  nxt.advance(sq, sr, n);
  // One vector (input xin, append position sp) at cur; the next one's loads
  // go to the other buffer before this one's stores.
  auto body = [&](const TIn (&xin)[32], const int sp) {

    // s = ||x||_2 (fp32 sum of squares: four interleaved partial sums per
    // lane, then a tree over the vector's lanes)
    float sp4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 32; ++k) sp4[k & 3] = fmaf((float)xin[k], (float)xin[k], sp4[k & 3]);
    float ss = (sp4[0] + sp4[1]) + (sp4[2] + sp4[3]);
#pragma unroll
    for (int m = 1; m < LPV; m <<= 1) ss += shfl_xor(ss, m);
    // the hardware square root and reciprocal (within an ulp or so): the norm
    // is rounded to fp16 anyway, and codes are exact only up to the fp32
    // rounding of the transform
    const float s = __builtin_amdgcn_sqrtf(ss);
    // x^ = x / s folded with the 1/sqrt(d) of the normalised transform
    const float inv = s > 0.f ? __builtin_amdgcn_rcpf(s * sqrtf((float)D)) : 0.f;
    float r[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) r[k] = (float)xin[k] * inv;

    wht_butterflies<LPV, (1 << fold_stages(VARIANT))>(r, j);

    // block rotations after the folded butterflies; the matrices carry the
    // butterflies' lane sign
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      float4 t = mat_vec<VARIANT>(qm[blk][0][j], qm[blk][1][j], qm[blk][2][j], qm[blk][3][j],
                         make_float4(r[4 * blk], r[4 * blk + 1], r[4 * blk + 2], r[4 * blk + 3]));
      r[4 * blk] = t.x;
      r[4 * blk + 1] = t.y;
      r[4 * blk + 2] = t.z;
      r[4 * blk + 3] = t.w;
    }

    // Lloyd-Max code = number of thresholds strictly below the value; packed
    // LSB-first: code k of this lane occupies bits BITS*k .. BITS*k+BITS-1.
    uint32_t w[BITS];
    auto pack = [&](auto code_of) {
#pragma unroll
      for (int i = 0; i < BITS; ++i) w[i] = 0u;
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const uint32_t code = code_of(r[k]);
        const int bit = BITS * k;
        w[bit >> 5] |= code << (bit & 31);
        if ((bit & 31) + BITS > 32) w[(bit >> 5) + 1] |= code >> (32 - (bit & 31));
      }
    };
    auto count_all = [&](float x) {
      uint32_t code = 0;
#pragma unroll
      for (int t = 0; t < NLEV - 1; ++t) code += (x > a.tab.thr[t]) ? 1u : 0u;
      return code;
    };
    if (a.cells.n > 0) {
      // One threshold test per value through the cell table.  The cell index
      // is rounded onto the integers by the fma itself (the offset holds 2^23,
      // where the fp32 spacing is 1) and read from the low bits of the clamped
      // result; the table address is those bits times 8 plus a base that
      // cancels the exponent bits modulo 2^32.
      const float cmin = 8388608.0f, cmax = 8388608.0f + (float)(a.cells.n - 1);
      const float cs = a.cells.scale, co = a.cells.offset;
      const uint32_t tbase = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)cells -
                             (0x4B000000u << 3);
      pack([&](float x) {
        const float y = __builtin_amdgcn_fmed3f(fmaf(x, cs, co), cmin, cmax);
        const uint32_t addr = (__float_as_uint(y) << 3) + tbase;
        const uint64_t e = *reinterpret_cast<const __attribute__((address_space(3))) uint64_t *>(addr);
        return (uint32_t)(e >> 32) + (x > __uint_as_float((uint32_t)e) ? 1u : 0u);
      });
    } else {
      pack(count_all);
    }

    // every lane of the vector stores the (same) norm
    int b, t;
    clamp(cur, b, t);
    const long long row = ((long long)b * a.hkv + h) * T.capacity + sp + t;
    uint32_t *dst = reinterpret_cast<uint32_t *>(T.codes + row * ROWB + 4 * BITS * j);
    if constexpr (BITS == 4) {
      *reinterpret_cast<uint4 *>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    } else if constexpr (BITS == 2) {
      *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[1]);
    } else {
#pragma unroll
      for (int i = 0; i < BITS; ++i) dst[i] = w[i];
    }
    T.norms[row] = float_to_half_bits(s);
    cur = nxt;
    nxt.advance(sq, sr, n);
  };
  // two input buffers in turn, so that no registers are copied per vector
  TIn xa[32], xb[32];
  int spa, spb;
  fetch(cur, xa, spa);
  for (long long v0 = (long long)blockIdx.x * VPB; v0 < nvec; v0 += 2 * (long long)stride) {
    fetch(nxt, xb, spb);
    body(xa, spa);
    if (v0 + stride >= nvec) break;
    fetch(nxt, xa, spa);
    body(xb, spb);
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

  // output staging: each lane's 32 values (one padded segment per lane, so
  // the segment writes do not collide in LDS banks), read back in output
  // order so that a store instruction writes whole contiguous rows
  constexpr int SZ = (int)sizeof(TOut);
  constexpr int CPL = 32 * SZ / 16;        // 16-byte chunks per lane
  constexpr int SEGP = 32 * SZ + 16;       // padded segment bytes
  constexpr int CPV = D * SZ / 16;         // chunks per output row
  __shared__ uint4 obuf[kThreads / 64][64 * SEGP / 16];

  __shared__ BlockMatrices<LPV> qm;
  __shared__ float cent[NLEV];
  load_block_matrices<D, VARIANT, false>(qm, a.quats + (size_t)h * (D / 4) * block_param_floats(VARIANT));
  if (threadIdx.x < NLEV) cent[threadIdx.x] = a.tab.cent[threadIdx.x];
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane % LPV;
  const long long nvec = (long long)a.batch * a.n;   // < 2^31 (checked by the host)
  const int n = a.n;
  const int stride = (int)gridDim.x * VPB;
  const int sq = stride / n, sr = stride - sq * n;
  // Lanes past the last vector (b >= batch) work on vector 0 instead and store
  // what its own lanes store, so that every memory access is unconditional.
  auto clamp = [&](const VecPos &p, int &b, int &t) {
    const bool ok = p.b < a.batch;
    b = ok ? p.b : 0;
    t = ok ? p.t : 0;
  };
  // codes and norm of the vector at p, its batch's append position being sp
  auto fetch = [&](const VecPos &p, int sp, uint32_t (&w)[BITS], uint16_t &nb) {
    int b, t;
    clamp(p, b, t);
    const long long row = ((long long)b * a.hkv + h) * a.capacity + sp + t;
    const uint32_t *src = reinterpret_cast<const uint32_t *>(a.codes + row * ROWB + 4 * BITS * j);
#pragma unroll
    for (int i = 0; i < BITS; ++i) w[i] = src[i];
    nb = a.norms[row];
  };
  auto position = [&](const VecPos &p) {
    int b, t;
    clamp(p, b, t);
    return a.start_pos[b];
  };
  // Workgroups stride over the vectors of one head, so the tables above are
  // built once per workgroup.  Loads run ahead of the stores (a load issued
  // after a store cannot be waited for alone): the codes one vector ahead,
  // the append position, which the codes' address needs, two ahead.  No
  // branch skips a load or a store, so that the waits stay exact.
  VecPos p0, p1, p2;                         // this vector, the next, the one after
  p0.init((int)blockIdx.x * VPB + wave * VPW + lane / LPV, n);
  p1 = p0;
  p1.advance(sq, sr, n);
  p2 = p1;
  p2.advance(sq, sr, n);
  uint32_t wn[BITS];
  uint16_t nn;
  fetch(p0, position(p0), wn, nn);
  int spn = position(p1);
  for (long long v0 = (long long)blockIdx.x * VPB; v0 < nvec; v0 += stride) {
    uint32_t w[BITS];
#pragma unroll
    for (int i = 0; i < BITS; ++i) w[i] = wn[i];
    const float s16 = half_bits_to_float(nn);
    fetch(p1, spn, wn, nn);
    spn = position(p2);

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
      float4 u = mat_t_vec<VARIANT>(qm[blk][0][j], qm[blk][1][j], qm[blk][2][j], qm[blk][3][j],
                           make_float4(r[4 * blk], r[4 * blk + 1], r[4 * blk + 2], r[4 * blk + 3]));
      r[4 * blk] = u.x;
      r[4 * blk + 1] = u.y;
      r[4 * blk + 2] = u.z;
      r[4 * blk + 3] = u.w;
    }

    wht_butterflies<LPV, (1 << fold_stages(VARIANT))>(r, j);

    const float scale = lane_sign<LPV>(j) * s16 / sqrtf((float)D);
#pragma unroll
    for (int k = 0; k < 32; ++k) r[k] *= scale;

    int b, t;
    clamp(p0, b, t);
    const int f = b * n + t;                 // row of the output
    char *seg = reinterpret_cast<char *>(obuf[wave]) + lane * SEGP;
    // (the asm statements keep the compiler from moving LDS accesses across
    // them; one wave's LDS accesses complete in issue order)
    asm volatile("" ::: "memory");
    IO<TOut>::store32(reinterpret_cast<TOut *>(seg), r);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = 64 * i + lane;           // chunk of the wave's rows, in output order
      const int src = c / CPL;               // the lane that computed it
      const uint4 val = *reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(obuf[wave]) +
                                                         src * SEGP + 16 * (c % CPL));
      const int frow = __shfl(f, (src / LPV) * LPV, 64);
      char *dst = static_cast<char *>(a.out) + ((size_t)frow * a.hkv + h) * (D * SZ) + 16 * (c % CPV);
      *reinterpret_cast<uint4 *>(dst) = val;
    }
    asm volatile("" ::: "memory");
    p0 = p1;
    p1 = p2;
    p2.advance(sq, sr, n);
  }
}

// RoPE coordinates (the last r of each input vector) to the fp16 side cache,
// 8 coordinates (16 output bytes) per thread, grid-stride.
template <typename TIn>
__global__ __launch_bounds__(kThreads) void rope_copy_kernel(RopeArgs a) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  const int cpv = a.r / 8;                                   // chunks per vector
  const long long total = (long long)a.batch * a.n * a.hkv * cpv;
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (long long)gridDim.x * kThreads) {
    const int c = (int)(i % cpv);
    const long long v = i / cpv;                             // (b * n + t) * hkv + h
    const int h = (int)(v % a.hkv);
    const long long bt = v / a.hkv;
    const int t = (int)(bt % a.n), b = (int)(bt / a.n);
    const TIn *src = static_cast<const TIn *>(a.x) + v * (a.d + a.r) + a.d + 8 * c;
    h8 o;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = static_cast<_Float16>(src[k]);
    const long long row = ((long long)b * a.hkv + h) * a.capacity + a.start_pos[b] + t;
    *reinterpret_cast<h8 *>(a.out + row * a.r + 8 * c) = o;
  }
}

// Workgroups per head (and tensor): one per VPB vectors, at most about 2048
// in all (8 per compute unit), each then looping over its share.
unsigned stage1_groups(long long nvec, int vpb, int heads) {
  long long g = (nvec + vpb - 1) / vpb;
  const long long cap = (2048 + heads - 1) / heads;
  if (g > cap) g = cap;
  return (unsigned)(g < 1 ? 1 : g);
}

template <int D, int BITS, int VARIANT>
hipError_t quantize_dispatch_io(int in_f16, const QuantArgs &a, hipStream_t s) {
  constexpr int VPB = (64 / (D / 32)) * (kThreads / 64);
  const long long nvec = (long long)a.batch * a.n;
  dim3 grid(stage1_groups(nvec, VPB, a.hkv * a.ntens), (unsigned)a.hkv, (unsigned)a.ntens);
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
  dim3 grid(stage1_groups(nvec, VPB, a.hkv), (unsigned)a.hkv);
  if (out_f16)
    hipLaunchKernelGGL((dequantize_kernel<D, BITS, VARIANT, _Float16>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((dequantize_kernel<D, BITS, VARIANT, float>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D, int BITS>
hipError_t quantize_dispatch_variant(int variant, int in_f16, const QuantArgs &a, hipStream_t s) {
  switch (variant) {
    case 0: return quantize_dispatch_io<D, BITS, 0>(in_f16, a, s);
    case 1: return quantize_dispatch_io<D, BITS, 1>(in_f16, a, s);
    case kPlanar: return quantize_dispatch_io<D, BITS, kPlanar>(in_f16, a, s);
  }
  return hipErrorInvalidValue;
}

template <int D, int BITS>
hipError_t dequantize_dispatch_variant(int variant, int out_f16, const DequantArgs &a, hipStream_t s) {
  switch (variant) {
    case 0: return dequantize_dispatch_io<D, BITS, 0>(out_f16, a, s);
    case 1: return dequantize_dispatch_io<D, BITS, 1>(out_f16, a, s);
    case kPlanar: return dequantize_dispatch_io<D, BITS, kPlanar>(out_f16, a, s);
  }
  return hipErrorInvalidValue;
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

hipError_t launch_rope_copy(int in_f16, const RopeArgs &a, hipStream_t s) {
  const long long chunks = (long long)a.batch * a.n * a.hkv * (a.r / 8);
  long long g = (chunks + kThreads - 1) / kThreads;
  if (g > 2048) g = 2048;
  if (in_f16)
    hipLaunchKernelGGL((rope_copy_kernel<_Float16>), dim3((unsigned)g), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((rope_copy_kernel<float>), dim3((unsigned)g), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

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
