// Compressed-space decode attention (RotaryQuant §3.4 Table 2, Appendix A).
//
// attention kernel: one workgroup per (split, KV head, sequence).  Its
//   prologue rotates the G query heads of the group once (q~ = R q, with
//   softmax_scale * log2(e) folded in).  Each of its waves walks its share of
//   the split in tiles of 64 tokens: scores of the G heads on the packed K rows
//   (lane = token), online base-2 softmax, then value accumulation on the
//   packed V rows staged in LDS (lane = output dimension).  Every wave writes
//   one partial state (m, l, argmax, o~[d]) per query head.
// merge kernel: one workgroup per (query head, sequence): merges the partial
//   states, divides by the softmax denominator and applies R^T once.
#include "iq_device.h"
#include "iq_internal.h"

namespace iq {
namespace {

constexpr int kThreads = kDecodeWaves * 64;

template <int BITS>
__device__ __forceinline__ uint32_t code_at(const uint32_t *row, int e) {
  const int bit = BITS * e;
  const int wd = bit >> 5;
  const int off = bit & 31;
  uint32_t c = row[wd] >> off;
  if (off + BITS > 32) c |= row[wd + 1] << (32 - off);
  return c & ((1u << BITS) - 1u);
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <int D, int BITS, int G>
__global__ __launch_bounds__(kThreads) void attention_kernel(DecodeArgs a) {
  constexpr int NLEV = 1 << BITS;
  constexpr int ROWW = D * BITS / 32;   // dwords per packed row
  constexpr int DPL = D / 64;           // output dimensions per lane
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int T = a.kv_len[b];

  __shared__ float qtmp[G][D];
  __shared__ float qt[D][G];
  __shared__ float cent[NLEV];
  __shared__ uint32_t vrow[kDecodeWaves][kDecodeTile][ROWW + 1];
  __shared__ float pw[kDecodeWaves][kDecodeTile][G];

  // ---- prologue: q~ = R q for the G query heads of this KV head -------------
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int hh = idx / D, i = idx % D;
    const size_t off = ((size_t)b * a.hq + g * G + hh) * D + i;
    qtmp[hh][i] = a.q_f16 ? static_cast<float>(static_cast<const _Float16 *>(a.q)[off])
                          : static_cast<const float *>(a.q)[off];
  }
  if (threadIdx.x < NLEV) cent[threadIdx.x] = a.tab.cent[threadIdx.x];
  __syncthreads();
  for (int st = 1; st < D; st <<= 1) {
    for (int p = threadIdx.x; p < G * D / 2; p += kThreads) {
      const int hh = p / (D / 2), pp = p % (D / 2);
      const int i = (pp / st) * 2 * st + (pp % st);
      const float x0 = qtmp[hh][i], x1 = qtmp[hh][i + st];
      qtmp[hh][i] = x0 + x1;
      qtmp[hh][i + st] = x0 - x1;
    }
    __syncthreads();
  }
  {
    const float scale = a.qscale / sqrtf((float)D);
    const float4 *qg = reinterpret_cast<const float4 *>(a.quats) + (size_t)g * (D / 4) * 2;
    for (int p = threadIdx.x; p < G * D / 4; p += kThreads) {
      const int hh = p / (D / 4), blk = p % (D / 4);
      float4 v = make_float4(qtmp[hh][4 * blk] * scale, qtmp[hh][4 * blk + 1] * scale,
                             qtmp[hh][4 * blk + 2] * scale, qtmp[hh][4 * blk + 3] * scale);
      const float4 qL = qg[2 * blk], qR = qg[2 * blk + 1];
      float4 t = a.variant == 0 ? so4_fwd<0>(v, qL, qR) : so4_fwd<1>(v, qL, qR);
      qt[4 * blk][hh] = t.x;
      qt[4 * blk + 1][hh] = t.y;
      qt[4 * blk + 2][hh] = t.z;
      qt[4 * blk + 3][hh] = t.w;
    }
  }
  __syncthreads();

  // ---- main loop over this wave's tokens -------------------------------------
  const int sub = a.chunk / kDecodeWaves;
  const int begin = split * a.chunk + wave * sub;
  const int end = min(T, begin + sub);
  const long long headrow = (long long)b * a.hkv + g;
  const uint32_t *kbase = reinterpret_cast<const uint32_t *>(a.kc) + headrow * a.kcap * ROWW;
  const uint32_t *vbase = reinterpret_cast<const uint32_t *>(a.vc) + headrow * a.vcap * ROWW;
  const uint16_t *knb = a.kn + headrow * a.kcap;
  const uint16_t *vnb = a.vn + headrow * a.vcap;

  float m[G], l[G], bs[G], acc[G][DPL];
  int bj[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
    bs[h] = -INFINITY;
    bj[h] = -1;
#pragma unroll
    for (int r = 0; r < DPL; ++r) acc[h][r] = 0.f;
  }

  for (int t0 = begin; t0 < end; t0 += kDecodeTile) {
    const int j = t0 + lane;
    const bool valid = j < end;
    const int jr = valid ? j : t0;
    uint32_t kw[ROWW];
#pragma unroll
    for (int i = 0; i < ROWW; ++i) kw[i] = kbase[(long long)jr * ROWW + i];
    float sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sc[h] = 0.f;
#pragma unroll 4
    for (int e = 0; e < D; ++e) {
      const float c = cent[code_at<BITS>(kw, e)];
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h] = fmaf(qt[e][h], c, sc[h]);
    }
    const float kn = half_bits_to_float(knb[jr]);
    const float vn = half_bits_to_float(vnb[jr]);
#pragma unroll
    for (int i = 0; i < ROWW; ++i) vrow[wave][lane][i] = vbase[(long long)jr * ROWW + i];

#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float s = valid ? sc[h] * kn : -INFINITY;
      const float mnew = fmaxf(m[h], wave_max(s));
      const float alpha = exp2f(m[h] - mnew);      // m = -inf -> 0
      const float p = valid ? exp2f(s - mnew) : 0.f;
      l[h] = l[h] * alpha + p;
#pragma unroll
      for (int r = 0; r < DPL; ++r) acc[h][r] *= alpha;
      m[h] = mnew;
      if (valid && s > bs[h]) {
        bs[h] = s;
        bj[h] = j;
      }
      pw[wave][lane][h] = p * vn;
    }
    wave_sync();

    const int nt = min(kDecodeTile, end - t0);
    for (int jj = 0; jj < nt; ++jj) {
      const uint32_t *row = vrow[wave][jj];
      float pv[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pv[h] = pw[wave][jj][h];
#pragma unroll
      for (int r = 0; r < DPL; ++r) {
        const float c = cent[code_at<BITS>(row, lane + 64 * r)];
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h][r] = fmaf(pv[h], c, acc[h][r]);
      }
    }
    wave_sync();
  }

  // ---- this wave's partial state ---------------------------------------------
  const int n_part = a.n_split * kDecodeWaves;
  const int part = split * kDecodeWaves + wave;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float lsum = wave_sum(l[h]);
    float s = bs[h];
    int jj = bj[h];
#pragma unroll
    for (int msk = 32; msk >= 1; msk >>= 1) {
      const float os = __shfl_xor(s, msk, 64);
      const int oj = __shfl_xor(jj, msk, 64);
      if (os > s || (os == s && oj >= 0 && (jj < 0 || oj < jj))) {
        s = os;
        jj = oj;
      }
    }
    float *rec = a.ws + (((size_t)b * a.hq + g * G + h) * n_part + part) * (D + kRecHeader);
    if (lane == 0) {
      rec[0] = m[h];
      rec[1] = lsum;
      rec[2] = __builtin_bit_cast(float, jj);
      rec[3] = 0.f;
    }
#pragma unroll
    for (int r = 0; r < DPL; ++r) rec[kRecHeader + lane + 64 * r] = acc[h][r];
  }
}

template <int D, int VARIANT>
__global__ __launch_bounds__(D) void merge_kernel(MergeArgs a) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int g = h / a.group;
  const int i = threadIdx.x;
  const float *recs = a.ws + ((size_t)b * a.hq + h) * a.n_part * (D + kRecHeader);

  float M = -INFINITY;
  for (int p = 0; p < a.n_part; ++p) {
    const float *rec = recs + (size_t)p * (D + kRecHeader);
    if (rec[1] > 0.f) M = fmaxf(M, rec[0]);
  }
  float L = 0.f, o = 0.f;
  int arg = -1;
  for (int p = 0; p < a.n_part; ++p) {
    const float *rec = recs + (size_t)p * (D + kRecHeader);
    const float lp = rec[1];
    if (lp > 0.f) {
      const float w = exp2f(rec[0] - M);
      L += lp * w;
      o += rec[kRecHeader + i] * w;
      if (arg < 0 && rec[0] == M) arg = __builtin_bit_cast(int, rec[2]);
    }
  }

  __shared__ float y[D];
  y[i] = L > 0.f ? o / L : 0.f;
  __syncthreads();
  if (i < D / 4) {
    const float4 *qg = reinterpret_cast<const float4 *>(a.quats) + (size_t)g * (D / 4) * 2;
    float4 u = so4_inv<VARIANT>(make_float4(y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]),
                                qg[2 * i], qg[2 * i + 1]);
    y[4 * i] = u.x;
    y[4 * i + 1] = u.y;
    y[4 * i + 2] = u.z;
    y[4 * i + 3] = u.w;
  }
  __syncthreads();
  for (int st = 1; st < D; st <<= 1) {
    float x0 = 0.f, x1 = 0.f;
    int lo = 0;
    if (i < D / 2) {
      lo = (i / st) * 2 * st + (i % st);
      x0 = y[lo];
      x1 = y[lo + st];
    }
    __syncthreads();
    if (i < D / 2) {
      y[lo] = x0 + x1;
      y[lo + st] = x0 - x1;
    }
    __syncthreads();
  }
  const float val = y[i] / sqrtf((float)D);
  const size_t off = ((size_t)b * a.hq + h) * D + i;
  if (a.out_f16)
    static_cast<_Float16 *>(a.out)[off] = static_cast<_Float16>(val);
  else
    static_cast<float *>(a.out)[off] = val;
  if (i == 0) {
    const size_t oh = (size_t)b * a.hq + h;
    if (a.lse) a.lse[oh] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
    if (a.argmax) a.argmax[oh] = L > 0.f ? arg : -1;
  }
}

template <int D, int BITS>
hipError_t decode_dispatch_group(const DecodeArgs &a, hipStream_t s) {
  dim3 grid((unsigned)a.n_split, (unsigned)a.hkv, (unsigned)a.batch);
  switch (a.group) {
    case 1: hipLaunchKernelGGL((attention_kernel<D, BITS, 1>), grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((attention_kernel<D, BITS, 2>), grid, dim3(kThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((attention_kernel<D, BITS, 4>), grid, dim3(kThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL((attention_kernel<D, BITS, 8>), grid, dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t decode_dispatch_bits(int bits, const DecodeArgs &a, hipStream_t s) {
  switch (bits) {
    case 2: return decode_dispatch_group<D, 2>(a, s);
    case 3: return decode_dispatch_group<D, 3>(a, s);
    case 4: return decode_dispatch_group<D, 4>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t merge_dispatch(int variant, const MergeArgs &a, hipStream_t s) {
  dim3 grid((unsigned)a.hq, (unsigned)a.batch);
  if (variant == 0)
    hipLaunchKernelGGL((merge_kernel<D, 0>), grid, dim3(D), 0, s, a);
  else
    hipLaunchKernelGGL((merge_kernel<D, 1>), grid, dim3(D), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(int d, int bits, const DecodeArgs &a, hipStream_t s) {
  switch (d) {
    case 128: return decode_dispatch_bits<128>(bits, a, s);
    case 256: return decode_dispatch_bits<256>(bits, a, s);
    case 512: return decode_dispatch_bits<512>(bits, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_merge(int d, int variant, const MergeArgs &a, hipStream_t s) {
  switch (d) {
    case 128: return merge_dispatch<128>(variant, a, s);
    case 256: return merge_dispatch<256>(variant, a, s);
    case 512: return merge_dispatch<512>(variant, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace iq
