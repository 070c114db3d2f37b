// Arguments and constants of the decode kernels, shared by the C-ABI layer
// and the kernels.  Not installed; the public interface is include/iq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iq {

// Split-K decode.  Each workgroup (4 waves) of the partial kernel covers
// `chunk` tokens of one (sequence, KV head) and writes one record per query
// head: running max M (log2 units, biased by the value-norm exponent), the
// softmax denominator L, the best score and its position, and the unnormalised
// rotated-space output o~[d].  The merge kernel combines the records of a
// (sequence, query head) and applies R^T once.
constexpr int kDecodeWaves = 4;            // waves per partial workgroup
constexpr int kDecodeStep = 32;            // tokens per wave iteration
constexpr int kRecHeader = 4;              // M, L, best score, best position
constexpr float kLazyTau = 4.0f;           // rescale only when the max grows by more than this
constexpr float kWeightBias = 25.0f;       // weights 2^(s - M + bias) * ||v|| stay below 2^15

struct DecodeArgs {
  const void *q;           // [batch][Hq][d]
  int q_f16;
  const uint8_t *kc;
  const uint16_t *kn;
  const uint8_t *vc;
  const uint16_t *vn;
  long long kcap, vcap;
  const int32_t *kv_len;
  const float *quats;
  int batch, hq, hkv, group;
  int variant;
  int chunk;               // tokens per workgroup (multiple of kDecodeWaves * kDecodeStep)
  int n_split;             // workgroups per (sequence, KV head)
  float qmul;              // softmax_scale * log2(e) / 2^cexp, applied to R q
  int argmax;              // track the position of the largest score
  float *ws;               // records [batch][Hq][n_split][d + kRecHeader]
  uint32_t lut[256];       // fp16 pairs (c_i 2^cexp | c_k 2^cexp << 16) at index i | k << bits
};

struct MergeArgs {
  const float *ws;
  const float *quats;
  void *out;               // [batch][Hq][d]
  int out_f16;
  float *lse;              // nullable
  int32_t *argmax;         // nullable
  int batch, hq, group;
  int n_part;              // records per (sequence, query head)
  float oscale;            // 2^-cexp
};

// Split-K geometry of the decode kernels: enough workgroups to cover the
// 256 compute units several times, each holding a whole number of
// (waves x tile) token blocks.
struct Geometry {
  int chunk;
  int n_split;
};

inline Geometry decode_geometry(int32_t batch, int32_t hkv, int64_t max_kv_len) {
  const int64_t unit = (int64_t)kDecodeWaves * kDecodeStep;
  const int64_t T = max_kv_len > 0 ? max_kv_len : 1;
  const int64_t pairs = (int64_t)batch * hkv;
  const int64_t target_groups = 1024;     // 4 resident workgroups on each of 256 CUs
  int64_t want = (target_groups + pairs - 1) / pairs;
  if (want < 1) want = 1;
  int64_t chunk = (T + want - 1) / want;
  chunk = (chunk + unit - 1) / unit * unit;
  Geometry g;
  g.chunk = (int)chunk;
  g.n_split = (int)((T + chunk - 1) / chunk);
  return g;
}

}  // namespace iq
