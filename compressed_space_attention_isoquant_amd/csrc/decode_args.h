// Arguments and constants of the decode kernels, shared by the C-ABI layer
// and the kernels.  Not installed; the public interface is include/iq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

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
constexpr int kDecodeRope = 64;            // RoPE coordinates per key the decode kernels take (head_dim 128)

struct DecodeArgs {
  const void *q;           // [batch][Hq][d + rope]
  int q_f16;
  const uint16_t *krope;   // [batch][H_kv][kcap][rope] fp16 RoPE coordinates of the keys (rope > 0)
  int rope;                // RoPE coordinates per key and query (0: none)
  float rmul;              // softmax_scale * log2(e), applied to the query's RoPE part
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
  // Nullable.  Entry P (workgroup (kvh, P mod batch, P / batch)) holds the
  // (sequence, split) it processes, (split << 16 | sequence, kv_len), in
  // longest-first order of the splits' token counts.
  int2 *order;
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

// Workspace of the decode path: the split records, then (256-byte aligned)
// the workgroup order when batch * n_split is at most kMaxOrderedPairs.
constexpr int kMaxOrderedPairs = 4096;

inline size_t decode_record_bytes(int32_t batch, int32_t hq, int n_split, int d) {
  return (size_t)batch * hq * n_split * (d + kRecHeader) * sizeof(float);
}
inline size_t decode_order_offset(int32_t batch, int32_t hq, int n_split, int d) {
  return (decode_record_bytes(batch, hq, n_split, d) + 255) / 256 * 256;
}
inline bool decode_ordered(int32_t batch, int n_split) {
  return (int64_t)batch * n_split <= kMaxOrderedPairs;
}
inline size_t decode_workspace_total(int32_t batch, int32_t hq, int n_split, int d) {
  return decode_ordered(batch, n_split)
             ? decode_order_offset(batch, hq, n_split, d) + (size_t)batch * n_split * sizeof(int2)
             : decode_record_bytes(batch, hq, n_split, d);
}

// Split-K geometry of the decode kernels.  About 2048 workgroups (8 per
// compute unit, two resident at a time): with ragged context lengths the
// extra, shorter workgroups even out the compute units' loads.  Chunks are
// kept at 8192 tokens or more while that still gives 512 workgroups (about
// one resident round), since each workgroup costs a fixed prologue and
// epilogue: a few long sequences then run in one round of workgroups instead
// of several rounds of one-tile ones.  Chunks are whole numbers of
// (waves x tile) token blocks.
struct Geometry {
  int chunk;
  int n_split;
};

inline Geometry decode_geometry(int32_t batch, int32_t hkv, int64_t max_kv_len) {
  const int64_t unit = (int64_t)kDecodeWaves * kDecodeStep;
  const int64_t T = max_kv_len > 0 ? max_kv_len : 1;
  const int64_t pairs = (int64_t)batch * hkv;
  auto chunk_for = [&](int64_t groups) {
    int64_t want = (groups + pairs - 1) / pairs;
    if (want < 1) want = 1;
    return (T + want - 1) / want;
  };
  int64_t chunk = chunk_for(2048);
  const int64_t floor_chunk = std::min<int64_t>(8192, chunk_for(512));
  if (chunk < floor_chunk) chunk = floor_chunk;
  chunk = (chunk + unit - 1) / unit * unit;
  Geometry g;
  g.chunk = (int)chunk;
  g.n_split = (int)((T + chunk - 1) / chunk);
  return g;
}

}  // namespace iq
