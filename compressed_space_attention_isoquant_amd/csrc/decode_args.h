// Arguments and constants of the decode kernels, shared by the C-ABI layer
// and the kernels.  Not installed; the public interface is include/iq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace iq {

// Decode attention runs in three launches:
//
// prep    one workgroup per (sequence, KV head) rotates its queries: q~ =
//         R q, scaled, split into fp16 hi + lo parts (the score product's
//         operand), in the workspace; the work plan (below) is computed by
//         every one of them for up to 256 (sequence, KV head) pairs, each
//         writing its share of it, else by one extra workgroup.
// partial every wave streams its own equal share of the 32-token tiles of all
//         (sequence, KV head) segments laid end to end (tiles of sequence b,
//         KV head 0 first, then KV head 1, ..., then sequence b + 1), so that
//         ragged lengths cost no imbalance.  Where a wave's share crosses a
//         segment boundary it writes one record per piece: running max M
//         (log2 units, biased by the value-norm exponent), softmax denominator
//         L, best score and its position, and the unnormalised rotated-space
//         output o~[d], per query head of the group.
// merge   one workgroup per (sequence, query head) combines the records of
//         its segment's pieces and applies R^T once.
//
// Pieces: tile range [w W, (w + 1) W) of wave w meets segment s in at most one
// piece, stored as record s + w (distinct for every piece that exists: if wave
// w met segment s and wave w - 1 met segment s + 1, wave w - 1 would end after
// wave w begins).  Segment s with tiles [S, S + n) has pieces for the waves
// S / W .. (S + n - 1) / W: a contiguous run of records.
constexpr int kDecodeWaves = 4;            // waves per partial workgroup
constexpr int kDecodeStep = 32;            // tokens per tile (one wave iteration)
constexpr int kRecHeader = 4;              // M, L, best score, best position
constexpr float kLazyTau = 4.0f;           // rescale only when the max grows by more than this
constexpr float kWeightBias = 25.0f;       // weights 2^(s - M + bias) * ||v|| stay below 2^15
constexpr int kDecodeRope = 64;            // RoPE coordinates per key the decode kernels take
constexpr int kMinTilesPerWave = 2;        // a wave's share is at least this many tiles
constexpr int kMaxPiecesPerSegment = 256;  // and large enough that no segment has more pieces
constexpr int kMaxDecodeWaves = 4096;      // waves of the partial launch at most (256 CUs x 16)
constexpr int kPrepThreads = 256;
static_assert(kMaxDecodeWaves % kPrepThreads == 0 && (kPrepThreads & (kPrepThreads - 1)) == 0, "plan lookup");

// Plan written by the prep kernel at the start of the workspace.
struct DecodePlan {
  int total;          // tiles of all segments
  int per_wave;       // W, tiles per wave (the last busy wave may have fewer)
  int pad_[2];
  // then: WaveShare share[kMaxDecodeWaves], and int seg_base[batch + 1]
  //       (tile index of segment (b, 0); the last entry is total, so
  //       sequence b has (seg_base[b + 1] - seg_base[b]) / H_kv tiles per KV
  //       head)
};

// Where wave w starts: segment s = b H_kv + h, tile i0 of that segment, its
// `count` tiles (0 for a wave without work), and the sequence's length.
struct WaveShare {
  int seg, i0, count, len;
};

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
  int n_waves;             // waves of the partial launch
  float qmul;              // softmax_scale * log2(e) / 2^cexp, applied to R q
  int argmax;              // track the position of the largest score
  DecodePlan *plan;        // workspace: plan header, wave shares, segment bases
  uint16_t *qrot;          // workspace: [batch][H_kv][2G][d + rope] fp16, hi rows then lo rows
  float *qscale;           // workspace: [batch][H_kv] 2^-f, the scale of the rows of q~
  float *ws;               // workspace: records [(batch H_kv + n_waves) G][d + kRecHeader]
  uint32_t lut[256];       // fp16 pairs (c_i 2^cexp | c_k 2^cexp << 16) at index i | k << bits
};

struct MergeArgs {
  const float *ws;
  const DecodePlan *plan;
  const float *quats;
  void *out;               // [batch][Hq][d]
  int out_f16;
  float *lse;              // nullable
  int32_t *argmax;         // nullable
  int batch, hq, hkv, group;
  float oscale;            // 2^-cexp
};

// Workspace layout: the plan (header, wave shares, segment bases), the
// rotated queries (sized for kDecodeRope RoPE coordinates whether or not a
// call has them), their scales (batch x Hq floats, at least batch x H_kv),
// the records; each part 256-byte aligned.
inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }
inline size_t decode_plan_bytes(int32_t batch) {
  return align256(sizeof(DecodePlan) + sizeof(WaveShare) * kMaxDecodeWaves + sizeof(int) * ((size_t)batch + 1));
}
inline size_t decode_qrot_bytes(int32_t batch, int32_t hq, int d, int rope) {
  return align256((size_t)batch * hq * 2 * (d + rope) * sizeof(uint16_t));
}
inline size_t decode_record_bytes(int32_t batch, int32_t hkv, int32_t hq, int d) {
  const int group = hq / hkv;
  return ((size_t)batch * hkv + kMaxDecodeWaves) * group * (d + kRecHeader) * sizeof(float);
}
inline size_t decode_qrot_offset(int32_t batch) { return decode_plan_bytes(batch); }
inline size_t decode_qscale_offset(int32_t batch, int32_t hq, int d) {
  return decode_qrot_offset(batch) + decode_qrot_bytes(batch, hq, d, kDecodeRope);
}
inline size_t decode_record_offset(int32_t batch, int32_t hq, int d) {
  return decode_qscale_offset(batch, hq, d) + align256((size_t)batch * hq * sizeof(float));
}
inline size_t decode_workspace_total(int32_t batch, int32_t hkv, int32_t hq, int d) {
  return decode_record_offset(batch, hq, d) + decode_record_bytes(batch, hkv, hq, d);
}

}  // namespace iq
