// Internal interface between the C-ABI layer (api.cpp) and the HIP kernels.
// Not installed; the public interface is include/iq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iq {

constexpr int kMaxLevels = 16;  // 2^4 centroids at most

// Per-call quantiser tables, passed to kernels by value (kernel arguments).
struct Tables {
  float cent[kMaxLevels];  // ascending centroids (fp32, as given by the caller)
  float thr[kMaxLevels];   // thr[k] = (cent[k] + cent[k+1]) / 2, k < 2^b - 1
};

// Lloyd-Max code lookup: a monotone cell index
// c(x) = clamp(fma(x, scale, offset), 2^23, 2^23 + n - 1) - 2^23 over n cells
// (offset includes 2^23, so the fp32 fma rounds onto the integers), each cell
// holding at most one threshold: entry c = (bits of that threshold, or of
// +inf; number of thresholds whose cell is below c).  The code of x is then
// entry.y + (x > entry.x) -- the same count of thresholds strictly below x.
// n = 0: no such table (thresholds too close); the kernel counts directly.
constexpr int kMaxCells = 256;
struct CellTable {
  float scale, offset;
  int n;
  int pad_;
  uint2 e[kMaxCells];
};

struct QuantArgs {
  const void *x;           // [batch][n][H_kv][d]
  const float *quats;      // [H_kv][d/4][2][4]
  const int32_t *start_pos;
  uint8_t *codes;          // [batch][H_kv][cap][row]
  uint16_t *norms;         // [batch][H_kv][cap]
  long long capacity;
  int batch, n, hkv;
  Tables tab;
  CellTable cells;
};

struct DequantArgs {
  const uint8_t *codes;
  const uint16_t *norms;
  const float *quats;
  const int32_t *start_pos;
  void *out;               // [batch][n][H_kv][d]
  long long capacity;
  int batch, n, hkv;
  Tables tab;
};

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

// Launchers (return hipSuccess or the launch error).
hipError_t launch_quantize(int d, int bits, int variant, int in_f16, const QuantArgs &a,
                           hipStream_t s);
hipError_t launch_dequantize(int d, int bits, int variant, int out_f16, const DequantArgs &a,
                             hipStream_t s);
hipError_t launch_decode(int d, int bits, const DecodeArgs &a, hipStream_t s);
hipError_t launch_merge(int d, int variant, const MergeArgs &a, hipStream_t s);

}  // namespace iq
