// Internal interface between the C-ABI layer (api.cpp) and the HIP kernels.
// Not installed; the public interface is include/iq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_args.h"
#include "iq.h"

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

// One tensor of an append: its input, rotation and cache.
struct AppendTensor {
  const void *x;           // [batch][n][H_kv][x_stride], the first d of each vector quantised
  const float *quats;      // [H_kv][d/4][2][4] (Full, Fast) or [H_kv][d/2][2] (Planar)
  uint8_t *codes;          // [batch][H_kv][cap][row]
  uint16_t *norms;         // [batch][H_kv][cap]
  long long capacity;
};

// Tensors one quantize launch takes (grid z); each shares the shape, the
// codebook and the append positions.
constexpr int kMaxAppendTensors = 16;

struct QuantArgs {
  AppendTensor t[kMaxAppendTensors];
  int ntens;
  const int32_t *start_pos;
  int batch, n, hkv;
  int x_stride;            // elements from one input vector to the next (d, or d + RoPE coordinates)
  Tables tab;
  CellTable cells;
};

// The RoPE coordinates of the keys, copied unrotated and unquantised (fp16).
struct RopeArgs {
  const void *x;           // [batch][n][H_kv][d + r]
  const int32_t *start_pos;
  uint16_t *out;           // [batch][H_kv][cap][r] fp16 bits
  long long capacity;
  int batch, n, hkv, d, r;
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

// Launchers (return hipSuccess or the launch error).
hipError_t launch_quantize(int d, int bits, int variant, int in_f16, const QuantArgs &a,
                           hipStream_t s);
hipError_t launch_dequantize(int d, int bits, int variant, int out_f16, const DequantArgs &a,
                             hipStream_t s);
hipError_t launch_rope_copy(int in_f16, const RopeArgs &a, hipStream_t s);
hipError_t launch_decode(int d, int bits, const DecodeArgs &a, hipStream_t s);
hipError_t launch_merge(int d, int variant, const MergeArgs &a, hipStream_t s);
// Validation of the decode sizes shared by every decode entry point: the
// status iq_decode_attention would return for them, and the workspace bytes
// they need.
int decode_workspace_check(const iq_config *cfg, int32_t batch, int32_t num_q_heads, int64_t max_kv_len,
                           size_t *need);
// Workgroups of the partial (split) kernel one compute unit holds at once.
int decode_groups_per_cu(int d, int bits, int rope);

}  // namespace iq
