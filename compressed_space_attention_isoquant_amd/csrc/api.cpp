// extern "C" entry points of libiq.so: argument validation, per-call tables,
// launch geometry and kernel dispatch.  See include/iq.h for the contract.
#include "iq.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

#include "iq_internal.h"

namespace {

using iq::Tables;

// RoPE coordinates per key: a multiple of 8 (16-byte fp16 rows) up to this;
// decode attention takes kDecodeRopeDim of them.
constexpr int32_t kMaxRopeDim = 512;
constexpr int32_t kDecodeRopeDim = 64;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_config(const iq_config *cfg) {
  if (!cfg || !cfg->quats || !cfg->centroids) return IQ_ERR_INVALID_ARG;
  if (cfg->head_dim != 128 && cfg->head_dim != 256 && cfg->head_dim != 512) return IQ_ERR_UNSUPPORTED;
  if (cfg->bits < 2 || cfg->bits > 4) return IQ_ERR_UNSUPPORTED;
  if (cfg->variant != IQ_FULL && cfg->variant != IQ_FAST && cfg->variant != IQ_PLANAR) return IQ_ERR_INVALID_ARG;
  if (cfg->num_kv_heads < 1) return IQ_ERR_INVALID_ARG;
  if (!aligned16(cfg->quats)) return IQ_ERR_MISALIGNED;
  const int n = 1 << cfg->bits;
  for (int k = 0; k < n; ++k) {
    const float c = cfg->centroids[k];
    if (!std::isfinite(c)) return IQ_ERR_INVALID_ARG;
    if (k > 0 && !(c > cfg->centroids[k - 1])) return IQ_ERR_INVALID_ARG;
  }
  return IQ_OK;
}

// Scale exponent e with max|c| * 2^e in [1, 2): the decode kernels feed the
// levels to fp16 matrix instructions as c * 2^e.
int centroid_exponent(const iq_config *cfg) {
  float hi = 0.f;
  for (int k = 0; k < (1 << cfg->bits); ++k) hi = std::fmax(hi, std::fabs(cfg->centroids[k]));
  if (hi == 0.f) return 0;
  int e = 0;
  std::frexp(hi, &e);        // hi = m 2^e, m in [0.5, 1)
  return 1 - e;
}

uint16_t fp16_bits(float x) {
  const _Float16 h = static_cast<_Float16>(x);
  uint16_t b;
  std::memcpy(&b, &h, 2);
  return b;
}

// Whether every level times 2^e (e from centroid_exponent) is an fp16 number
// exactly, so that the decode kernels attend with the same centroids the
// quantiser used.  Levels with at most 11 significant bits (what iq_codebook
// produces) pass whenever max/min nonzero magnitude is below 2^14; past that
// a level passes only if it is an exact fp16 subnormal once scaled.
bool decode_codebook_exact(const iq_config *cfg) {
  const int e = centroid_exponent(cfg);
  for (int k = 0; k < (1 << cfg->bits); ++k) {
    const float s = std::ldexp(cfg->centroids[k], e);
    const _Float16 h = static_cast<_Float16>(s);
    if (static_cast<float>(h) != s) return false;
  }
  return true;
}

// The table of fp16 pairs (c_i 2^e, c_k 2^e) at index i | k << bits; exact
// (decode_codebook_exact is checked before any decode launch).
void fill_pair_table(const iq_config *cfg, int e, uint32_t *lut) {
  const int n = 1 << cfg->bits;
  for (int i = 0; i < n; ++i)
    for (int k = 0; k < n; ++k) {
      const uint32_t lo = fp16_bits(std::ldexp(cfg->centroids[i], e));
      const uint32_t hi = fp16_bits(std::ldexp(cfg->centroids[k], e));
      lut[i | (k << cfg->bits)] = lo | (hi << 16);
    }
}

int check_cache(const iq_cache *c) {
  if (!c || !c->codes || !c->norms) return IQ_ERR_INVALID_ARG;
  if (c->capacity < 1) return IQ_ERR_INVALID_ARG;
  if (!aligned16(c->codes) || !aligned16(c->norms)) return IQ_ERR_MISALIGNED;
  return IQ_OK;
}

bool valid_dtype(int32_t t) { return t == IQ_F32 || t == IQ_F16; }

// The stage-1 kernels index the vectors of a call with 32-bit integers.
bool vector_count_ok(int32_t batch, int32_t n) {
  return static_cast<int64_t>(batch) * n < (int64_t(1) << 31) - (int64_t(1) << 20);
}

Tables make_tables(const iq_config *cfg) {
  Tables t;
  std::memset(&t, 0, sizeof(t));
  const int n = 1 << cfg->bits;
  for (int k = 0; k < n; ++k) t.cent[k] = cfg->centroids[k];
  // midpoint of neighbouring centroids, evaluated in double and rounded once
  for (int k = 0; k + 1 < n; ++k)
    t.thr[k] = static_cast<float>(0.5 * (static_cast<double>(cfg->centroids[k]) +
                                         static_cast<double>(cfg->centroids[k + 1])));
  return t;
}

// Cell index of a value exactly as the quantize kernel computes it: fp32 fma
// whose offset includes 2^23 (so the result is rounded to an integer),
// clamped to [2^23, 2^23 + n - 1].
constexpr float kCellMagic = 8388608.0f;  // 2^23
uint32_t cell_of(float x, float scale, float offset, int n) {
  float y = std::fma(x, scale, offset);
  y = std::min(std::max(y, kCellMagic), kCellMagic + static_cast<float>(n - 1));
  return static_cast<uint32_t>(y - kCellMagic);
}

// Smallest power-of-two cell table (8..kMaxCells cells) with at most one
// threshold per cell; n = 0 when none exists.
iq::CellTable make_cells(const Tables &t, int bits) {
  iq::CellTable c;
  std::memset(&c, 0, sizeof(c));
  const int nthr = (1 << bits) - 1;
  const float lo = t.thr[0], hi = t.thr[nthr - 1];
  if (!(hi > lo)) return c;
  for (int n = 8; n <= iq::kMaxCells; n *= 2) {
    const float scale = static_cast<float>(n - 1) / (hi - lo);
    const float offset = kCellMagic - lo * scale;
    if (!std::isfinite(scale) || !std::isfinite(offset)) break;
    std::vector<int> owner(n, -1);
    bool ok = true;
    for (int k = 0; k < nthr && ok; ++k) {
      const uint32_t ci = cell_of(t.thr[k], scale, offset, n);
      if (owner[ci] >= 0) ok = false;
      owner[ci] = k;
    }
    if (!ok) continue;
    uint32_t below = 0;
    for (int ci = 0; ci < n; ++ci) {
      const float th = owner[ci] >= 0 ? t.thr[owner[ci]] : std::numeric_limits<float>::infinity();
      uint32_t bitsv;
      std::memcpy(&bitsv, &th, 4);
      c.e[ci] = make_uint2(bitsv, below);
      if (owner[ci] >= 0) ++below;
    }
    c.scale = scale;
    c.offset = offset;
    c.n = n;
    return c;
  }
  return c;
}

int hip_status(hipError_t e) { return e == hipSuccess ? IQ_OK : IQ_ERR_HIP; }

// Lloyd iteration for the minimum-MSE quantiser of N(0,1): thresholds are the
// midpoints of neighbouring levels; levels are the conditional means of their
// cells, (phi(a) - phi(b)) / P(a < X <= b).
double std_normal_pdf(double x) { return std::isinf(x) ? 0.0 : std::exp(-0.5 * x * x) * 0.39894228040143267794; }

double cell_mass(double a, double b) {
  const double r2 = 0.70710678118654752440;
  if (a >= 0.0) {
    const double qa = 0.5 * std::erfc(a * r2);
    const double qb = std::isinf(b) ? 0.0 : 0.5 * std::erfc(b * r2);
    return qa - qb;
  }
  const double pb = std::isinf(b) ? 1.0 : 0.5 * std::erfc(-b * r2);
  const double pa = std::isinf(a) ? 0.0 : 0.5 * std::erfc(-a * r2);
  return pb - pa;
}

}  // namespace

extern "C" {

const char *iq_status_string(int status) {
  switch (status) {
    case IQ_OK: return "ok";
    case IQ_ERR_INVALID_ARG: return "invalid argument";
    case IQ_ERR_UNSUPPORTED:
      return "unsupported head_dim, bits, group size, dtype or shape, or (decode) a codebook whose levels "
             "are not exact fp16 numbers once scaled";
    case IQ_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case IQ_ERR_WORKSPACE: return "workspace too small";
    case IQ_ERR_HIP: return "HIP runtime or launch error";
  }
  return "unknown status";
}

int iq_codebook(int32_t bits, int32_t head_dim, float *centroids_out) {
  if (!centroids_out) return IQ_ERR_INVALID_ARG;
  if (bits < 1 || bits > 4) return IQ_ERR_UNSUPPORTED;
  if (head_dim < 1) return IQ_ERR_UNSUPPORTED;
  const int n = 1 << bits;
  double c[16], t[17];
  for (int k = 0; k < n; ++k) c[k] = -2.0 + 4.0 * k / (n - 1);
  for (int it = 0; it < 200000; ++it) {
    t[0] = -INFINITY;
    t[n] = INFINITY;
    for (int k = 1; k < n; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
    double moved = 0.0;
    for (int k = 0; k < n; ++k) {
      const double next = (std_normal_pdf(t[k]) - std_normal_pdf(t[k + 1])) / cell_mass(t[k], t[k + 1]);
      moved = std::fmax(moved, std::fabs(next - c[k]));
      c[k] = next;
    }
    if (moved < 1e-15) break;
  }
  // Levels held at fp16 precision: 11 significant bits, ties to even, so a
  // power-of-two multiple of each is an exact fp16 number (the decode kernel
  // feeds them to fp16 matrix instructions without rounding).
  const double s = 1.0 / std::sqrt(static_cast<double>(head_dim));
  for (int k = 0; k < n; ++k) {
    int e = 0;
    const double m = std::frexp(c[k] * s, &e);            // |m| in [0.5, 1)
    centroids_out[k] = static_cast<float>(std::ldexp(std::nearbyint(std::ldexp(m, 11)), e - 11));
  }
  return IQ_OK;
}

static int quantize_append_impl(const iq_config *cfg, const void *x, int32_t x_dtype, int32_t batch, int32_t n_new,
                                int32_t rope_dim, const int32_t *start_pos, const iq_cache *out, uint16_t *rope_out,
                                hipStream_t stream) {
  int st = check_config(cfg);
  if (st != IQ_OK) return st;
  if (!x || !start_pos) return IQ_ERR_INVALID_ARG;
  if (!valid_dtype(x_dtype)) return IQ_ERR_UNSUPPORTED;
  if (batch < 1 || n_new < 1 || !vector_count_ok(batch, n_new)) return IQ_ERR_INVALID_ARG;
  st = check_cache(out);
  if (st != IQ_OK) return st;
  if (n_new > out->capacity) return IQ_ERR_INVALID_ARG;
  if (!aligned16(x)) return IQ_ERR_MISALIGNED;
  if (rope_dim > 0) {
    if (!rope_out) return IQ_ERR_INVALID_ARG;
    if (rope_dim % 8 != 0 || rope_dim > kMaxRopeDim) return IQ_ERR_UNSUPPORTED;
    if (!aligned16(rope_out)) return IQ_ERR_MISALIGNED;
  }
  iq::QuantArgs a;
  a.ntens = 1;
  a.t[0] = iq::AppendTensor{x, cfg->quats, out->codes, out->norms, out->capacity};
  a.x_stride = cfg->head_dim + rope_dim;
  a.start_pos = start_pos;
  a.batch = batch;
  a.n = n_new;
  a.hkv = cfg->num_kv_heads;
  a.tab = make_tables(cfg);
  a.cells = make_cells(a.tab, cfg->bits);
  st = hip_status(iq::launch_quantize(cfg->head_dim, cfg->bits, cfg->variant, x_dtype == IQ_F16, a, stream));
  if (st != IQ_OK || rope_dim == 0) return st;
  iq::RopeArgs r;
  r.x = x;
  r.start_pos = start_pos;
  r.out = rope_out;
  r.capacity = out->capacity;
  r.batch = batch;
  r.n = n_new;
  r.hkv = cfg->num_kv_heads;
  r.d = cfg->head_dim;
  r.r = rope_dim;
  return hip_status(iq::launch_rope_copy(x_dtype == IQ_F16, r, stream));
}

int iq_quantize_append(const iq_config *cfg, const void *x, int32_t x_dtype, int32_t batch,
                       int32_t n_new, const int32_t *start_pos, const iq_cache *out,
                       hipStream_t stream) {
  return quantize_append_impl(cfg, x, x_dtype, batch, n_new, 0, start_pos, out, nullptr, stream);
}

int iq_quantize_append_rope(const iq_config *cfg, const void *x, int32_t x_dtype, int32_t batch,
                            int32_t n_new, int32_t rope_dim, const int32_t *start_pos,
                            const iq_cache *out, uint16_t *rope_out, hipStream_t stream) {
  if (rope_dim < 1) return IQ_ERR_INVALID_ARG;
  return quantize_append_impl(cfg, x, x_dtype, batch, n_new, rope_dim, start_pos, out, rope_out, stream);
}

int iq_quantize_append_many(const iq_config *cfgs, int32_t count, const void *const *xs, int32_t x_dtype,
                            int32_t batch, int32_t n_new, const int32_t *start_pos, const iq_cache *outs,
                            hipStream_t stream) {
  if (!cfgs || !xs || !outs || count < 1) return IQ_ERR_INVALID_ARG;
  // every tensor: valid on its own, the same shape and codebook as the first
  for (int32_t i = 0; i < count; ++i) {
    const iq_config *c = &cfgs[i];
    int st = check_config(c);
    if (st != IQ_OK) return st;
    if (c->head_dim != cfgs[0].head_dim || c->bits != cfgs[0].bits || c->variant != cfgs[0].variant ||
        c->num_kv_heads != cfgs[0].num_kv_heads)
      return IQ_ERR_INVALID_ARG;
    for (int k = 0; k < (1 << c->bits); ++k)
      if (c->centroids[k] != cfgs[0].centroids[k]) return IQ_ERR_INVALID_ARG;
    if (!xs[i]) return IQ_ERR_INVALID_ARG;
    if (!aligned16(xs[i])) return IQ_ERR_MISALIGNED;
    st = check_cache(&outs[i]);
    if (st != IQ_OK) return st;
    if (n_new > outs[i].capacity) return IQ_ERR_INVALID_ARG;
  }
  if (!start_pos) return IQ_ERR_INVALID_ARG;
  if (!valid_dtype(x_dtype)) return IQ_ERR_UNSUPPORTED;
  if (batch < 1 || n_new < 1 || !vector_count_ok(batch, n_new)) return IQ_ERR_INVALID_ARG;
  const iq_config *cfg = &cfgs[0];
  iq::QuantArgs a;
  a.x_stride = cfg->head_dim;
  a.start_pos = start_pos;
  a.batch = batch;
  a.n = n_new;
  a.hkv = cfg->num_kv_heads;
  a.tab = make_tables(cfg);
  a.cells = make_cells(a.tab, cfg->bits);
  for (int32_t i0 = 0; i0 < count; i0 += iq::kMaxAppendTensors) {
    a.ntens = std::min<int32_t>(iq::kMaxAppendTensors, count - i0);
    for (int k = 0; k < a.ntens; ++k) {
      const int32_t i = i0 + k;
      a.t[k] = iq::AppendTensor{xs[i], cfgs[i].quats, outs[i].codes, outs[i].norms, outs[i].capacity};
    }
    const int st = hip_status(iq::launch_quantize(cfg->head_dim, cfg->bits, cfg->variant, x_dtype == IQ_F16, a,
                                                  stream));
    if (st != IQ_OK) return st;
  }
  return IQ_OK;
}

int iq_dequantize(const iq_config *cfg, const iq_cache *in, int32_t batch, const int32_t *start_pos,
                  int32_t n, void *out, int32_t out_dtype, hipStream_t stream) {
  int st = check_config(cfg);
  if (st != IQ_OK) return st;
  st = check_cache(in);
  if (st != IQ_OK) return st;
  if (!out || !start_pos) return IQ_ERR_INVALID_ARG;
  if (!valid_dtype(out_dtype)) return IQ_ERR_UNSUPPORTED;
  if (batch < 1 || n < 1 || n > in->capacity || !vector_count_ok(batch, n)) return IQ_ERR_INVALID_ARG;
  if (!aligned16(out)) return IQ_ERR_MISALIGNED;
  iq::DequantArgs a;
  a.codes = in->codes;
  a.norms = in->norms;
  a.quats = cfg->quats;
  a.start_pos = start_pos;
  a.out = out;
  a.capacity = in->capacity;
  a.batch = batch;
  a.n = n;
  a.hkv = cfg->num_kv_heads;
  a.tab = make_tables(cfg);
  return hip_status(iq::launch_dequantize(cfg->head_dim, cfg->bits, cfg->variant, out_dtype == IQ_F16, a, stream));
}

// The decode grids carry the sequence index in their second dimension.
constexpr int32_t kMaxDecodeBatch = 65535;

// Tiles of all (sequence, KV head) segments together stay below this (the
// kernels index them with 32-bit integers).
constexpr int64_t kMaxDecodeTiles = int64_t(1) << 30;

size_t iq_decode_workspace_bytes(const iq_config *cfg, int32_t batch, int32_t num_q_heads,
                                 int64_t max_kv_len) {
  if (check_config(cfg) != IQ_OK || !decode_codebook_exact(cfg)) return 0;
  if (batch < 1 || batch > kMaxDecodeBatch || num_q_heads < 1 || max_kv_len < 0) return 0;
  if (num_q_heads % cfg->num_kv_heads) return 0;
  const int64_t tiles = (max_kv_len + iq::kDecodeStep - 1) / iq::kDecodeStep;
  if (tiles * batch * cfg->num_kv_heads >= kMaxDecodeTiles) return 0;
  return iq::decode_workspace_total(batch, cfg->num_kv_heads, num_q_heads, cfg->head_dim);
}

extern "C++" {
namespace iq {
int decode_workspace_check(const iq_config *cfg, int32_t batch, int32_t num_q_heads, int64_t max_kv_len,
                           size_t *need) {
  int st = check_config(cfg);
  if (st != IQ_OK) return st;
  if (!decode_codebook_exact(cfg)) return IQ_ERR_UNSUPPORTED;
  if (batch < 1 || num_q_heads < 1 || max_kv_len < 0) return IQ_ERR_INVALID_ARG;
  if (batch > kMaxDecodeBatch) return IQ_ERR_UNSUPPORTED;
  if (num_q_heads % cfg->num_kv_heads) return IQ_ERR_INVALID_ARG;
  const int group = num_q_heads / cfg->num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8) return IQ_ERR_UNSUPPORTED;
  *need = iq_decode_workspace_bytes(cfg, batch, num_q_heads, max_kv_len);
  return *need > 0 ? IQ_OK : IQ_ERR_UNSUPPORTED;
}
}  // namespace iq
}

static int check_decode_common(const iq_config *cfg, int32_t batch, int32_t num_q_heads,
                               int64_t max_kv_len, const void *workspace, size_t workspace_bytes,
                               int *group) {
  int st = check_config(cfg);
  if (st != IQ_OK) return st;
  if (!decode_codebook_exact(cfg)) return IQ_ERR_UNSUPPORTED;
  if (!workspace) return IQ_ERR_INVALID_ARG;
  if (batch < 1 || num_q_heads < 1 || max_kv_len < 0) return IQ_ERR_INVALID_ARG;
  if (batch > kMaxDecodeBatch) return IQ_ERR_UNSUPPORTED;
  if (num_q_heads % cfg->num_kv_heads) return IQ_ERR_INVALID_ARG;
  if ((max_kv_len + iq::kDecodeStep - 1) / iq::kDecodeStep * batch * cfg->num_kv_heads >= kMaxDecodeTiles)
    return IQ_ERR_UNSUPPORTED;
  *group = num_q_heads / cfg->num_kv_heads;
  if (*group != 1 && *group != 2 && *group != 4 && *group != 8) return IQ_ERR_UNSUPPORTED;
  if (!aligned16(workspace)) return IQ_ERR_MISALIGNED;
  if (workspace_bytes < iq_decode_workspace_bytes(cfg, batch, num_q_heads, max_kv_len)) return IQ_ERR_WORKSPACE;
  return IQ_OK;
}

// The split phase; with rope_dim > 0 the keys carry rope_dim fp16 RoPE
// coordinates in k_rope and the query d + rope_dim coordinates.
static int decode_partial_impl(const iq_config *cfg, const void *q, int32_t q_dtype, int32_t batch,
                               int32_t num_q_heads, const iq_cache *k, const uint16_t *k_rope, int32_t rope_dim,
                               const iq_cache *v, const int32_t *kv_len, int64_t max_kv_len, float softmax_scale,
                               int32_t track_argmax, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  int group = 0;
  int st = check_decode_common(cfg, batch, num_q_heads, max_kv_len, workspace, workspace_bytes, &group);
  if (st != IQ_OK) return st;
  if (!q || !kv_len) return IQ_ERR_INVALID_ARG;
  if (!valid_dtype(q_dtype)) return IQ_ERR_UNSUPPORTED;
  if (!std::isfinite(softmax_scale)) return IQ_ERR_INVALID_ARG;
  st = check_cache(k);
  if (st != IQ_OK) return st;
  st = check_cache(v);
  if (st != IQ_OK) return st;
  if (max_kv_len > k->capacity || max_kv_len > v->capacity) return IQ_ERR_INVALID_ARG;
  // the kernels address one (sequence, head) region of packed rows with 32-bit
  // offsets and use offsets from 2^30 up as out of range
  const int64_t rb = int64_t(cfg->head_dim) * cfg->bits / 8;
  if (k->capacity * rb >= (int64_t(1) << 30) || v->capacity * rb >= (int64_t(1) << 30)) return IQ_ERR_UNSUPPORTED;
  // norms are streamed as 4-byte words (two rows each) that must lie inside
  // the region, so a region holds an even number of rows
  if ((k->capacity & 1) || (v->capacity & 1)) return IQ_ERR_UNSUPPORTED;
  if (!aligned16(q)) return IQ_ERR_MISALIGNED;
  if (rope_dim > 0) {
    if (!k_rope) return IQ_ERR_INVALID_ARG;
    if (rope_dim != kDecodeRopeDim) return IQ_ERR_UNSUPPORTED;
    // at head_dim 512 and 4 bits two stages of rows, norms and RoPE rows per
    // wave no longer fit next to the pair table in LDS
    if (cfg->head_dim == 512 && cfg->bits == 4) return IQ_ERR_UNSUPPORTED;
    if (!aligned16(k_rope)) return IQ_ERR_MISALIGNED;
    if (k->capacity * rope_dim * 2 >= (int64_t(1) << 30)) return IQ_ERR_UNSUPPORTED;
  }

  // one resident round of partial workgroups on this device
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return IQ_ERR_HIP;
  const int groups = iq::decode_groups_per_cu(cfg->head_dim, cfg->bits, rope_dim);
  const int e = centroid_exponent(cfg);
  iq::DecodeArgs a;
  a.q = q;
  a.q_f16 = q_dtype == IQ_F16;
  a.krope = k_rope;
  a.rope = rope_dim;
  a.rmul = static_cast<float>(static_cast<double>(softmax_scale) * 1.4426950408889634);
  a.kc = k->codes;
  a.kn = k->norms;
  a.vc = v->codes;
  a.vn = v->norms;
  a.kcap = k->capacity;
  a.vcap = v->capacity;
  a.kv_len = kv_len;
  a.quats = cfg->quats;
  a.batch = batch;
  a.hq = num_q_heads;
  a.hkv = cfg->num_kv_heads;
  a.group = group;
  a.variant = cfg->variant;
  a.n_waves = std::min<int64_t>(iq::kMaxDecodeWaves, int64_t(cus) * groups * iq::kDecodeWaves);
  a.qmul = static_cast<float>(static_cast<double>(softmax_scale) * 1.4426950408889634 * std::ldexp(1.0, -e));
  a.argmax = track_argmax != 0;
  char *ws = static_cast<char *>(workspace);
  a.plan = reinterpret_cast<iq::DecodePlan *>(ws);
  a.qrot = reinterpret_cast<uint16_t *>(ws + iq::decode_qrot_offset(batch));
  a.qscale = reinterpret_cast<float *>(ws + iq::decode_qscale_offset(batch, num_q_heads, cfg->head_dim));
  a.ws = reinterpret_cast<float *>(ws + iq::decode_record_offset(batch, num_q_heads, cfg->head_dim));
  std::memset(a.lut, 0, sizeof(a.lut));
  fill_pair_table(cfg, e, a.lut);
  return hip_status(iq::launch_decode(cfg->head_dim, cfg->bits, a, stream));
}

int iq_decode_attention_partial(const iq_config *cfg, const void *q, int32_t q_dtype, int32_t batch,
                                int32_t num_q_heads, const iq_cache *k, const iq_cache *v,
                                const int32_t *kv_len, int64_t max_kv_len, float softmax_scale,
                                int32_t track_argmax, void *workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  return decode_partial_impl(cfg, q, q_dtype, batch, num_q_heads, k, nullptr, 0, v, kv_len, max_kv_len,
                             softmax_scale, track_argmax, workspace, workspace_bytes, stream);
}

int iq_decode_attention_merge(const iq_config *cfg, int32_t batch, int32_t num_q_heads,
                              int64_t max_kv_len, void *out, int32_t out_dtype, float *lse_out,
                              int32_t *argmax_out, const void *workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  int group = 0;
  int st = check_decode_common(cfg, batch, num_q_heads, max_kv_len, workspace, workspace_bytes, &group);
  if (st != IQ_OK) return st;
  if (!out) return IQ_ERR_INVALID_ARG;
  if (!valid_dtype(out_dtype)) return IQ_ERR_UNSUPPORTED;
  if (!aligned16(out)) return IQ_ERR_MISALIGNED;
  if ((lse_out && !aligned16(lse_out)) || (argmax_out && !aligned16(argmax_out))) return IQ_ERR_MISALIGNED;
  const char *ws = static_cast<const char *>(workspace);
  iq::MergeArgs m;
  m.plan = reinterpret_cast<const iq::DecodePlan *>(ws);
  m.ws = reinterpret_cast<const float *>(ws + iq::decode_record_offset(batch, num_q_heads, cfg->head_dim));
  m.quats = cfg->quats;
  m.out = out;
  m.out_f16 = out_dtype == IQ_F16;
  m.lse = lse_out;
  m.argmax = argmax_out;
  m.batch = batch;
  m.hq = num_q_heads;
  m.hkv = cfg->num_kv_heads;
  m.group = group;
  m.oscale = std::ldexp(1.0f, -centroid_exponent(cfg));
  return hip_status(iq::launch_merge(cfg->head_dim, cfg->variant, m, stream));
}

static int decode_fused(const iq_config *cfg, const void *q, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                        const iq_cache *k, const uint16_t *k_rope, int32_t rope_dim, const iq_cache *v,
                        const int32_t *kv_len, int64_t max_kv_len, float softmax_scale, void *out, int32_t out_dtype,
                        float *lse_out, int32_t *argmax_out, void *workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  // validate both phases before enqueueing either
  int group = 0;
  int st = check_decode_common(cfg, batch, num_q_heads, max_kv_len, workspace, workspace_bytes, &group);
  if (st != IQ_OK) return st;
  if (!out) return IQ_ERR_INVALID_ARG;
  if (!valid_dtype(out_dtype)) return IQ_ERR_UNSUPPORTED;
  if (!aligned16(out)) return IQ_ERR_MISALIGNED;
  if ((lse_out && !aligned16(lse_out)) || (argmax_out && !aligned16(argmax_out))) return IQ_ERR_MISALIGNED;
  st = decode_partial_impl(cfg, q, q_dtype, batch, num_q_heads, k, k_rope, rope_dim, v, kv_len, max_kv_len,
                           softmax_scale, argmax_out != nullptr, workspace, workspace_bytes, stream);
  if (st != IQ_OK) return st;
  return iq_decode_attention_merge(cfg, batch, num_q_heads, max_kv_len, out, out_dtype, lse_out,
                                   argmax_out, workspace, workspace_bytes, stream);
}

int iq_decode_attention(const iq_config *cfg, const void *q, int32_t q_dtype, int32_t batch,
                        int32_t num_q_heads, const iq_cache *k, const iq_cache *v,
                        const int32_t *kv_len, int64_t max_kv_len, float softmax_scale, void *out,
                        int32_t out_dtype, float *lse_out, int32_t *argmax_out, void *workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  return decode_fused(cfg, q, q_dtype, batch, num_q_heads, k, nullptr, 0, v, kv_len, max_kv_len, softmax_scale,
                      out, out_dtype, lse_out, argmax_out, workspace, workspace_bytes, stream);
}

int iq_decode_attention_rope(const iq_config *cfg, const void *q, int32_t q_dtype, int32_t batch,
                             int32_t num_q_heads, const iq_cache *k, const uint16_t *k_rope,
                             int32_t rope_dim, const iq_cache *v, const int32_t *kv_len, int64_t max_kv_len,
                             float softmax_scale, void *out, int32_t out_dtype, float *lse_out,
                             int32_t *argmax_out, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (rope_dim < 1) return IQ_ERR_INVALID_ARG;
  return decode_fused(cfg, q, q_dtype, batch, num_q_heads, k, k_rope, rope_dim, v, kv_len, max_kv_len,
                      softmax_scale, out, out_dtype, lse_out, argmax_out, workspace, workspace_bytes, stream);
}

}  // extern "C"
