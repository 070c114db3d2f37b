// Compressed-space decode attention (RotaryQuant §3.4 Table 2, Appendix A),
// split-K over the context, scores and value accumulation on fp16 matrix
// cores (v_mfma_f32_16x16x32_f16) directly from the packed codes.
//
// partial kernel: one workgroup of 4 waves per (split, KV head, sequence);
//   the order kernel (decode.hip) may assign the (sequence, split) pairs
//   longest-first.
//   Prologue: q~ = R q for the G query heads of the KV head (WHT butterflies
//   and SO(4) blocks in LDS), scaled, split into fp16 hi + lo parts and held
//   in registers as the B operand of the score product.
//   The split's 32-token tiles are dealt to the waves round-robin; per tile:
//     scores  S^T (16 tokens x 16 columns) = C_K (16 x d) . Q~^T (d x 16) for
//             two 16-token tiles; column j < G holds q~_hi of head j, column
//             G + j holds q~_lo of head j, so S_hi + S_lo is the full-precision
//             score.  C_K comes from the packed K rows through a 2-code table
//             of exact fp16 centroid pairs (the codebook has 11 significant
//             bits, scaled by a power of two).
//     softmax online, base 2, with a lazily raised running maximum (only
//             rescaled when a score exceeds it by more than kLazyTau).
//     values  O~ (16 rows x d) += P (16 x 32 tokens) . C_V (32 x d); row j < G
//             carries the fp16 hi part of p * ||v|| for head j, row G + j the
//             lo part, so the fp32 accumulators see the weights to ~2^-22.
//   The 4 waves merge their states in LDS; the workgroup writes one partial
//   record (M, L, best score, best position, o~[d]) per query head.
// merge kernel: one workgroup per (query head, sequence): combines the split
//   records, divides by the softmax denominator and applies R^T once.
#pragma once

#include <type_traits>
#include <utility>

#include "iq_device.h"
#include "iq_internal.h"

namespace iq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = kDecodeWaves * 64;

// W-bit field at bit position pos of the little-endian bit string w[].
template <int N>
__device__ __forceinline__ uint32_t field(const uint32_t (&w)[N], int pos, int width) {
  const int wd = pos >> 5, off = pos & 31;
  uint32_t v = (off + width <= 32 || wd + 1 >= N) ? (w[wd] >> off)
                                                  : __builtin_amdgcn_alignbit(w[wd + 1], w[wd], off);
  return v & ((1u << width) - 1u);
}

// f(std::integral_constant<int, i>) for i = 0 .. N-1: loop indices that stay
// constant expressions (bit positions of immediate operands).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Value of lane (lane ^ G) for the hi/lo partner column.
template <int G>
__device__ __forceinline__ float xor_g(float v) {
  const int x = __builtin_bit_cast(int, v);
  int r;
  if constexpr (G == 8)
    r = __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false);      // row_ror:8 == lane ^ 8
  else if constexpr (G == 4)
    r = __builtin_amdgcn_ds_swizzle(x, (4 << 10) | 0x1F);          // lane ^ 4
  else if constexpr (G == 2)
    r = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);       // quad_perm [2,3,0,1]
  else
    r = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);       // quad_perm [1,0,3,2]
  return __builtin_bit_cast(float, r);
}

__device__ __forceinline__ half8 as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  u4 u = {a, b, c, d};
  return __builtin_bit_cast(half8, u);
}

typedef int int32x4_t __attribute__((ext_vector_type(4)));

// Buffer resource (raw, stride 0) over `bytes` bytes at `base`: loads past the
// end return zeros instead of touching memory.
__device__ __forceinline__ int32x4_t make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  int32x4_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32) & 0xFFFF);
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// Asynchronous buffer -> LDS copy: lane i's SIZE bytes at byte offset
// voff + soff of the buffer land at LDS byte address lds + SIZE * i.  The
// instruction writes no registers; completion is awaited with wait_vmem.
template <int SIZE>
__device__ __forceinline__ void dma_to_lds(int32x4_t rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  static_assert(SIZE == 4 || SIZE == 16, "dword or dwordx4");
  if constexpr (SIZE == 16)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Layout of one wave's LDS stage: 32 packed K rows, 32 packed V rows, 32 K
// norms, 32 V norms, and with ROPE > 0 the keys' 32 fp16 RoPE rows.  Rows sit
// RS = ROWB + PAD bytes apart; PAD (0 or one 16-byte granule) is chosen per
// shape so that the row reads of a wave spread over the LDS banks; RoPE rows
// are padded by one granule.
template <int D, int BITS, int ROPE = 0>
struct Stage {
  static constexpr int ROWB = D * BITS / 8;
  static constexpr int PAD = (D == 128 && BITS == 3) ? 0 : 16;
  static constexpr int RS = ROWB + PAD;
  static constexpr int ROWS_B = kDecodeStep * RS;             // bytes of 32 rows in LDS
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = ROWS_B;
  static constexpr int KN_OFF = 2 * ROWS_B;
  static constexpr int VN_OFF = 2 * ROWS_B + 2 * kDecodeStep;
  static constexpr int ROW_LOADS = (ROWS_B + 1023) / 1024;    // 16-byte-per-lane loads per row block
  static constexpr int RROWB = ROPE * 2;                      // bytes of one RoPE row
  static constexpr int RRS = ROPE ? RROWB + 16 : 0;
  static constexpr int R_OFF = 2 * ROWS_B + 4 * kDecodeStep;
  static constexpr int R_B = kDecodeStep * RRS;
  static constexpr int R_LOADS = (R_B + 1023) / 1024;
  static constexpr int BYTES = R_OFF + R_B;                   // multiple of 16
  static constexpr int LOADS = 2 * ROW_LOADS + 2 + R_LOADS;   // buffer->LDS loads per stage
};

// Byte offset past every cache buffer (the host keeps each (sequence, head)
// region of packed rows below it): loads there return zeros and touch no
// memory.
constexpr uint32_t kOutOfRange = 0x40000000u;

// Byte offset inside a 32-row block of the cache of the 16-byte granule that
// lane `lane` of row load c places in LDS (granule 64c + lane of the padded
// stage rows), or kOutOfRange for a pad granule.
template <int D, int BITS>
__device__ __forceinline__ uint32_t granule_offset(int c, int lane) {
  using S = Stage<D, BITS>;
  const int g = 64 * c + lane;
  const int r = g / (S::RS / 16), o = g % (S::RS / 16);
  return o < S::ROWB / 16 ? (uint32_t)(r * S::ROWB + 16 * o) : kOutOfRange;
}

// The same for RoPE row load c (rows of RROWB bytes padded to RRS in LDS).
template <int D, int BITS, int ROPE>
__device__ __forceinline__ uint32_t rope_granule_offset(int c, int lane) {
  using S = Stage<D, BITS, ROPE>;
  const int g = 64 * c + lane;
  const int r = g / (S::RRS / 16), o = g % (S::RRS / 16);
  return o < S::RROWB / 16 ? (uint32_t)(r * S::RROWB + 16 * o) : kOutOfRange;
}

// Issue the asynchronous buffer->LDS loads of one 32-token stage starting at
// token t0 (wave-uniform); stage_lds is the stage's LDS byte address and
// goff[c] the lane's granule offsets.  The token offset rides in the per-lane
// offset, which the buffer range check always covers.  A stage that is not
// needed (valid false) is still issued, pointing out of range, so that every
// stage counts the same number of loads.
template <int D, int BITS, int ROPE>
__device__ __forceinline__ void load_stage(uint32_t stage_lds, int32x4_t kr, int32x4_t vr, int32x4_t knr,
                                           int32x4_t vnr, int32x4_t rr, int t0, bool valid, int lane,
                                           const uint32_t (&goff)[Stage<D, BITS, ROPE>::ROW_LOADS],
                                           const uint32_t (&groff)[Stage<D, BITS, ROPE>::R_LOADS > 0
                                                                      ? Stage<D, BITS, ROPE>::R_LOADS : 1]) {
  using S = Stage<D, BITS, ROPE>;
  const uint32_t row_off = valid ? (uint32_t)(t0 * S::ROWB) : kOutOfRange;
  const uint32_t norm_off = valid ? (uint32_t)(t0 * 2) : kOutOfRange;
#pragma unroll
  for (int c = 0; c < S::ROW_LOADS; ++c) {
    if (c * 1024 + lane * 16 < S::ROWS_B) {
      dma_to_lds<16>(kr, stage_lds + S::K_OFF + c * 1024, goff[c] + row_off, 0);
      dma_to_lds<16>(vr, stage_lds + S::V_OFF + c * 1024, goff[c] + row_off, 0);
    }
  }
  if (lane < kDecodeStep / 2) {
    dma_to_lds<4>(knr, stage_lds + S::KN_OFF, norm_off + lane * 4, 0);
    dma_to_lds<4>(vnr, stage_lds + S::VN_OFF, norm_off + lane * 4, 0);
  }
  if constexpr (ROPE > 0) {
    const uint32_t rope_off = valid ? (uint32_t)(t0 * S::RROWB) : kOutOfRange;
#pragma unroll
    for (int c = 0; c < S::R_LOADS; ++c)
      if (c * 1024 + lane * 16 < S::R_B) dma_to_lds<16>(rr, stage_lds + S::R_OFF + c * 1024, groff[c] + rope_off, 0);
  }
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Replicas of the code-pair table in LDS: lane l reads replica l % REPL
// (entry e at dword e * REPL + l % REPL), so that a wave's table reads fall
// in distinct banks whatever the codes are.
template <int BITS>
constexpr int lut_repl() {
  return BITS <= 3 ? 32 : 8;
}

template <int N>
constexpr int ilog2() {
  return N <= 1 ? 0 : 1 + ilog2<N / 2>();
}

// LDS layout: workgroups per CU (each holds one wave per SIMD) and stages
// per wave.  Three workgroups per CU where each can still keep 3 stages per
// wave next to its pair table and `extra` bytes (more waves hide latency
// better than a deeper ring), else two where each keeps 2 stages, else one;
// then as many stages as fit, up to 4, at least 2 (double buffering).
template <int D, int BITS, int ROPE = 0>
constexpr int stages_fitting(int budget, int extra) {
  const int table = (1 << (2 * BITS)) * lut_repl<BITS>() * 4;
  return (budget - table - extra) / (kDecodeWaves * Stage<D, BITS, ROPE>::BYTES);
}

template <int D, int BITS, int ROPE = 0>
constexpr int resident_groups(int extra) {
  return stages_fitting<D, BITS, ROPE>(160 * 1024 / 3, extra) >= 3   ? 3
         : stages_fitting<D, BITS, ROPE>(160 * 1024 / 2, extra) >= 2 ? 2
                                                                     : 1;
}

template <int D, int BITS, int ROPE = 0>
constexpr int stage_count(int extra) {
  const int n = stages_fitting<D, BITS, ROPE>(160 * 1024 / resident_groups<D, BITS, ROPE>(extra), extra);
  return n > 4 ? 4 : (n < 2 ? 2 : n);
}

// Waves per SIMD the register allocation is held to, matching the LDS
// layout: three where three workgroups share a CU (at most 168 registers per
// lane), two where the LDS of two fits (head_dim <= 256; 256 registers),
// else no constraint.
template <int D, int BITS, int ROPE = 0>
constexpr int partial_waves(int extra) {
  const int table = (1 << (2 * BITS)) * lut_repl<BITS>() * 4;
  const int lds = table + extra + kDecodeWaves * stage_count<D, BITS, ROPE>(extra) * Stage<D, BITS, ROPE>::BYTES;
  return resident_groups<D, BITS, ROPE>(extra) == 3 ? 3 : ((D <= 256 && lds <= 80 * 1024) ? 2 : 1);
}

template <int D, int BITS, int G, bool ARGMAX, int ROPE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(partial_waves<D, BITS, ROPE>(G * (D + ROPE) * 4))))
void partial_kernel(DecodeArgs a) {
  constexpr int NLEV = 1 << BITS;
  constexpr int KS = D / 32;                 // k-steps of the score product
  constexpr int NB = D / 16;                 // 16-column blocks of the value product
  constexpr int ROWB = D * BITS / 8;         // bytes per packed row
  constexpr int CW = ROWB / 16;              // dwords of a row held by one lane group (d/4 dims)
  // K rows are read in units of UDW dwords holding whole code pairs (32 codes
  // at 3 bits, one dword otherwise); lane group g4 holds units g4, g4+4, ...
  // so that the four groups read neighbouring banks.  A unit covers SPU
  // k-steps of 8 dims.
  constexpr int UDW = BITS == 3 ? 3 : 1;
  constexpr int SPU = UDW * 32 / BITS / 8;
  static_assert(CW % UDW == 0 && KS % SPU == 0, "K row units");
  constexpr int VCB = (D / 16) * BITS;       // bits of the d/16 codes a lane owns in the value product
  constexpr int VW = (VCB + 31) / 32 + 1;    // dwords read to cover them at any bit offset
  constexpr int VX = (VCB + 31) / 32;        // dwords after extraction
  constexpr int NROW = 2 * G;                // live rows/columns (hi + lo)
  using S = Stage<D, BITS, ROPE>;
  constexpr int RK = ROPE / 32;                                     // k-steps of the RoPE score product
  constexpr int DQ = D + ROPE;                                      // query coordinates
  constexpr int PRO_B = G * DQ * 4;                                 // prologue q~ staging
  constexpr int NST = stage_count<D, BITS, ROPE>(PRO_B);
  static_assert((NST - 1) * S::LOADS < 64, "in-flight loads exceed the vmcnt range");
  constexpr int STG_B = kDecodeWaves * NST * S::BYTES;              // ring of stages per wave
  constexpr int RED_B = kDecodeWaves * G * (D + 4) * 4;             // wave states at the end
  constexpr int MAIN_B = STG_B > RED_B ? STG_B : RED_B;

  // Grid (KV head, rank): workgroups are handed to the 8 dies (XCDs) in turn
  // by linear index, KV head fastest, so every die gets an even mix.  With an
  // order table (a.order) rank P runs the (sequence, split) of P-th most
  // tokens, so each die works longest-first; without one, rank
  // (sequence + batch * split) runs that pair (first splits, the fullest,
  // first).
  const int kvh = blockIdx.x;
  int b, split, T;
  if (a.order) {
    const int2 o = a.order[blockIdx.y + gridDim.y * blockIdx.z];
    b = __builtin_amdgcn_readfirstlane(o.x & 0xffff);
    split = __builtin_amdgcn_readfirstlane(o.x >> 16);
    T = __builtin_amdgcn_readfirstlane(o.y);
  } else {
    b = blockIdx.y;
    split = blockIdx.z;
    T = __builtin_amdgcn_readfirstlane(a.kv_len[b]);
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  constexpr int REPL = lut_repl<BITS>();
  constexpr int LSH = ilog2<REPL * 4>();     // table entry -> byte offset shift
  // aligned to its own size, so that the entry offset can be OR-ed into the
  // lane's replica offset (pair below)
  __shared__ __attribute__((aligned(NLEV * NLEV * REPL * 4))) uint32_t lut[NLEV * NLEV * REPL];
  __shared__ __attribute__((aligned(16))) char smem[MAIN_B];
  // q~ staging in LDS of its own where it fits (then the first stages load
  // during the prologue), else in the stage memory (loads after it)
  constexpr bool EARLY = MAIN_B + NLEV * NLEV * REPL * 4 + PRO_B <= 160 * 1024;
  __shared__ float qs_own[EARLY ? G : 1][EARLY ? DQ : 1];
  float (*qs)[DQ] = EARLY ? reinterpret_cast<float (*)[DQ]>(&qs_own[0][0]) : reinterpret_cast<float (*)[DQ]>(smem);

  // The workgroup's tokens [base, end) are dealt to the waves tile by tile
  // (tile i to wave i mod 4), so that its waves finish together whatever the
  // length: the workgroup holds its compute unit until its slowest wave ends.
  const int base = split * a.chunk;
  const int end = min(T, base + a.chunk);
  const int len = end > base ? end - base : 0;
  auto tile_t0 = [&](int k) { return base + (wave + kDecodeWaves * k) * kDecodeStep; };
  const long long hrow = (long long)b * a.hkv + kvh;
  const int32x4_t kr = make_rsrc(a.kc + hrow * a.kcap * ROWB, (uint32_t)(a.kcap * ROWB));
  const int32x4_t vr = make_rsrc(a.vc + hrow * a.vcap * ROWB, (uint32_t)(a.vcap * ROWB));
  const int32x4_t knr = make_rsrc(a.kn + hrow * a.kcap, (uint32_t)(a.kcap * 2));
  const int32x4_t vnr = make_rsrc(a.vn + hrow * a.vcap, (uint32_t)(a.vcap * 2));
  const int32x4_t rr = ROPE ? make_rsrc(a.krope + hrow * a.kcap * ROPE, (uint32_t)(a.kcap * ROPE * 2)) : kr;
  char *stages = smem + wave * NST * S::BYTES;
  const uint32_t stages_lds = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(stages));
  uint32_t goff[S::ROW_LOADS];
#pragma unroll
  for (int c = 0; c < S::ROW_LOADS; ++c) goff[c] = granule_offset<D, BITS>(c, lane);
  uint32_t groff[S::R_LOADS > 0 ? S::R_LOADS : 1];
#pragma unroll
  for (int c = 0; c < S::R_LOADS; ++c) groff[c] = rope_granule_offset<D, BITS, ROPE>(c, lane);
  // this wave's tiles k = 0, 1, ...: workgroup tiles wave + 4k
  auto count = [&](int tiles) { return tiles > wave ? (tiles - wave + kDecodeWaves - 1) / kDecodeWaves : 0; };
  const int n_tiles = count((len + kDecodeStep - 1) / kDecodeStep);
  const int n_full = count(len / kDecodeStep);
  // The first NST - 1 stages are requested before the prologue, whose work
  // then overlaps their memory latency.
  auto first_stages = [&] {
    if (n_tiles > 0) {
#pragma unroll
      for (int i = 0; i < NST - 1; ++i)
        load_stage<D, BITS, ROPE>(stages_lds + i * S::BYTES, kr, vr, knr, vnr, rr, tile_t0(i), i < n_tiles, lane,
                                  goff, groff);
    }
  };
  if constexpr (EARLY) first_stages();

  // ---- prologue: q~ = R q for this KV head's query heads --------------------
  for (int i = threadIdx.x; i < NLEV * NLEV * REPL; i += kThreads) lut[i] = a.lut[i / REPL];
  for (int idx = threadIdx.x; idx < G * DQ; idx += kThreads) {
    const int hh = idx / DQ, i = idx % DQ;
    const size_t off = ((size_t)b * a.hq + kvh * G + hh) * DQ + i;
    qs[hh][i] = a.q_f16 ? static_cast<float>(static_cast<const _Float16 *>(a.q)[off])
                        : static_cast<const float *>(a.q)[off];
  }
  __syncthreads();
  for (int st = 1; st < D; st <<= 1) {
    for (int p = threadIdx.x; p < G * D / 2; p += kThreads) {
      const int hh = p / (D / 2), pp = p % (D / 2);
      const int i = (pp / st) * 2 * st + (pp % st);
      const float x0 = qs[hh][i], x1 = qs[hh][i + st];
      qs[hh][i] = x0 + x1;
      qs[hh][i + st] = x0 - x1;
    }
    __syncthreads();
  }
  {
    const float scale = a.qmul / sqrtf((float)D);
    const float *pg = a.quats + (size_t)kvh * (D / 4) * block_param_floats(a.variant);
    for (int p = threadIdx.x; p < G * D / 4; p += kThreads) {
      const int hh = p / (D / 4), blk = p % (D / 4);
      float4 v = make_float4(qs[hh][4 * blk] * scale, qs[hh][4 * blk + 1] * scale,
                             qs[hh][4 * blk + 2] * scale, qs[hh][4 * blk + 3] * scale);
      float4 t = a.variant == 0 ? block_fwd<0>(v, pg, blk)
                 : a.variant == 1 ? block_fwd<1>(v, pg, blk) : block_fwd<kPlanar>(v, pg, blk);
      qs[hh][4 * blk] = t.x;
      qs[hh][4 * blk + 1] = t.y;
      qs[hh][4 * blk + 2] = t.z;
      qs[hh][4 * blk + 3] = t.w;
    }
  }
  __syncthreads();

  const int j = lane & 15;      // column of the score tile / row of the value operand
  const int g4 = lane >> 4;     // lane group: k-slice of the operands, row quad of results
  const bool live = j < NROW;
  const bool lo_lane = live && j >= G;
  const int head = j % G;

  // B operand of the score product: k-step s of lane group g4 holds dims
  // 8 (s mod SPU) .. +7 of row unit 4 (s / SPU) + g4 (the dims the K operand
  // carries at the same k positions).
  half8 qB[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int dim = (4 * (s / SPU) + g4) * (8 * SPU) + 8 * (s % SPU) + e;
      const float v = live ? qs[head][dim] : 0.f;
      const _Float16 hi = static_cast<_Float16>(v);
      qB[s][e] = lo_lane ? static_cast<_Float16>(v - static_cast<float>(hi)) : hi;
    }
  }
  // B operand of the RoPE score product: k-step s of lane group g4 holds RoPE
  // coordinates 32 s + 8 g4 .. +7 (the natural order of the RoPE rows), times
  // softmax_scale * log2(e), hi and lo fp16 parts as for qB.
  half8 qR[RK > 0 ? RK : 1];
#pragma unroll
  for (int s = 0; s < RK; ++s) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = live ? qs[head][D + 32 * s + 8 * g4 + e] * a.rmul : 0.f;
      const _Float16 hi = static_cast<_Float16>(v);
      qR[s][e] = lo_lane ? static_cast<_Float16>(v - static_cast<float>(hi)) : hi;
    }
  }
  if constexpr (!EARLY) {
    __syncthreads();                         // qs is reused as stage memory
    first_stages();
  }

  // ---- main loop ---------------------------------------------------------------
  const int my_tile = lo_lane ? 1 : 0;
  const int vbit = VCB * j;                  // bit offset of this lane's codes in a row
  const float lo_mask = lo_lane ? 1.f : 0.f;
  // per-lane LDS byte offsets inside a stage
  const int k_off = S::K_OFF + j * S::RS + g4 * UDW * 4;
  const int v_off = S::V_OFF + 4 * g4 * S::RS + (vbit >> 5) * 4;
  const int n_off = (16 * my_tile + 4 * g4) * 2;
  // byte address of this lane's replica of table entry 0
  const uint32_t lut_base = lds_addr(lut) | (uint32_t)(lane % REPL) * 4u;
  // table entry at the 2*BITS-bit field at bit `pos` of w: the field is
  // shifted to bit LSH and masked, and the lane's replica offset OR-ed in
  // (the table is aligned to its size): a shift and one three-input bit
  // operation, or the bit operation alone where pos = LSH
  auto pair = [&](uint32_t w, auto pos) -> uint32_t {
    constexpr int P = decltype(pos)::value;
    constexpr uint32_t M = ((1u << (2 * BITS)) - 1u) << LSH;
    const uint32_t f = P >= LSH ? (w >> (P - LSH)) : (w << (LSH - P));
    const uint32_t addr = (f & M) | lut_base;
    return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t *>(addr);
  };

  float Mh = -INFINITY, Mb = -INFINITY, Lh = 0.f, best_s = -INFINITY;
  int best_j = -1;
  floatx4 O[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) O[nb] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto process = [&](const char *cur, const int t0, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    // packed K rows of the two 16-token tiles (lane: token j, dims slice g4)
    uint32_t kw[2][CW];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      const uint32_t *src = reinterpret_cast<const uint32_t *>(cur + k_off + tile * 16 * S::RS);
#pragma unroll
      for (int m = 0; m < CW / UDW; ++m)
#pragma unroll
        for (int t = 0; t < UDW; ++t) kw[tile][m * UDW + t] = src[4 * m * UDW + t];
    }
    // the 8 tokens of this lane in the operand/result layouts: 4*g4 + r of each tile
    uint32_t vch[8][VX];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const uint32_t *src = reinterpret_cast<const uint32_t *>(cur + v_off + (16 * (r >> 2) + (r & 3)) * S::RS);
      uint32_t w[VW];
#pragma unroll
      for (int i = 0; i < VW; ++i) w[i] = src[i];            // may read one dword past the row: still in LDS
#pragma unroll
      for (int i = 0; i < VX; ++i) vch[r][i] = __builtin_amdgcn_alignbit(w[i + 1], w[i], vbit & 31);
    }
    typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
    const u16x4 kb = *reinterpret_cast<const u16x4 *>(cur + S::KN_OFF + n_off);
    const u16x4 vb = *reinterpret_cast<const u16x4 *>(cur + S::VN_OFF + n_off);

    // Table reads for both operands are issued up front, so that their LDS
    // latency overlaps the score products and the softmax.
    // K operand: lane (token j, dims slice g4), k-step s holds dims 8s..8s+7
    // of the slice as 4 code pairs.
    uint32_t ka[2][KS][4];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      static_for<KS>([&](auto s) {
        static_for<4>([&](auto p) {
          constexpr int W = 2 * BITS;
          constexpr int sv = decltype(s)::value;
          constexpr int pos = (sv / SPU) * UDW * 32 + (8 * (sv % SPU) + 2 * decltype(p)::value) * BITS;
          constexpr int wd = pos >> 5, off = pos & 31;
          if constexpr (off + W <= 32 || wd + 1 >= CW)
            ka[tile][s][p] = pair(kw[tile][wd], std::integral_constant<int, off>{});
          else {
            // a pair across two dwords: the funnel shift also moves the field
            // to bit LSH, where the table offset wants it
            static_assert(off >= LSH, "straddling field below the table shift");
            ka[tile][s][p] = pair(__builtin_amdgcn_alignbit(kw[tile][wd + 1], kw[tile][wd], off - LSH),
                                  std::integral_constant<int, LSH>{});
          }
        });
      });
    }
    // V operand: column block nb holds dims (D/16) * n + nb of lane column
    // n = j; dword p is the pair of tokens (2p, 2p+1) of the lane's 8
    // (code_a | code_b << BITS).  Per group of 8 column blocks the two tokens'
    // fields are interleaved first (SWAR): X[g][p][parity] holds the pair
    // indices of the group's dims of that parity at 2*BITS-bit strides.
    uint32_t vbw[NB][4];
    {
      constexpr int NGRP = NB / 8;
      constexpr uint32_t M = (1u << BITS) - 1u;
      constexpr uint32_t ME = M | (M << (2 * BITS)) | (M << (4 * BITS)) | (M << (6 * BITS));
      uint32_t X[NGRP][4][2];
      static_for<NGRP>([&](auto gi) {
        constexpr int bit0 = decltype(gi)::value * 8 * BITS, wd = bit0 >> 5, off = bit0 & 31;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          uint32_t ca, cb;
          if constexpr (off + 8 * BITS <= 32) {
            ca = vch[2 * p][wd] >> off;
            cb = vch[2 * p + 1][wd] >> off;
          } else {
            ca = __builtin_amdgcn_alignbit(vch[2 * p][wd + 1], vch[2 * p][wd], off);
            cb = __builtin_amdgcn_alignbit(vch[2 * p + 1][wd + 1], vch[2 * p + 1][wd], off);
          }
          // bit-field inserts (one v_bfi_b32 each): the fields of ca under
          // ME, those of cb shifted into the gaps; only the group's 8 * BITS
          // low bits are read afterwards
          X[gi][p][0] = (ca & ME) | ((cb << BITS) & ~ME);
          X[gi][p][1] = ((ca >> BITS) & ME) | (cb & ~ME);
        }
      });
      static_for<NB>([&](auto nb) {
        constexpr int nbv = decltype(nb)::value;
        constexpr int sh = ((nbv % 8) >> 1) * 2 * BITS;
#pragma unroll
        for (int p = 0; p < 4; ++p) vbw[nb][p] = pair(X[nbv / 8][p][nbv & 1], std::integral_constant<int, sh>{});
      });
    }

    // scores for both tiles
    floatx4 S2[2];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      S2[tile] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s)
        S2[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            as_half8(ka[tile][s][0], ka[tile][s][1], ka[tile][s][2], ka[tile][s][3]), qB[s], S2[tile], 0, 0, 0);
    }
    // RoPE part of the scores (not scaled by the key norm): the keys' fp16
    // RoPE rows straight from the stage, lane (token j, group g4)
    floatx4 SR[2];
    if constexpr (ROPE > 0) {
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        SR[tile] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < RK; ++s) {
          const half8 kr8 = *reinterpret_cast<const half8 *>(cur + S::R_OFF + (16 * tile + j) * S::RRS +
                                                             (32 * s + 8 * g4) * 2);
          SR[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kr8, qR[s], SR[tile], 0, 0, 0);
        }
      }
    }

    // softmax on this lane's tile (hi lanes: tile 0, lo lanes: tile 1).
    // u = score + an upper bound of the value-norm exponent (byte 1 of its
    // fp16 bits / 4) drives the running maximum.
    float sig[4], u[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float own = my_tile ? S2[1][r] : S2[0][r];
      const float give = my_tile ? S2[0][r] : S2[1][r];      // what the partner lane needs
      float c = (own + xor_g<G>(give)) * half_bits_to_float(kb[r]);
      if constexpr (ROPE > 0) {
        const float rown = my_tile ? SR[1][r] : SR[0][r];
        const float rgive = my_tile ? SR[0][r] : SR[1][r];
        c += rown + xor_g<G>(rgive);
      }
      if constexpr (!FULL) {
        const int tok = t0 + 16 * my_tile + 4 * g4 + r;
        c = (live && tok < end) ? c : -INFINITY;
      } else {
        c = live ? c : -INFINITY;
      }
      sig[r] = c;
      u[r] = fmaf((float)((vb[r] >> 8) & 0xFF), 0.25f, c);
    }
    if constexpr (ARGMAX) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (sig[r] > best_s) {
          best_s = sig[r];
          best_j = t0 + 16 * my_tile + 4 * g4 + r;
        }
      }
    }
    const float lmax = fmaxf(fmaxf(u[0], u[1]), fmaxf(u[2], u[3]));
    if (__any(lmax > Mh + kLazyTau)) {
      float umax = fmaxf(lmax, xor_g<G>(lmax));
      umax = fmaxf(umax, __shfl_xor(umax, 16, 64));
      umax = fmaxf(umax, __shfl_xor(umax, 32, 64));
      const float mnew = fmaxf(Mh, umax);
      const float alpha = (Mh == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(Mh - mnew);
      Lh *= alpha;
      Mh = mnew;
      Mb = mnew - kWeightBias;
      // rows 4*g4 + i of the value accumulators belong to head (4*g4 + i) % G
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * g4 + i;
        const float ar = __shfl(alpha, row < NROW ? row % G : 0, 64);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) O[nb][i] *= ar;
      }
    }
    float y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x = __builtin_amdgcn_exp2f(sig[r] - Mb);   // 2^(s - M + bias); 0 for masked tokens
      Lh += x;
      y[r] = live ? x * half_bits_to_float(vb[r]) : 0.f;
    }
    // A operand, k order = tile-0 tokens 4*g4..+3 then tile-1 tokens; hi lanes
    // carry fp16(y) (round toward zero), lo lanes the exact remainder.
    uint32_t pw[4];
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      float pa[2], pb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int r = 2 * q2 + t;
        const float other = xor_g<G>(y[r]);
        pa[t] = my_tile ? other : y[r];      // tile 0 token 4*g4 + r
        pb[t] = my_tile ? y[r] : other;      // tile 1 token 4*g4 + r
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const float e0 = half ? pb[0] : pa[0];
        const float e1 = half ? pb[1] : pa[1];
        const auto h = __builtin_amdgcn_cvt_pkrtz(e0, e1);
        const float d0 = fmaf(-lo_mask, static_cast<float>(h[0]), e0);
        const float d1 = fmaf(-lo_mask, static_cast<float>(h[1]), e1);
        pw[2 * half + q2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(d0, d1));
      }
    }
    const half8 P = as_half8(pw[0], pw[1], pw[2], pw[3]);

    // values
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      O[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(P, as_half8(vbw[nb][0], vbw[nb][1], vbw[nb][2], vbw[nb][3]),
                                                     O[nb], 0, 0, 0);
  };

  // Ring of NST stages per wave: the next NST - 1 tiles are in flight while
  // one is processed.  Every iteration issues one stage (out of range past
  // the wave's last tile), so one fixed wait finds the oldest stage landed.
  if (n_tiles > 0) {
    int slot = 0;                            // stage of tile `it`
    for (int it = 0; it < n_full; ++it) {
      const int ahead = it + NST - 1;
      const int aslot = slot == 0 ? NST - 1 : slot - 1;     // (it + NST - 1) mod NST, processed last iteration
      load_stage<D, BITS, ROPE>(stages_lds + aslot * S::BYTES, kr, vr, knr, vnr, rr, tile_t0(ahead), ahead < n_tiles,
                                lane, goff, groff);
      wait_vmem<(NST - 1) * S::LOADS>();
      process(stages + slot * S::BYTES, tile_t0(it), std::true_type{});
      slot = slot == NST - 1 ? 0 : slot + 1;
    }
    wait_vmem<0>();                          // also drains the out-of-range stages before LDS is reused
    if (n_full < n_tiles)                    // the last, partial tile
      process(stages + slot * S::BYTES, tile_t0(n_full), std::false_type{});
  }
  __syncthreads();                           // stage memory is reused for the wave states below
  float (*red_o)[G][D + 4] = reinterpret_cast<float (*)[G][D + 4]>(smem);

  // ---- wave state -> LDS -----------------------------------------------------------
  // softmax denominator and argmax per head: lanes (head, head + G) x 4 groups
  float lsum = live ? Lh : 0.f;
  lsum += xor_g<G>(lsum);
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  float bs = live ? best_s : -INFINITY;
  int bj = live ? best_j : -1;
  {
    auto take = [&](float os, int oj) {
      if (os > bs || (os == bs && oj >= 0 && (bj < 0 || oj < bj))) {
        bs = os;
        bj = oj;
      }
    };
    take(xor_g<G>(bs), __builtin_bit_cast(int, xor_g<G>(__builtin_bit_cast(float, bj))));
    take(__shfl_xor(bs, 16, 64), __shfl_xor(bj, 16, 64));
    take(__shfl_xor(bs, 32, 64), __shfl_xor(bj, 32, 64));
  }
  if (lane < G) {
    red_o[wave][lane][D + 0] = Mh;
    red_o[wave][lane][D + 1] = lsum;
    red_o[wave][lane][D + 2] = bs;
    red_o[wave][lane][D + 3] = __builtin_bit_cast(float, bj);
  }
  // value rows: hi row h + lo row h + G
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = O[nb][i];
      float partner;
      if constexpr (G >= 4)
        partner = __shfl_xor(v, 16 * (G / 4), 64);
      else
        partner = O[nb][i ^ G];
      const int row = 4 * g4 + i;
      if (row < G) red_o[wave][row][(D / 16) * j + nb] = v + partner;
    }
  }
  __syncthreads();

  // ---- combine the waves, write this split's records ---------------------------------
  const int n_part = a.n_split;
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int hh = idx / D, i = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w)
      if (red_o[w][hh][D + 1] > 0.f) M = fmaxf(M, red_o[w][hh][D]);
    float o = 0.f, L = 0.f, bsc = -INFINITY;
    int bpos = -1;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      if (red_o[w][hh][D + 1] > 0.f) {
        const float sc = exp2f(red_o[w][hh][D] - M);
        o += red_o[w][hh][i] * sc;
        L += red_o[w][hh][D + 1] * sc;
        if (red_o[w][hh][D + 2] > bsc) {
          bsc = red_o[w][hh][D + 2];
          bpos = __builtin_bit_cast(int, red_o[w][hh][D + 3]);
        }
      }
    }
    float *rec = a.ws + (((size_t)b * a.hq + kvh * G + hh) * n_part + split) * (D + kRecHeader);
    rec[kRecHeader + i] = o;
    if (i == 0) {
      rec[0] = M;
      rec[1] = L;
      rec[2] = bsc;
      rec[3] = __builtin_bit_cast(float, bpos);
    }
  }
}

constexpr int kMergeChunk = 1024;          // split records whose weights are staged in LDS at a time

template <int D, int VARIANT>
__global__ __launch_bounds__(D) void merge_kernel(MergeArgs a) {
  constexpr int RS = D + kRecHeader;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int g = h / a.group;
  const int i = threadIdx.x;
  const int n = a.n_part;
  const float *recs = a.ws + ((size_t)b * a.hq + h) * n * RS;
  constexpr int NW = D / 64;                 // waves of the workgroup
  __shared__ float redf[NW];
  __shared__ int redi[NW];
  __shared__ float wbuf[kMergeChunk];
  const int lane = i & 63, wave = i >> 6;
  // (score, position) pairs: the larger score, ties to the lower valid position
  auto better = [](float s1, int p1, float s0, int p0) {
    return s1 > s0 || (s1 == s0 && p1 >= 0 && (p0 < 0 || p1 < p0));
  };

  // Headers are read in parallel (thread t: records t, t + D, ...): the
  // running maximum and the best score with its position (ties: the lower
  // position; splits cover increasing positions).  Reductions: across the
  // wave by lane exchanges, then across the waves through LDS.
  float Mt = -INFINITY, bt = -INFINITY;
  int at = -1;
  for (int p = i; p < n; p += D) {
    const float *rec = recs + (size_t)p * RS;
    if (rec[1] > 0.f) {
      Mt = fmaxf(Mt, rec[0]);
      const float sc = rec[2];
      const int pos = __builtin_bit_cast(int, rec[3]);
      if (better(sc, pos, bt, at)) {
        bt = sc;
        at = pos;
      }
    }
  }
  for (int m = 32; m > 0; m >>= 1) {
    Mt = fmaxf(Mt, __shfl_xor(Mt, m, 64));
    const float os = __shfl_xor(bt, m, 64);
    const int oj = __shfl_xor(at, m, 64);
    if (better(os, oj, bt, at)) {
      bt = os;
      at = oj;
    }
  }
  if (lane == 0) {
    redf[wave] = Mt;
    redi[wave] = at;
    wbuf[wave] = bt;                         // wbuf is free until the weights below
  }
  __syncthreads();
  float M = redf[0], bsc = wbuf[0];
  int arg = redi[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    M = fmaxf(M, redf[w]);
    if (better(wbuf[w], redi[w], bsc, arg)) {
      bsc = wbuf[w];
      arg = redi[w];
    }
  }
  __syncthreads();

  // Weights 2^(M_p - M) (0 for empty splits) staged in LDS chunk by chunk;
  // each thread then sums its coordinate over the records in split order,
  // with independent loads.
  float Lt = 0.f, o = 0.f;
  for (int c0 = 0; c0 < n; c0 += kMergeChunk) {
    const int cn = min(kMergeChunk, n - c0);
    for (int p = i; p < cn; p += D) {
      const float *rec = recs + (size_t)(c0 + p) * RS;
      const float lp = rec[1];
      const float w = lp > 0.f ? exp2f(rec[0] - M) : 0.f;
      wbuf[p] = w;
      Lt += lp > 0.f ? lp * w : 0.f;
    }
    __syncthreads();
    const float *col = recs + (size_t)c0 * RS + kRecHeader + i;
#pragma unroll 8
    for (int p = 0; p < cn; ++p) {
      const float w = wbuf[p];
      const float v = col[(size_t)p * RS];
      o += w > 0.f ? v * w : 0.f;
    }
    __syncthreads();
  }
  for (int m = 32; m > 0; m >>= 1) Lt += __shfl_xor(Lt, m, 64);
  if (lane == 0) redf[wave] = Lt;
  __syncthreads();
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) L += redf[w];

  __shared__ float y[D];
  y[i] = L > 0.f ? o * a.oscale / L : 0.f;
  __syncthreads();
  if (i < D / 4) {
    const float *pg = a.quats + (size_t)g * (D / 4) * block_param_floats(VARIANT);
    float4 u = block_inv<VARIANT>(make_float4(y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]), pg, i);
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
    if (a.lse) a.lse[oh] = L > 0.f ? (M - kWeightBias + log2f(L)) * 0.69314718055994531f : -INFINITY;
    if (a.argmax) a.argmax[oh] = L > 0.f ? arg : -1;
  }
}

template <int D, int BITS, bool ARGMAX, int ROPE>
hipError_t partial_dispatch_group(const DecodeArgs &a, hipStream_t s) {
  dim3 grid((unsigned)a.hkv, (unsigned)a.batch, (unsigned)a.n_split);
  switch (a.group) {
    case 1: hipLaunchKernelGGL((partial_kernel<D, BITS, 1, ARGMAX, ROPE>), grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((partial_kernel<D, BITS, 2, ARGMAX, ROPE>), grid, dim3(kThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((partial_kernel<D, BITS, 4, ARGMAX, ROPE>), grid, dim3(kThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL((partial_kernel<D, BITS, 8, ARGMAX, ROPE>), grid, dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, int BITS, int ROPE>
hipError_t partial_dispatch_argmax(const DecodeArgs &a, hipStream_t s) {
  return a.argmax ? partial_dispatch_group<D, BITS, true, ROPE>(a, s)
                  : partial_dispatch_group<D, BITS, false, ROPE>(a, s);
}

// Whether the pair table and a ring of two stages per wave fit in one
// compute unit's LDS (every shape without RoPE coordinates does; with them
// head_dim 512 at 4 bits does not).
template <int D, int BITS, int ROPE>
constexpr bool partial_fits() {
  return (1 << (2 * BITS)) * lut_repl<BITS>() * 4 + kDecodeWaves * 2 * Stage<D, BITS, ROPE>::BYTES <= 160 * 1024;
}

// ROPE: the RoPE coordinates per key these instantiations take (0: none).
template <int D, int ROPE = 0>
hipError_t partial_dispatch_bits(int bits, const DecodeArgs &a, hipStream_t s) {
  if (a.rope != ROPE) return hipErrorInvalidValue;
  switch (bits) {
    case 2: return partial_dispatch_argmax<D, 2, ROPE>(a, s);
    case 3: return partial_dispatch_argmax<D, 3, ROPE>(a, s);
    case 4:
      if constexpr (partial_fits<D, 4, ROPE>()) return partial_dispatch_argmax<D, 4, ROPE>(a, s);
      break;
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t merge_dispatch(int variant, const MergeArgs &a, hipStream_t s) {
  dim3 grid((unsigned)a.hq, (unsigned)a.batch);
  switch (variant) {
    case 0: hipLaunchKernelGGL((merge_kernel<D, 0>), grid, dim3(D), 0, s, a); break;
    case 1: hipLaunchKernelGGL((merge_kernel<D, 1>), grid, dim3(D), 0, s, a); break;
    case kPlanar: hipLaunchKernelGGL((merge_kernel<D, kPlanar>), grid, dim3(D), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace
}  // namespace iq
