// Compressed-space decode attention (RotaryQuant §3.4 Table 2, Appendix A):
// scores and value accumulation on fp16 matrix cores
// (v_mfma_f32_16x16x32_f16) directly from the packed codes, the work of a
// call spread evenly over the waves of one resident round.
//
// prep kernel: plans the work (DecodePlan, decode_args.h) and rotates the G
//   query heads of each (sequence, KV head): q~ = R q (WHT butterflies in
//   registers and across lanes, then the SO(4) blocks), scaled by a power of
//   two, split into fp16 hi + lo parts, stored as 2G rows (hi rows, then lo
//   rows).  Up to 256 segments every workgroup computes the plan and writes
//   its share of it beside its rotation; beyond that workgroup 0 plans alone.
// partial kernel: every wave owns W consecutive tiles of 32 tokens of the
//   (sequence, KV head) segments laid end to end; waves never synchronise.
//   Per tile:
//     scores  S^T (16 tokens x 16 columns) = C_K (16 x d) . Q~^T (d x 16) for
//             two 16-token tiles; column j < G holds q~_hi of head j, column
//             G + j holds q~_lo of head j, so S_hi + S_lo is the full-precision
//             score.  C_K comes from the packed K rows through a 2-code table
//             of exact fp16 centroid pairs (each level times 2^e is an fp16
//             number) replicated in LDS.
//     softmax online, base 2, with a lazily raised running maximum (only
//             rescaled when a score plus a bound of its value norm's exponent
//             exceeds it by more than kLazyTau).
//     values  O~ (16 rows x d) += P (16 x 32 tokens) . C_V (32 x d); row j < G
//             carries the fp16 hi part of p * ||v|| for head j, row G + j the
//             lo part, so the fp32 accumulators see the weights to ~2^-22.
//   At the end of a segment or of its share the wave writes one record
//   (M, L, best score, best position, o~[d]) per query head.
// merge kernel: one workgroup per (query head, sequence): combines the records
//   of the segment's pieces, divides by the softmax denominator and applies
//   R^T once.
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
  // (bound_ctrl set: every source lane of these patterns exists, and the
  // compiler can then fold the move into the instruction that uses it)
  if constexpr (G == 8)
    r = __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, true);       // row_ror:8 == lane ^ 8
  else if constexpr (G == 4)
    r = __builtin_amdgcn_ds_swizzle(x, (4 << 10) | 0x1F);          // lane ^ 4
  else if constexpr (G == 2)
    r = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);        // quad_perm [2,3,0,1]
  else
    r = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);        // quad_perm [1,0,3,2]
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

// A load from an LDS byte address (the constant part of an address folds
// into the instruction's offset field).
template <typename T>
__device__ __forceinline__ T lds_ld(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T *>(addr);
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
// Issued through the builtin, not inline asm, so that the compiler sees the
// wait: its own loads before a vmcnt(0) count as done, and it inserts no
// wait of its own for them later (a compiler-inserted vmcnt(0) in the tile
// loop would also wait for every stage in flight).  The builtin touches no
// memory as far as the compiler knows, so an empty asm with a memory clobber
// follows it: no LDS read of a stage may be scheduled above the wait.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));   // expcnt, lgkmcnt at max
  asm volatile("" ::: "memory");
}

// The code-pair table lives in LDS, replicated so that a wave's reads fall
// in distinct banks whatever the codes: lane l reads replica l mod REPL
// (entry e at dword e * REPL + l mod REPL); 32 replicas of the 16 or 64
// pairs at 2 and 3 bits, 8 of the 256 pairs at 4 bits.  (Reading the table
// from a register by lane permutation instead saves an instruction per read
// but ran a quarter slower: the permutes cost more than conflict-free reads.)
template <int BITS>
constexpr int lut_repl() {
  return BITS <= 3 ? 32 : 8;
}
template <int BITS>
constexpr int lds_table_bytes() {
  return (1 << (2 * BITS)) * lut_repl<BITS>() * 4;
}

template <int N>
constexpr int ilog2() {
  return N <= 1 ? 0 : 1 + ilog2<N / 2>();
}

// LDS layout: workgroups per CU (each holds one wave per SIMD) and stages
// per wave.  Four workgroups per CU at head_dim 128 without RoPE rows where
// each keeps at least 2 stages per wave next to its table (2 at 3 bits, 3 at
// 2 bits, whose table is smaller; these kernels fit 128
// registers once the value operand is built after the softmax, and the
// fourth wave per SIMD fills VALU issue slots the other three leave: 6%
// faster than three waves with 3 stages); else three where each can keep 3
// stages per wave (more waves hide latency better than a deeper ring), else
// two where each keeps 2 stages, else one; then as many stages as fit, up
// to 4, at least 2 (double buffering).
template <int D, int BITS, int ROPE = 0>
constexpr int stages_fitting(int budget) {
  return (budget - lds_table_bytes<BITS>()) / (kDecodeWaves * Stage<D, BITS, ROPE>::BYTES);
}

template <int D, int BITS, int ROPE = 0>
constexpr int resident_groups() {
  return (D == 128 && ROPE == 0 && stages_fitting<D, BITS, ROPE>(160 * 1024 / 4) >= 2) ? 4
         : stages_fitting<D, BITS, ROPE>(160 * 1024 / 3) >= 3                           ? 3
         : stages_fitting<D, BITS, ROPE>(160 * 1024 / 2) >= 2 ? 2
                                                               : 1;
}

template <int D, int BITS, int ROPE = 0>
constexpr int stage_count() {
  const int n = stages_fitting<D, BITS, ROPE>(160 * 1024 / resident_groups<D, BITS, ROPE>());
  return n > 4 ? 4 : (n < 2 ? 2 : n);
}

// Waves per SIMD the register allocation is held to, matching the LDS
// layout: four or three where that many workgroups share a CU (at most 128
// or 168 registers per lane), two where the LDS of two fits (head_dim <=
// 256; 256 registers), else no constraint.
template <int D, int BITS, int ROPE = 0>
constexpr int partial_waves() {
  const int lds = lds_table_bytes<BITS>() + kDecodeWaves * stage_count<D, BITS, ROPE>() * Stage<D, BITS, ROPE>::BYTES;
  return resident_groups<D, BITS, ROPE>() >= 3 ? resident_groups<D, BITS, ROPE>()
                                               : ((D <= 256 && lds <= 80 * 1024) ? 2 : 1);
}

// ---------------------------------------------------------------------------
// prep kernel
// ---------------------------------------------------------------------------

// Workgroup 0: tiles per segment, their prefix (segment s = b H_kv + h starts
// at seg_base[b] + h tiles(b)), the per-wave share W and every wave's
// starting point, so that a partial wave begins with one load.  Thread t owns
// segments [t per, (t + 1) per); the inclusive scan of the threads' tile
// counts (lane exchanges within each wave, one barrier across the waves)
// locates the owner of any tile by binary search.
__device__ void plan_work(const DecodeArgs &a) {
  static_assert(kPrepThreads == 256, "four waves");
  __shared__ int part[kPrepThreads];
  __shared__ int first_len[kPrepThreads];
  __shared__ int wsum[4], wmax[4];
  WaveShare *share = reinterpret_cast<WaveShare *>(a.plan + 1);
  int *seg_base = reinterpret_cast<int *>(share + kMaxDecodeWaves);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int nseg = a.batch * a.hkv;
  const int per = (nseg + kPrepThreads - 1) / kPrepThreads;
  const int s0 = min(nseg, t * per), s1 = min(nseg, s0 + per);
  auto tiles = [](int len) { return (len + kDecodeStep - 1) / kDecodeStep; };
  int mine = 0, longest = 0, len0 = 0;
  for (int sg = s0, len = 0; sg < s1; ++sg) {
    if (sg == s0 || sg % a.hkv == 0) len = a.kv_len[sg / a.hkv];
    if (sg == s0) len0 = len;
    mine += tiles(len);
    longest = max(longest, len);
  }
  first_len[t] = len0;
  int incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) longest = max(longest, __shfl_xor(longest, o, 64));
  if (lane == 63) wsum[wave] = incl;
  if (lane == 0) wmax[wave] = longest;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) before += w < wave ? wsum[w] : 0;
  const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  const int most = tiles(max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3])));
  part[t] = before + incl;
  // W: every tile within n_waves shares, no segment cut into more than
  // kMaxPiecesPerSegment pieces (the merge reads one record per piece)
  const int W = max(max(kMinTilesPerWave, (total + a.n_waves - 1) / a.n_waves),
                    (most + kMaxPiecesPerSegment - 1) / kMaxPiecesPerSegment);
  {
    int base = before + incl - mine;
    for (int sg = s0, len = len0; sg < s1; ++sg) {
      if (sg % a.hkv == 0) {
        if (sg != s0) len = a.kv_len[sg / a.hkv];
        seg_base[sg / a.hkv] = base;
      }
      base += tiles(len);
    }
  }
  if (t == 0) {
    a.plan->total = total;
    a.plan->per_wave = W;
    seg_base[a.batch] = total;
  }
  __syncthreads();
  // Wave w starts at tile T = w W (no work when T >= total).  Thread t
  // serves waves t + k kPrepThreads; the owners of its KP starting tiles are
  // found by binary searches run in lockstep, so that their LDS reads overlap.
  constexpr int KP = kMaxDecodeWaves / kPrepThreads;
  int T[KP], u[KP];
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    T[k] = min(t + k * kPrepThreads, a.n_waves) * W;    // n_waves W stays below 2^31
    u[k] = 0;
  }
#pragma unroll
  for (int step = kPrepThreads / 2; step > 0; step >>= 1) {
#pragma unroll
    for (int k = 0; k < KP; ++k)
      if (part[u[k] + step - 1] <= T[k]) u[k] += step;   // the first thread whose inclusive sum exceeds T
  }
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    const int w = t + k * kPrepThreads;
    if (w >= a.n_waves) break;
    WaveShare sh{0, 0, 0, 0};
    if (T[k] < total) {
      const int o = u[k];
      int sg = o * per, at = o > 0 ? part[o - 1] : 0, len = first_len[o];
      while (T[k] >= at + tiles(len)) {    // only when a thread owns several segments
        at += tiles(len);
        ++sg;
        if (sg % a.hkv == 0) len = a.kv_len[sg / a.hkv];
      }
      sh = WaveShare{sg, T[k] - at, min(W, total - T[k]), len};
    }
    share[w] = sh;
  }
}

// Other workgroups: q~ for the G query heads of (sequence, KV head) r.  Each
// half-wave rotates one query head in registers: lane l of the half holds the
// D/32 consecutive coordinates from l D/32 (the SO(4) blocks stay inside a
// lane), the WHT runs its in-lane butterflies and then five lane-exchange
// stages, lower index first at every stage as in the Sylvester order.  One
// barrier, for the scale below.  `between` runs once the query and parameter
// loads are issued (the plan, where every workgroup computes it).
template <int D, int ROPE, int G, class Between>
__device__ void rotate_queries(const DecodeArgs &a, int r, Between &&between) {
  static_assert(kPrepThreads == 256 && G <= 8, "four waves, two heads each");
  constexpr int DQ = D + ROPE;
  constexpr int E = D / 32;                  // content coordinates per lane
  constexpr int ER = ROPE / 32;              // RoPE coordinates per lane
  constexpr int NBL = E / 4;                 // SO(4) blocks per lane
  static_assert(E % 4 == 0 && ROPE % 32 == 0, "lane layout");
  const int b = r / a.hkv, kvh = r - b * a.hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 31;
  const int hh = 2 * wave + (lane >> 5);     // query head of the group
  const bool act = hh < G;
  const size_t qoff = ((size_t)b * a.hq + kvh * G + (act ? hh : 0)) * DQ;
  float x[E], xr[ER > 0 ? ER : 1];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const size_t o = qoff + li * E + e;
    const float v = a.q_f16 ? static_cast<float>(static_cast<const _Float16 *>(a.q)[o]) : static_cast<const float *>(a.q)[o];
    x[e] = act ? v : 0.f;
  }
#pragma unroll
  for (int e = 0; e < ER; ++e) {
    const size_t o = qoff + D + li * ER + e;
    const float v = a.q_f16 ? static_cast<float>(static_cast<const _Float16 *>(a.q)[o]) : static_cast<const float *>(a.q)[o];
    xr[e] = act ? v * a.rmul : 0.f;
  }
  // this lane's block parameters (Full/Fast: q_L, q_R; Planar: two pair rotations)
  float4 prm[NBL][2];
  {
    const float4 *pg = reinterpret_cast<const float4 *>(a.quats + (size_t)kvh * (D / 4) * block_param_floats(a.variant));
#pragma unroll
    for (int k = 0; k < NBL; ++k) {
      const int blk = li * NBL + k;
      if (a.variant == kPlanar) {
        prm[k][0] = pg[blk];
        prm[k][1] = prm[k][0];
      } else {
        prm[k][0] = pg[2 * blk];
        prm[k][1] = pg[2 * blk + 1];
      }
    }
  }
  between();                                 // other work while the loads are in flight
#pragma unroll
  for (int st = 1; st < E; st <<= 1)
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (!(e & st)) {
        const float x0 = x[e], x1 = x[e + st];
        x[e] = x0 + x1;
        x[e + st] = x0 - x1;
      }
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) {
    const bool upper = li & m;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float y = __shfl_xor(x[e], m, 64);
      x[e] = upper ? y - x[e] : x[e] + y;
    }
  }
  const float scale = a.qmul / sqrtf((float)D);
#pragma unroll
  for (int k = 0; k < NBL; ++k) {
    const float4 v = make_float4(x[4 * k] * scale, x[4 * k + 1] * scale, x[4 * k + 2] * scale, x[4 * k + 3] * scale);
    const float4 t = a.variant == 0   ? so4_fwd<0>(v, prm[k][0], prm[k][1])
                     : a.variant == 1 ? so4_fwd<1>(v, prm[k][0], prm[k][1])
                                      : planar_fwd(v, prm[k][0]);
    x[4 * k] = t.x;
    x[4 * k + 1] = t.y;
    x[4 * k + 2] = t.z;
    x[4 * k + 3] = t.w;
  }
  // Power-of-two scale 2^f bringing the largest |q~| of the G heads into
  // [2^13, 2^14): the fp16 hi and lo parts then hold every coordinate down to
  // 2^-17 of the largest to 22 bits (unscaled, the small coordinates' lo
  // parts fall into the fp16 subnormals and lose most of their bits); the
  // partial kernel works in scores times 2^f and applies 2^-f where it needs
  // true units.
  __shared__ float redm[kPrepThreads / 64];
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) m = fmaxf(m, fabsf(x[e]));
#pragma unroll
  for (int e = 0; e < ER; ++e) m = fmaxf(m, fabsf(xr[e]));
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if (lane == 0) redm[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(redm[0], redm[1]), fmaxf(redm[2], redm[3]));
  const int f = m > 0.f ? 13 - ilogbf(m) : 0;
  const float up = ldexpf(1.f, f);
  _Float16 *dst = reinterpret_cast<_Float16 *>(a.qrot) + (size_t)r * 2 * G * DQ;
  if (act) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float v = x[e] * up;
      const _Float16 hi = static_cast<_Float16>(v);
      dst[hh * DQ + li * E + e] = hi;
      dst[(G + hh) * DQ + li * E + e] = static_cast<_Float16>(v - static_cast<float>(hi));
    }
#pragma unroll
    for (int e = 0; e < ER; ++e) {
      const float v = xr[e] * up;
      const _Float16 hi = static_cast<_Float16>(v);
      dst[hh * DQ + D + li * ER + e] = hi;
      dst[(G + hh) * DQ + D + li * ER + e] = static_cast<_Float16>(v - static_cast<float>(hi));
    }
  }
  if (threadIdx.x == 0) a.qscale[r] = ldexpf(1.f, -f);
}

// The plan for at most kPrepThreads segments, computed by every workgroup of
// the prep launch (thread t takes segment t; the segment lengths are a few
// cached loads): workgroup r of nwg writes the starts of waves r, r + nwg,
// ..., and the segment base of segment r's sequence if r is its first
// segment, so that no workgroup waits for another.
__device__ void plan_small(const DecodeArgs &a, int r, int nwg) {
  static_assert(kPrepThreads == 256, "four waves");
  __shared__ int part[kPrepThreads], lens[kPrepThreads];
  __shared__ int wsum[4], wmax[4];
  WaveShare *share = reinterpret_cast<WaveShare *>(a.plan + 1);
  int *seg_base = reinterpret_cast<int *>(share + kMaxDecodeWaves);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int nseg = a.batch * a.hkv;
  auto tiles = [](int len) { return (len + kDecodeStep - 1) / kDecodeStep; };
  const int len = t < nseg ? a.kv_len[t / a.hkv] : 0;
  const int mine = tiles(len);
  int incl = mine, longest = len;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) longest = max(longest, __shfl_xor(longest, o, 64));
  if (lane == 63) wsum[wave] = incl;
  if (lane == 0) wmax[wave] = longest;
  lens[t] = len;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) before += w < wave ? wsum[w] : 0;
  const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  const int most = tiles(max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3])));
  part[t] = before + incl;
  const int W = max(max(kMinTilesPerWave, (total + a.n_waves - 1) / a.n_waves),
                    (most + kMaxPiecesPerSegment - 1) / kMaxPiecesPerSegment);
  if (t == r && r % a.hkv == 0) seg_base[r / a.hkv] = before + incl - mine;
  if (r == 0 && t == 0) {
    a.plan->total = total;
    a.plan->per_wave = W;
    seg_base[a.batch] = total;
  }
  __syncthreads();
  for (int w = r + nwg * t; w < a.n_waves; w += nwg * kPrepThreads) {
    const int T = w * W;
    WaveShare sh{0, 0, 0, 0};
    if (T < total) {
      int u = 0;                             // the first segment whose inclusive sum exceeds T
#pragma unroll
      for (int step = kPrepThreads / 2; step > 0; step >>= 1)
        if (part[u + step - 1] <= T) u += step;
      sh = WaveShare{u, T - (part[u] - tiles(lens[u])), min(W, total - T), lens[u]};
    }
    share[w] = sh;
  }
}

// Up to kPrepThreads segments every workgroup plans (its share of the wave
// starts) and rotates the queries of one segment; beyond that workgroup 0
// plans alone.
__host__ __device__ inline bool plan_in_every_group(int batch, int hkv) { return batch * hkv <= kPrepThreads; }

template <int D, int ROPE, int G>
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(DecodeArgs a) {
  if (plan_in_every_group(a.batch, a.hkv)) {
    rotate_queries<D, ROPE, G>(a, (int)blockIdx.x, [&] { plan_small(a, (int)blockIdx.x, (int)gridDim.x); });
  } else if (blockIdx.x == 0) {
    plan_work(a);
  } else {
    rotate_queries<D, ROPE, G>(a, (int)blockIdx.x - 1, [] {});
  }
}

// ---------------------------------------------------------------------------
// partial kernel
// ---------------------------------------------------------------------------

template <int D, int BITS, int G, bool ARGMAX, int ROPE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(partial_waves<D, BITS, ROPE>())))
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
  constexpr int RK = ROPE / 32;              // k-steps of the RoPE score product
  constexpr int DQ = D + ROPE;               // query coordinates
  constexpr int NST = stage_count<D, BITS, ROPE>();
  static_assert((NST - 1) * S::LOADS < 64, "in-flight loads exceed the vmcnt range");
  constexpr int REPL = lut_repl<BITS>();
  constexpr int TB = lds_table_bytes<BITS>();
  constexpr bool kLateV = resident_groups<D, BITS, ROPE>() == 4;   // value operand after the softmax

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // lane exchanges at distances 16 and 32 without the lane index in the loop:
  // a swizzle inside each half-wave, and a permute with a fixed address
  // (head_dim 128 keeps the permute address in a register; at 256 and 512,
  // where every register is taken, it is recomputed)
  constexpr bool kSpare = D <= 128;          // registers to spare for such conveniences
  const int xaddr32 = (lane ^ 32) << 2;
  auto xor16 = [](auto v) {
    return __builtin_bit_cast(decltype(v), __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
  };
  auto xor32 = [&](auto v) {
    const int addr = kSpare ? xaddr32 : (((int)threadIdx.x & 63) ^ 32) << 2;
    return __builtin_bit_cast(decltype(v), __builtin_amdgcn_ds_bpermute(addr, __builtin_bit_cast(int, v)));
  };

  // the code-pair table, aligned to its own size so that an entry's offset
  // can be OR-ed into the lane's replica address
  __shared__ __attribute__((aligned(TB))) uint32_t lut[TB / 4];
  __shared__ __attribute__((aligned(16))) char smem[kDecodeWaves * NST * S::BYTES];
  for (int i = threadIdx.x; i < TB / 4; i += kThreads) lut[i] = a.lut[i / REPL];
  __syncthreads();                           // the kernel's only barrier: before any wave leaves

  // this wave's share of the tiles: `count` tiles from tile i0 of segment seg
  const int w = (int)blockIdx.x * kDecodeWaves + wave;
  const WaveShare my = reinterpret_cast<const WaveShare *>(a.plan + 1)[w];
  const int count = __builtin_amdgcn_readfirstlane(my.count);
  if (count <= 0) return;
  const int t_begin = 0, t_end = count;      // the share's tiles, counted from its first

  // A position in the tile sequence: sequence b, KV head h, tile i of the
  // segment's n tiles (len tokens).  Wave-uniform.
  struct Cursor {
    int b, h, i, n, len;
  };
  auto seq_len = [&](int b) { return __builtin_amdgcn_readfirstlane(a.kv_len[b]); };
  Cursor c0;
  {
    const int s = __builtin_amdgcn_readfirstlane(my.seg);
    c0.b = s / a.hkv;
    c0.h = s - c0.b * a.hkv;
    c0.len = __builtin_amdgcn_readfirstlane(my.len);
    c0.n = (c0.len + kDecodeStep - 1) / kDecodeStep;
    c0.i = __builtin_amdgcn_readfirstlane(my.i0);
  }
  // the next tile (one exists whenever this is called)
  auto advance = [&](Cursor &c) {
    if (++c.i < c.n) return;
    c.i = 0;
    if (++c.h < a.hkv) return;
    c.h = 0;
    do {
      ++c.b;
      c.len = seq_len(c.b);
    } while (c.len == 0);
    c.n = (c.len + kDecodeStep - 1) / kDecodeStep;
  };

  char *stages = smem + wave * NST * S::BYTES;
  const uint32_t stages_lds = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(stages));
  uint32_t goff[S::ROW_LOADS];
#pragma unroll
  for (int c = 0; c < S::ROW_LOADS; ++c) goff[c] = granule_offset<D, BITS>(c, lane);
  uint32_t groff[S::R_LOADS > 0 ? S::R_LOADS : 1];
#pragma unroll
  for (int c = 0; c < S::R_LOADS; ++c) groff[c] = rope_granule_offset<D, BITS, ROPE>(c, lane);
  // buffer resources of the segment the loads are in (rebuilt when the
  // loads move to the next segment)
  int32x4_t kr, vr, knr, vnr, rr;
  auto resources = [&](const Cursor &c) {
    const long long hrow = (long long)c.b * a.hkv + c.h;
    kr = make_rsrc(a.kc + hrow * a.kcap * ROWB, (uint32_t)(a.kcap * ROWB));
    vr = make_rsrc(a.vc + hrow * a.vcap * ROWB, (uint32_t)(a.vcap * ROWB));
    knr = make_rsrc(a.kn + hrow * a.kcap, (uint32_t)(a.kcap * 2));
    vnr = make_rsrc(a.vn + hrow * a.vcap, (uint32_t)(a.vcap * 2));
    rr = ROPE ? make_rsrc(a.krope + hrow * a.kcap * ROPE, (uint32_t)(a.kcap * ROPE * 2)) : kr;
  };
  // loads of the stage of tile c (out of range when !valid) into ring slot
  auto issue = [&](const Cursor &c, bool valid, int slot) {
    load_stage<D, BITS, ROPE>(stages_lds + slot * S::BYTES, kr, vr, knr, vnr, rr, c.i * kDecodeStep, valid, lane,
                              goff, groff);
  };
  // the load cursor's next tile (rebuilding the resources on a new segment)
  auto advance_loads = [&](Cursor &c) {
    const bool seg_end = c.i == c.n - 1;
    advance(c);
    if (seg_end) resources(c);
  };

  const int j = lane & 15;      // column of the score tile / row of the value operand
  const int g4 = lane >> 4;     // lane group: k-slice of the operands, row quad of results
  const bool live = j < NROW;
  const bool lo_lane = live && j >= G;
  const int head = j % G;

  // B operands of the score products, from the prep kernel's rows: k-step s
  // of lane group g4 holds dims 8 (s mod SPU) .. +7 of row unit 4 (s / SPU) +
  // g4 (the dims the K operand carries at the same k positions); RoPE k-step
  // s holds RoPE coordinates 32 s + 8 g4 .. +7.  Lanes past the live columns
  // hold zeros.
  half8 qB[KS];
  half8 qR[RK > 0 ? RK : 1];
  // the segment's query scale 2^-f: scores s' = 2^f s (log2 units) come out
  // of the products; the running maximum and its threshold stay in those
  // units, the weights and the record's maximum are taken back to true ones
  float qsc = 1.f, tau_s = kLazyTau, q4 = 0.25f;
  auto load_query = [&](const Cursor &c) {
    qsc = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                        __builtin_bit_cast(int, a.qscale[c.b * a.hkv + c.h])));
    tau_s = kLazyTau / qsc;
    q4 = 0.25f / qsc;
    const _Float16 *row = reinterpret_cast<const _Float16 *>(a.qrot) +
                          (((size_t)c.b * a.hkv + c.h) * 2 * G + (live ? j : 0)) * DQ;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int dim = (4 * (s / SPU) + g4) * (8 * SPU) + 8 * (s % SPU);
      const half8 v = *reinterpret_cast<const half8 *>(row + dim);
      qB[s] = live ? v : half8{};
    }
#pragma unroll
    for (int s = 0; s < RK; ++s) {
      const half8 v = *reinterpret_cast<const half8 *>(row + D + 32 * s + 8 * g4);
      qR[s] = live ? v : half8{};
    }
  };

  const int my_tile = lo_lane ? 1 : 0;
  const int vbit = VCB * j;                  // bit offset of this lane's codes in a row
  // -1 held in a register rather than as a literal, so that a weight's
  // remainder below stays one mixed-precision FMA (n_waves < 2^30)
  const float neg1 = -1.f - static_cast<float>(a.n_waves >> 30);
  constexpr int LSH = ilog2<REPL * 4>();     // table entry -> byte offset shift
  // A lane's value codes are taken VS bits early, so that in the interleaved
  // words below the first pair field already sits at the table shift (where
  // a group of 8 codes still fits a dword after it and no more dwords are
  // needed); the VS bits under it belong to the previous codes and are never
  // read.
  constexpr int VS = (LSH + 8 * BITS <= 32 && (VCB + LSH + 31) / 32 == VX) ? LSH : 0;
  const int vbs = vbit - VS;                 // lane 0: -VS, the dword before the row (still in LDS)
  // per-lane LDS byte offsets inside a stage
  const int k_off = S::K_OFF + j * S::RS + g4 * UDW * 4;
  const int v_off = S::V_OFF + 4 * g4 * S::RS + (vbs >> 5) * 4;
  const int n_off = (16 * my_tile + 4 * g4) * 2;
  // byte address of this lane's replica of table entry 0
  const uint32_t lut_base = lds_addr(lut) | (uint32_t)(lane % REPL) * 4u;
  // table entry at the 2*BITS-bit field at bit `pos` of w: the field is
  // shifted to bit LSH and masked, and the lane's replica offset OR-ed in: a
  // shift and one three-input bit operation, or the bit operation alone
  // where pos = LSH
  auto pair = [&](uint32_t w, auto pos) -> uint32_t {
    constexpr int P = decltype(pos)::value;
    constexpr uint32_t M = ((1u << (2 * BITS)) - 1u) << LSH;
    const uint32_t f = P >= LSH ? (w >> (P - LSH)) : (w << (LSH - P));
    const uint32_t addr = (f & M) | lut_base;
    return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t *>(addr);
  };

  float Mh, Mthr, Mb, Lh, best_s;           // Mthr = Mh + tau_s, the lazy rescale threshold
  int best_j;
  floatx4 O[NB];
  auto reset = [&] {
    Mh = -INFINITY;
    Mthr = -INFINITY;
    Mb = -INFINITY;
    Lh = 0.f;
    best_s = -INFINITY;
    best_j = -1;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) O[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
  };

  // Masking: score row r of this lane is token 16 my_tile + 4 g4 + r of the
  // tile; the score is fma(product, key norm, mbias[r]) with mbias 0 for a
  // live token and -inf otherwise (dead columns always; tokens past the end
  // of a segment in its last tile).  The biases change only at a segment's
  // last tile, so full tiles pay nothing for masking and one code path
  // serves both (a second inlined copy of the tile body would not fit the
  // register budget).
  const int tok0 = live ? 16 * my_tile + 4 * g4 : (1 << 30);
  float mbias[4];
  auto set_mask = [&](int limit) {          // tokens of the tile below `limit` are live
#pragma unroll
    for (int r = 0; r < 4; ++r) mbias[r] = tok0 + r < limit ? 0.f : -INFINITY;
  };
  set_mask(kDecodeStep);

  // One 32-token tile from the stage at LDS address `cur`: tokens t0 .. t0 +
  // 31 of a segment (masked by mbias).  Each operand's reads share one lane
  // base address, their constant offsets going into the instructions.
  auto process = [&](const uint32_t cur, const int t0) {
    // packed K rows of the two 16-token tiles (lane: token j, dims slice g4)
    const uint32_t kbase = cur + k_off;
    uint32_t kw[2][CW];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
#pragma unroll
      for (int m = 0; m < CW / UDW; ++m)
#pragma unroll
        for (int t = 0; t < UDW; ++t)
          kw[tile][m * UDW + t] = lds_ld<uint32_t>(kbase + tile * 16 * S::RS + (4 * m * UDW + t) * 4);
    }
    typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
    const uint32_t nbase = cur + n_off;
    const u16x4 kb = lds_ld<u16x4>(nbase + S::KN_OFF);
    const u16x4 vb = lds_ld<u16x4>(nbase + S::VN_OFF);

    // K operand: lane (token j, dims slice g4), k-step s holds dims 8s..8s+7
    // of the slice as 4 code pairs.
    uint32_t ka[2][KS][4];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      static_for<KS>([&](auto s) {
        static_for<4>([&](auto p) {
          constexpr int Wd = 2 * BITS;
          constexpr int sv = decltype(s)::value;
          constexpr int pos = (sv / SPU) * UDW * 32 + (8 * (sv % SPU) + 2 * decltype(p)::value) * BITS;
          constexpr int wd = pos >> 5, off = pos & 31;
          if constexpr (off + Wd <= 32 || wd + 1 >= CW)
            ka[tile][s][p] = pair(kw[tile][wd], std::integral_constant<int, off>{});
          else {
            // a pair across two dwords: the funnel shift also moves the field
            // to bit LSH, where the table read wants it
            static_assert(off >= LSH, "straddling field below the table shift");
            ka[tile][s][p] = pair(__builtin_amdgcn_alignbit(kw[tile][wd + 1], kw[tile][wd], off - LSH),
                                  std::integral_constant<int, LSH>{});
          }
        });
      });
    }
    // The value operand (the lane's value codes from the stage, their pair
    // interleave and table reads): built here, so that its table reads
    // overlap the score products and the softmax, or, in the four-wave
    // layout, after the softmax, in the registers the key operand has freed
    // (the other three waves of the SIMD cover the reads' latency).
    uint32_t vbw[NB][4];
    auto build_v = [&] {
    // the 8 tokens of this lane in the operand/result layouts: 4*g4 + r of each tile
    const uint32_t vbase = cur + v_off;
    uint32_t vch[8][VX];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      uint32_t w[VW];
#pragma unroll
      for (int i = 0; i < VW; ++i)                           // may read one dword past the row: still in LDS
        w[i] = lds_ld<uint32_t>(vbase + (16 * (r >> 2) + (r & 3)) * S::RS + 4 * i);
#pragma unroll
      for (int i = 0; i < VX; ++i) vch[r][i] = __builtin_amdgcn_alignbit(w[i + 1], w[i], vbs & 31);
    }
    // V operand: column block nb holds dims (D/16) * n + nb of lane column
    // n = j; dword p is the pair of tokens (2p, 2p+1) of the lane's 8
    // (code_a | code_b << BITS).  Per group of 8 column blocks the two tokens'
    // fields are interleaved first (SWAR): X[g][p][parity] holds the pair
    // indices of the group's dims of that parity at 2*BITS-bit strides.
    {
      constexpr int NGRP = NB / 8;
      constexpr uint32_t M = (1u << BITS) - 1u;
      constexpr uint32_t ME = (M | (M << (2 * BITS)) | (M << (4 * BITS)) | (M << (6 * BITS))) << VS;
      uint32_t X[NGRP][4][2];
      static_for<NGRP>([&](auto gi) {
        constexpr int bit0 = decltype(gi)::value * 8 * BITS, wd = bit0 >> 5, off = bit0 & 31;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          uint32_t ca, cb;
          if constexpr (off + 8 * BITS + VS <= 32) {
            ca = vch[2 * p][wd] >> off;
            cb = vch[2 * p + 1][wd] >> off;
          } else {
            ca = __builtin_amdgcn_alignbit(vch[2 * p][wd + 1], vch[2 * p][wd], off);
            cb = __builtin_amdgcn_alignbit(vch[2 * p + 1][wd + 1], vch[2 * p + 1][wd], off);
          }
          // bitwise selects (one v_bitop3_b32 each, truth table 0xCA = S0 ?
          // S1 : S2): the fields of ca under ME, those of cb shifted into
          // the gaps; only the group's 8 * BITS bits from bit VS are read
          // afterwards.  (Written as and/or, one of the two comes out as two
          // instructions once the compiler folds the later table masks.)
          X[gi][p][0] = __builtin_amdgcn_bitop3_b32(ME, ca, cb << BITS, 0xCA);
          X[gi][p][1] = __builtin_amdgcn_bitop3_b32(ME, ca >> BITS, cb, 0xCA);
        }
      });
      static_for<NB>([&](auto nb) {
        constexpr int nbv = decltype(nb)::value;
        constexpr int sh = ((nbv % 8) >> 1) * 2 * BITS + VS;
#pragma unroll
        for (int p = 0; p < 4; ++p) vbw[nb][p] = pair(X[nbv / 8][p][nbv & 1], std::integral_constant<int, sh>{});
      });
    }

    };
    if constexpr (!kLateV) build_v();

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
          const half8 kr8 = lds_ld<half8>(cur + S::R_OFF + (16 * tile + j) * S::RRS + (32 * s + 8 * g4) * 2);
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
      float c = fmaf(own + xor_g<G>(give), half_bits_to_float(kb[r]), mbias[r]);
      if constexpr (ROPE > 0) {
        const float rown = my_tile ? SR[1][r] : SR[0][r];
        const float rgive = my_tile ? SR[0][r] : SR[1][r];
        c += rown + xor_g<G>(rgive);
      }
      sig[r] = c;
      u[r] = fmaf((float)((vb[r] >> 8) & 0xFF), q4, c);
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
    if (__any(lmax > (kSpare ? Mthr : Mh + tau_s))) {
      float umax = fmaxf(lmax, xor_g<G>(lmax));
      umax = fmaxf(umax, xor16(umax));
      umax = fmaxf(umax, xor32(umax));
      const float mnew = fmaxf(Mh, umax);
      const float alpha = (Mh == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((Mh - mnew) * qsc);
      Lh *= alpha;
      Mh = mnew;
      Mthr = mnew + tau_s;
      Mb = mnew * qsc - kWeightBias;
      // rows 4*g4 + i of the value accumulators belong to head (4*g4 + i) % G
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * g4 + i;
        const float ar = __builtin_bit_cast(
            float, __builtin_amdgcn_ds_bpermute((row < NROW ? row % G : 0) << 2, __builtin_bit_cast(int, alpha)));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) O[nb][i] *= ar;
      }
    }
    float y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x = __builtin_amdgcn_exp2f(fmaf(sig[r], qsc, -Mb));   // 2^(s - M + bias); 0 for masked tokens
      Lh += x;
      y[r] = live ? fmaf(x, half_bits_to_float(vb[r]), 0.f) : 0.f;   // x ||v||, one mixed-precision FMA
    }
    // A operand, k order = tile-0 tokens 4*g4..+3 then tile-1 tokens; row j
    // < G carries the fp16 hi parts (round toward zero) of head j's weights,
    // row G + j the exact remainders.  Each lane splits its own tile's two
    // weight pairs once and hands its partner (lane ^ G, which owns the other
    // tile) the part the partner's row carries.
    uint32_t pw[4];
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      const auto h = __builtin_amdgcn_cvt_pkrtz(y[2 * q2], y[2 * q2 + 1]);
      const float d0 = fmaf(neg1, static_cast<float>(h[0]), y[2 * q2]);
      const float d1 = fmaf(neg1, static_cast<float>(h[1]), y[2 * q2 + 1]);
      const uint32_t hw = __builtin_bit_cast(uint32_t, h);
      const uint32_t lw = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(d0, d1));
      const uint32_t got =
          __builtin_bit_cast(uint32_t, xor_g<G>(__builtin_bit_cast(float, lo_lane ? hw : lw)));
      pw[q2] = lo_lane ? got : hw;         // tile 0: a hi lane's own, a lo lane's from its partner
      pw[2 + q2] = lo_lane ? lw : got;     // tile 1: a lo lane's own, a hi lane's from its partner
    }
    const half8 P = as_half8(pw[0], pw[1], pw[2], pw[3]);
    if constexpr (kLateV) {
      __builtin_amdgcn_sched_barrier(0);     // nothing of the value operand moves above this point
      build_v();
    }

    // values
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      O[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(P, as_half8(vbw[nb][0], vbw[nb][1], vbw[nb][2], vbw[nb][3]),
                                                     O[nb], 0, 0, 0);
  };

  // The record of the piece of segment (c.b, c.h) this wave has covered: per
  // query head the softmax state and o~ (hi + lo rows added), straight from
  // registers.  Record index: segment + wave.
  auto write_record = [&](const Cursor &c) {
    float lsum = live ? Lh : 0.f;
    lsum += xor_g<G>(lsum);
    lsum += xor16(lsum);
    lsum += xor32(lsum);
    float bs = live ? best_s : -INFINITY;
    int bj = live ? best_j : -1;
    if constexpr (ARGMAX) {
      // the larger score; on equal scores the lower position
      auto take = [&](float os, int oj) {
        if (os > bs || (os == bs && oj >= 0 && (bj < 0 || oj < bj))) {
          bs = os;
          bj = oj;
        }
      };
      take(xor_g<G>(bs), __builtin_bit_cast(int, xor_g<G>(__builtin_bit_cast(float, bj))));
      take(xor16(bs), xor16(bj));
      take(xor32(bs), xor32(bj));
    }
    const long long piece = (long long)c.b * a.hkv + c.h + w;
    float *rec = a.ws + piece * G * (D + kRecHeader);
    // (the best score stays in the segment's scaled units: the merge only
    // compares the pieces of one segment)
    if (lane < G)
      *reinterpret_cast<float4 *>(rec + lane * (D + kRecHeader)) =
          make_float4(Mh * qsc, lsum, bs, __builtin_bit_cast(float, bj));
    // value rows: hi row h + lo row h + G; lane (j, g4) holds rows 4 g4 + i,
    // columns (D/16) j .. +NB-1; one row (i) at a time, four columns per store
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * g4 + i;
      float *dst = rec + row * (D + kRecHeader) + kRecHeader + (D / 16) * j;
#pragma unroll
      for (int q = 0; q < NB / 4; ++q) {
        float v4[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float v = O[4 * q + k][i];
          if constexpr (G == 4)
            v4[k] = v + xor16(v);
          else if constexpr (G == 8)
            v4[k] = v + xor32(v);
          else
            v4[k] = v + O[4 * q + k][i ^ G];
        }
        if (row < G) *reinterpret_cast<float4 *>(dst + 4 * q) = make_float4(v4[0], v4[1], v4[2], v4[3]);
      }
    }
  };

  // ---- main loop ---------------------------------------------------------------
  // Ring of NST stages: the next NST - 1 tiles are in flight while one is
  // processed.  Every iteration issues one stage (out of range past the
  // wave's last tile), so one fixed wait finds the oldest stage landed; other
  // memory operations in between only make that wait longer, never short.
  // At a segment boundary the next query rows are loaded and everything in
  // flight is awaited.
  Cursor cp = c0, ca = c0;                   // tile processed, tile loaded next
  int ta = t_begin;
  reset();
  resources(ca);
#pragma unroll
  for (int i = 0; i < NST - 1; ++i) {
    issue(ca, ta < t_end, i);
    if (ta + 1 < t_end) advance_loads(ca);
    ++ta;
  }
  // the first query rows, then one wait that the compiler sees (it also
  // lands the first stages, which the first tile needs anyway)
  load_query(cp);
  wait_vmem<0>();
  int slot = 0;                              // stage of tile tp
  for (int tp = t_begin; tp < t_end; ++tp) {
    const int aslot = slot == 0 ? NST - 1 : slot - 1;       // (tp + NST - 1) mod NST, processed last iteration
    issue(ca, ta < t_end, aslot);
    if (ta + 1 < t_end) advance_loads(ca);
    ++ta;
    wait_vmem<(NST - 1) * S::LOADS>();
    const bool seg_last = cp.i == cp.n - 1;
    const int tail = cp.len - cp.i * kDecodeStep;       // tokens of the segment from this tile on
    if (seg_last && tail < kDecodeStep) set_mask(tail);
    process(stages_lds + slot * S::BYTES, cp.i * kDecodeStep);
    if (seg_last || tp + 1 == t_end) write_record(cp);
    if (tp + 1 < t_end) {
      advance(cp);
      if (seg_last) {
        if (tail < kDecodeStep) set_mask(kDecodeStep);
        load_query(cp);
        wait_vmem<0>();
        reset();
      }
    }
    slot = slot == NST - 1 ? 0 : slot + 1;
  }
  wait_vmem<0>();                            // no load into LDS may outlive the wave
}

// ---------------------------------------------------------------------------
// merge kernel
// ---------------------------------------------------------------------------

constexpr int kMergeChunk = kMaxPiecesPerSegment + 8;   // pieces of one segment the merge holds in LDS
static_assert(kMaxPiecesPerSegment + 1 <= kMergeChunk, "a segment's pieces fit the merge's LDS");
constexpr int kMergeThreads = 256;

// One workgroup per (query head, sequence).  Thread t sums four neighbouring
// coordinates (one 16-byte load per record) over every NP-th piece, so that
// many loads are in flight however few or many pieces the segment has.
template <int D, int VARIANT>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
  constexpr int RS = D + kRecHeader;
  constexpr int NT = kMergeThreads;
  constexpr int C4 = D / 4;                  // float4 columns of o~
  constexpr int NP = NT / C4;                // parts
  static_assert(NT % C4 == 0 && RS % 4 == 0, "merge geometry");
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int G = a.group;
  const int g = h / G, hh = h - g * G;
  const int tid = threadIdx.x;
  const int c = tid % C4, part = tid / C4;
  // the records of this segment's pieces: s + first .. s + last, G records apart
  const int *seg_base = reinterpret_cast<const int *>(reinterpret_cast<const WaveShare *>(a.plan + 1) +
                                                      kMaxDecodeWaves);
  const int nt = (seg_base[b + 1] - seg_base[b]) / a.hkv;      // tiles per KV head of sequence b
  const int W = a.plan->per_wave;
  const long long s = (long long)b * a.hkv + g;
  int n = 0;
  const float *recs = a.ws;
  if (nt > 0) {
    const int S0 = seg_base[b] + g * nt;
    const int first = S0 / W, last = (S0 + nt - 1) / W;
    n = min(last - first + 1, kMergeChunk);   // at most kMaxPiecesPerSegment + 1 by the plan's W
    recs = a.ws + ((s + first) * G + hh) * RS;
  }
  const size_t stride = (size_t)G * RS;       // from one piece's record to the next
  constexpr int NW = NT / 64;                // waves of the workgroup
  __shared__ float redf[NW];
  __shared__ int redi[NW];
  __shared__ float reds[NW];
  __shared__ float hm[kMergeChunk], hl[kMergeChunk];      // each piece's M and L
  __shared__ __attribute__((aligned(16))) float part_o[NP][D];
  __shared__ __attribute__((aligned(16))) float y[D];
  const int lane = tid & 63, wave = tid >> 6;
  // (score, position) pairs: the larger score, ties to the lower valid position
  auto better = [](float s1, int p1, float s0, int p0) {
    return s1 > s0 || (s1 == s0 && p1 >= 0 && (p0 < 0 || p1 < p0));
  };
  // the coordinates of this thread's first KPF records, requested before the
  // headers are reduced (they do not depend on them); deeper prefetching
  // costs registers, and below 64 per lane a one-round grid of 2,048
  // workgroups (64 sequences x 32 heads) still fits the chip
  constexpr int KPF = 4;
  const float4 *col = reinterpret_cast<const float4 *>(recs + kRecHeader) + c;
  const size_t stride4 = stride / 4;
  float4 pre[KPF];
#pragma unroll
  for (int k = 0; k < KPF; ++k) {
    const int p = part + k * NP;
    pre[k] = p < n ? col[(size_t)p * stride4] : make_float4(0.f, 0.f, 0.f, 0.f);
  }

  // Headers are read in parallel (thread t: records t, t + NT, ...) and kept
  // in LDS: the running maximum and the best score with its position (ties:
  // the lower position; pieces cover increasing positions).  Reductions:
  // across the wave by lane exchanges, then across the waves through LDS.
  float Mt = -INFINITY, bt = -INFINITY;
  int at = -1;
  for (int p = tid; p < n; p += NT) {
    const float4 hd = *reinterpret_cast<const float4 *>(recs + (size_t)p * stride);
    hm[p] = hd.x;
    hl[p] = hd.y;
    if (hd.y > 0.f) {
      Mt = fmaxf(Mt, hd.x);
      const int pos = __builtin_bit_cast(int, hd.w);
      if (better(hd.z, pos, bt, at)) {
        bt = hd.z;
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
    reds[wave] = bt;
  }
  __syncthreads();
  float M = redf[0], bsc = reds[0];
  int arg = redi[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    M = fmaxf(M, redf[w]);
    if (better(reds[w], redi[w], bsc, arg)) {
      bsc = reds[w];
      arg = redi[w];
    }
  }
  __syncthreads();                           // redf is reused below

  // Weights 2^(M_p - M) (0 for empty pieces) from the headers in LDS; each
  // thread sums its four coordinates over its part's records, and the parts
  // are added in LDS.
  auto weight = [&](int p) { return hl[p] > 0.f ? exp2f(hm[p] - M) : 0.f; };
  float Lt = 0.f;
  for (int p = tid; p < n; p += NT) Lt += hl[p] > 0.f ? hl[p] * weight(p) : 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add = [&](float w, const float4 &v) {
    o.x += w > 0.f ? v.x * w : 0.f;
    o.y += w > 0.f ? v.y * w : 0.f;
    o.z += w > 0.f ? v.z * w : 0.f;
    o.w += w > 0.f ? v.w * w : 0.f;
  };
#pragma unroll
  for (int k = 0; k < KPF; ++k) {
    const int p = part + k * NP;
    if (p < n) add(weight(p), pre[k]);
  }
#pragma unroll 4
  for (int p = part + KPF * NP; p < n; p += NP) add(weight(p), col[(size_t)p * stride4]);
  *reinterpret_cast<float4 *>(&part_o[part][4 * c]) = o;
  for (int m = 32; m > 0; m >>= 1) Lt += __shfl_xor(Lt, m, 64);
  if (lane == 0) redf[wave] = Lt;
  __syncthreads();
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) L += redf[w];
  for (int i = tid; i < D; i += NT) {
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < NP; ++q) sum += part_o[q][i];
    y[i] = L > 0.f ? sum * a.oscale / L : 0.f;
  }
  __syncthreads();
  // R^T in one half-wave, in registers: lane l holds the D/32 consecutive
  // coordinates from l D/32 (whole inverse blocks), then the WHT's in-lane
  // butterflies and five lane-exchange stages, lower index first at every
  // stage as in the Sylvester order; no barrier.
  const size_t oh = (size_t)b * a.hq + h;
  if (tid < 32) {
    constexpr int E = D / 32;
    const float *pg = a.quats + (size_t)g * (D / 4) * block_param_floats(VARIANT);
    float x[E];
#pragma unroll
    for (int k = 0; k < E / 4; ++k) {
      const float4 u = block_inv<VARIANT>(*reinterpret_cast<const float4 *>(&y[tid * E + 4 * k]), pg,
                                          tid * (E / 4) + k);
      x[4 * k] = u.x;
      x[4 * k + 1] = u.y;
      x[4 * k + 2] = u.z;
      x[4 * k + 3] = u.w;
    }
#pragma unroll
    for (int st = 1; st < E; st <<= 1)
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (!(e & st)) {
          const float x0 = x[e], x1 = x[e + st];
          x[e] = x0 + x1;
          x[e + st] = x0 - x1;
        }
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) {
      const bool upper = tid & m;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float v = __shfl_xor(x[e], m, 64);
        x[e] = upper ? v - x[e] : x[e] + v;
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float val = x[e] / sqrtf((float)D);
      if (a.out_f16)
        static_cast<_Float16 *>(a.out)[oh * D + tid * E + e] = static_cast<_Float16>(val);
      else
        static_cast<float *>(a.out)[oh * D + tid * E + e] = val;
    }
  }
  if (tid == 0) {
    if (a.lse) a.lse[oh] = L > 0.f ? (M - kWeightBias + log2f(L)) * 0.69314718055994531f : -INFINITY;
    if (a.argmax) a.argmax[oh] = L > 0.f ? arg : -1;
  }
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------

// Whether the pair table and a ring of two stages per wave fit in one
// compute unit's LDS (every shape without RoPE coordinates does; with them
// head_dim 512 at 4 bits does not).
template <int D, int BITS, int ROPE>
constexpr bool partial_fits() {
  return lds_table_bytes<BITS>() + kDecodeWaves * 2 * Stage<D, BITS, ROPE>::BYTES <= 160 * 1024;
}

template <int D, int ROPE>
hipError_t prep_dispatch(const DecodeArgs &a, hipStream_t s) {
  const dim3 grid((plan_in_every_group(a.batch, a.hkv) ? 0u : 1u) + (unsigned)(a.batch * a.hkv));
  switch (a.group) {
    case 1: hipLaunchKernelGGL((prep_kernel<D, ROPE, 1>), grid, dim3(kPrepThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((prep_kernel<D, ROPE, 2>), grid, dim3(kPrepThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((prep_kernel<D, ROPE, 4>), grid, dim3(kPrepThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL((prep_kernel<D, ROPE, 8>), grid, dim3(kPrepThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, int BITS, bool ARGMAX, int ROPE>
hipError_t partial_dispatch_group(const DecodeArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)(a.n_waves / kDecodeWaves));
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
  hipError_t e = prep_dispatch<D, ROPE>(a, s);
  if (e != hipSuccess) return e;
  return a.argmax ? partial_dispatch_group<D, BITS, true, ROPE>(a, s)
                  : partial_dispatch_group<D, BITS, false, ROPE>(a, s);
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

// Workgroups of the partial kernel resident on one compute unit (one wave
// per SIMD each): the smaller of what LDS and the register budget allow.
template <int D, int BITS, int ROPE>
constexpr int groups_per_cu() {
  return resident_groups<D, BITS, ROPE>() < partial_waves<D, BITS, ROPE>() ? resident_groups<D, BITS, ROPE>()
                                                                             : partial_waves<D, BITS, ROPE>();
}

template <int D, int ROPE = 0>
int partial_groups_per_cu(int bits) {
  switch (bits) {
    case 2: return groups_per_cu<D, 2, ROPE>();
    case 3: return groups_per_cu<D, 3, ROPE>();
    case 4: return groups_per_cu<D, 4, ROPE>();
  }
  return 1;
}

template <int D>
hipError_t merge_dispatch(int variant, const MergeArgs &a, hipStream_t s) {
  dim3 grid((unsigned)a.hq, (unsigned)a.batch);
  switch (variant) {
    case 0: hipLaunchKernelGGL((merge_kernel<D, 0>), grid, dim3(kMergeThreads), 0, s, a); break;
    case 1: hipLaunchKernelGGL((merge_kernel<D, 1>), grid, dim3(kMergeThreads), 0, s, a); break;
    case kPlanar: hipLaunchKernelGGL((merge_kernel<D, kPlanar>), grid, dim3(kMergeThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace
}  // namespace iq
