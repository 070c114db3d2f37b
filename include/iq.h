/*
 * iq.h -- C ABI of the MI355X (gfx950) IsoQuant packed-KV library (libiq.so).
 *
 * What is computed (the operations are defined on the pages of
 * "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
 * Compressed-Space Attention", arXiv 2608.08081, and "IsoQuant:
 * Hardware-Aligned SO(4) Isoclinic Rotations for LLM KV Cache Compression",
 * arXiv 2603.28430):
 *
 *   quantize (RotaryQuant §3.2, Algorithm 1 and eq. (2)):
 *     s = ||x||_2, x^ = x / s, x~ = R_SO(4)(H_d x^), codes = LloydMax(x~),
 *     row = BitPack_b(codes), norm = fp16(s).
 *     R_SO(4) acts on contiguous 4-element blocks seen as quaternions:
 *     Full: v -> q_L v conj(q_R); Fast: v -> q_L v (IsoQuant abstract).
 *     Planar, the framework's 2-D special case: each coordinate pair, seen as
 *     a complex number, times a unit complex number.
 *   dequantize (RotaryQuant §3.4: R^-1 = R^T via the same butterfly and the
 *     block transpose): x' = fp16(s) * H_d R_SO(4)^T c[codes].
 *   decode attention (RotaryQuant §3.4 Table 2 and Appendix A): q~ = R q once
 *     per query head, scores and an online softmax on the packed K rows in
 *     rotated space, value accumulation on the packed V rows in rotated space,
 *     one R^T on the aggregated output.  No fp16/fp32 K or V is written.
 *   RoPE sub-block (RotaryQuant §5, the MLA/RoPE limitation): keys whose last
 *     coordinates are RoPE coordinates keep those unrotated and unquantised
 *     in fp16; their dot product with the query's RoPE part joins the score.
 *
 * Conventions shared by every entry point
 *   - Every pointer is DEVICE memory owned by the caller unless marked HOST.
 *     The library never allocates device memory and keeps no mutable global
 *     state (except iq_decode_attention_noalloc's fixed workspace array and
 *     its per-device address); calls on different streams may run
 *     concurrently (except iq_decode_attention_noalloc calls, see there).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without host synchronisation.
 *   - Arguments are validated before anything is enqueued; a negative
 *     iq_status is returned and nothing runs.  Launch failures return
 *     IQ_ERR_HIP.  Values that live in device memory (start_pos, kv_len) cannot
 *     be checked without a synchronisation: keeping every row index inside
 *     [0, capacity) is the caller's precondition.  NaN/Inf inputs and norms
 *     above 65504 (fp16 overflow of the stored scale) are outside the contract.
 *   - No C++ exception crosses this interface.
 *
 * Data layout
 *   head vectors x      [batch][n][H_kv][d]              fp32 or fp16
 *   quaternions         [H_kv][d/4][2][4] fp32, (w,x,y,z), q_L then q_R, unit
 *                       length; one rotation per KV head shared by K, V and the
 *                       query heads of that group (RotaryQuant Appendix A).
 *                       Planar: [H_kv][d/2][2] fp32 (cos, sin).
 *   packed codes        [batch][H_kv][capacity][d*b/8]   uint8
 *                       LSB-first bitstream: bit r of code i is bit (b*i + r)
 *                       of the row, bytes little-endian (d*b/8 = 48 bytes at
 *                       d = 128, b = 3, RotaryQuant §3.2 Step 4).
 *   norms               [batch][H_kv][capacity]          IEEE fp16 bits
 *   RoPE side cache     [batch][H_kv][capacity][r]       IEEE fp16 bits
 *   queries / outputs   [batch][Hq][d]                   fp32 or fp16
 *   code of a value v:  number of thresholds t_k = (c_k + c_{k+1})/2 with
 *                       v > t_k (ascending centroids c).
 */
#ifndef IQ_H
#define IQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  IQ_OK = 0,
  IQ_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, bad enum value */
  IQ_ERR_UNSUPPORTED = -2, /* d, b, group size, dtype or shape outside the built
                              set, or (decode) a codebook the fp16 matrix cores
                              cannot hold exactly */
  IQ_ERR_MISALIGNED = -3,  /* a base pointer is not 16-byte aligned */
  IQ_ERR_WORKSPACE = -4,   /* workspace smaller than iq_decode_workspace_bytes */
  IQ_ERR_HIP = -5          /* a HIP runtime call or kernel launch failed */
} iq_status;

/* Block rotation applied after the WHT (IsoQuant abstract): Full is the SO(4)
 * map v -> q_L v conj(q_R) on 4-D blocks, Fast keeps the left factor
 * v -> q_L v, Planar is the framework's 2-D special case: each coordinate
 * pair (x[2i], x[2i+1]), read as a complex number, is multiplied by a unit
 * complex number (one SO(2) rotation per pair). */
typedef enum { IQ_FULL = 0, IQ_FAST = 1, IQ_PLANAR = 2 } iq_variant;
typedef enum { IQ_F32 = 0, IQ_F16 = 1 } iq_dtype;

/* Per-layer quantiser configuration (a HOST struct). */
typedef struct {
  int32_t head_dim;        /* d: 128, 256 or 512 */
  int32_t bits;            /* b: 2, 3 or 4 */
  int32_t variant;         /* iq_variant; Fast reads q_L only */
  int32_t num_kv_heads;    /* H_kv >= 1 */
  const float *quats;      /* DEVICE fp32 block-rotation parameters, used as
                              given (no renormalisation): Full and Fast
                              [H_kv][d/4][2][4] unit quaternions (q_L, q_R),
                              each (w, x, y, z); Planar [H_kv][d/2][2] unit
                              complex numbers (cos, sin) */
  const float *centroids;  /* HOST [2^b] fp32, strictly ascending and finite
                              (else IQ_ERR_INVALID_ARG).  The decode entry
                              points also need every level, times the power
                              of two 2^e that brings the largest magnitude
                              into [1, 2), to be an fp16 number exactly: they
                              multiply the levels on fp16 matrix cores.  Levels
                              with at most 11 significant bits (iq_codebook's)
                              meet this whenever max/min nonzero magnitude is
                              below 2^14; otherwise the decode entry points
                              return IQ_ERR_UNSUPPORTED (and
                              iq_decode_workspace_bytes 0), while quantize and
                              dequantize take any such codebook. */
} iq_config;

/* One packed tensor (K or V) of a KV cache (a HOST struct). */
typedef struct {
  uint8_t *codes;          /* DEVICE [batch][H_kv][capacity][d*b/8], 16-B aligned */
  uint16_t *norms;         /* DEVICE [batch][H_kv][capacity] fp16 bits, 16-B aligned */
  int64_t capacity;        /* rows per (sequence, KV head), >= 1 */
} iq_cache;

/* Lloyd-Max codebook for the coordinates of a rotated unit vector, taken as
 * N(0, 1/d) (RotaryQuant §3.2 Step 3: minimum expected distortion under the
 * post-rotation marginal).  Runs the Lloyd iteration for N(0,1) in double on
 * the host, scales by 1/sqrt(d) and rounds each level to 11 significant bits
 * (ties to even): the codebook is held at fp16 precision so that the decode
 * kernel's fp16 matrix operands represent every level exactly.
 *   centroids_out: HOST array of 2^bits floats, written in ascending order.
 * Returns IQ_OK, IQ_ERR_INVALID_ARG (null) or IQ_ERR_UNSUPPORTED (bits, d). */
int iq_codebook(int32_t bits, int32_t head_dim, float *centroids_out);

/* Quantize and append (RotaryQuant Algorithm 1; appends as in §3.4 "deferred
 * prefill" and Appendix D: each new K or V vector is compressed on arrival).
 *   x:         [batch][n_new][H_kv][d] of x_dtype (IQ_F32 or IQ_F16).
 *   start_pos: DEVICE int32 [batch]; vector t of sequence b is written to row
 *              start_pos[b] + t of `out`.  The library does not advance it.
 *   out:       the packed tensor written (codes and norms).
 * batch * n_new must stay below 2^31 - 2^20 (IQ_ERR_INVALID_ARG otherwise;
 * an input that large would not fit in device memory anyway).
 * K and V are two calls on two caches that share one iq_config (or one
 * iq_quantize_append_many call). */
int iq_quantize_append(const iq_config *cfg, const void *x, int32_t x_dtype,
                       int32_t batch, int32_t n_new, const int32_t *start_pos,
                       const iq_cache *out, hipStream_t stream);

/* iq_quantize_append for `count` tensors of the same shape in one go, e.g.
 * the K and V buffers of every layer at the prefill -> decode boundary
 * (RotaryQuant §3.4 deferred prefill, Appendix C): tensor i quantises xs[i]
 * with cfgs[i] into outs[i].  One launch covers up to 16 tensors.
 *   cfgs:      HOST array of `count` configs with equal head_dim, bits,
 *              variant, num_kv_heads and centroid values (each its own
 *              rotation); IQ_ERR_INVALID_ARG otherwise.
 *   xs:        HOST array of `count` DEVICE pointers, each
 *              [batch][n_new][H_kv][d] of x_dtype, 16-B aligned.
 *   outs:      HOST array of `count` caches (capacities may differ).
 *   start_pos: DEVICE int32 [batch], the rows of every tensor.
 * Other arguments and errors as iq_quantize_append; the results are those of
 * `count` iq_quantize_append calls. */
int iq_quantize_append_many(const iq_config *cfgs, int32_t count, const void *const *xs,
                            int32_t x_dtype, int32_t batch, int32_t n_new,
                            const int32_t *start_pos, const iq_cache *outs,
                            hipStream_t stream);

/* Quantize and append keys with a RoPE sub-block (RotaryQuant §5, the
 * MLA/RoPE limitation: positional coordinates must be neither rotated nor
 * quantised).  Each key is (content, positional) with the rope_dim RoPE
 * coordinates last; the content part (d coordinates) is quantised exactly as
 * by iq_quantize_append (its own norm, rotation and codes), the RoPE part is
 * stored unrotated and unquantised as fp16 (round to nearest even).
 *   x:         [batch][n_new][H_kv][d + rope_dim] of x_dtype, 16-B aligned.
 *   rope_dim:  multiple of 8, 8 .. 512 (IQ_ERR_UNSUPPORTED otherwise; decode
 *              attention takes 64).
 *   rope_out:  DEVICE [batch][H_kv][out->capacity][rope_dim] fp16 bits,
 *              16-B aligned; row start_pos[b] + t receives vector t's RoPE
 *              coordinates, like `out`.
 * Other arguments and errors as iq_quantize_append.  Values have no RoPE part
 * and use iq_quantize_append. */
int iq_quantize_append_rope(const iq_config *cfg, const void *x, int32_t x_dtype,
                            int32_t batch, int32_t n_new, int32_t rope_dim,
                            const int32_t *start_pos, const iq_cache *out,
                            uint16_t *rope_out, hipStream_t stream);

/* Dequantize n rows per (sequence, KV head) starting at start_pos[b]
 * (the stage-1 return path of the IsoQuant abstract; inverse of RotaryQuant
 * eq. (2) as in §3.4):  out[b][t][h][:] = fp16(s) * R^T c[codes].
 *   start_pos: DEVICE int32 [batch].
 *   out:       [batch][n][H_kv][d] of out_dtype.
 * batch * n must stay below 2^31 - 2^20 (IQ_ERR_INVALID_ARG otherwise). */
int iq_dequantize(const iq_config *cfg, const iq_cache *in, int32_t batch,
                  const int32_t *start_pos, int32_t n, void *out,
                  int32_t out_dtype, hipStream_t stream);

/* Bytes of workspace iq_decode_attention needs for these sizes.  Returns 0 if
 * the arguments are invalid.  A work plan (64 KiB plus 4 bytes per sequence),
 * the rotated queries (about 4 (d + 64) bytes per query head), and
 * (batch * H_kv + 4096) * (Hq / H_kv) partial records of d + 4 floats; the
 * size does not depend on max_kv_len and is never O(T * d) -- the decode
 * path writes no dequantized K or V, the
 * zero-materialization property RotaryQuant Appendix D confirms with its
 * instrumentation counters (no decompress or key-read calls). */
size_t iq_decode_workspace_bytes(const iq_config *cfg, int32_t batch,
                                 int32_t num_q_heads, int64_t max_kv_len);

/* Decode attention on packed K/V (RotaryQuant §3.4 Table 2, Appendix A).
 * Equivalent to iq_decode_attention_partial followed by
 * iq_decode_attention_merge on the same stream and workspace.
 * One query token per sequence; query head h reads KV head h / (Hq / H_kv);
 * batch at most 65535 (IQ_ERR_UNSUPPORTED otherwise).
 *   q:          [batch][Hq][d] of q_dtype.
 *   k, v:       packed caches written by iq_quantize_append with this cfg.
 *   kv_len:     DEVICE int32 [batch]; attends rows [0, kv_len[b]) (includes a
 *               token appended this step).  kv_len[b] = 0 gives out = 0,
 *               lse = -inf, argmax = -1.
 *   max_kv_len: HOST upper bound of kv_len, used for the grid only; every
 *               kv_len[b] must be <= max_kv_len (rows at and past kv_len[b]
 *               do not affect the results).  Each cache's capacity must
 *               be even and capacity * d*b/8 below 2^30 bytes
 *               (IQ_ERR_UNSUPPORTED otherwise).
 *   softmax_scale: multiplies q.k (1/sqrt(d) in Appendix A).
 *   out:        [batch][Hq][d] of out_dtype, in the original (un-rotated)
 *               domain.
 *   lse_out:    nullable, [batch][Hq] fp32 natural-log sum of exp(scores).
 *   argmax_out: nullable, [batch][Hq] int32 position of the largest score
 *               (ties: lowest position).
 *   workspace:  at least iq_decode_workspace_bytes(...) bytes, 16-B aligned;
 *               its content on entry does not matter. */
int iq_decode_attention(const iq_config *cfg, const void *q, int32_t q_dtype,
                        int32_t batch, int32_t num_q_heads,
                        const iq_cache *k, const iq_cache *v,
                        const int32_t *kv_len, int64_t max_kv_len,
                        float softmax_scale, void *out, int32_t out_dtype,
                        float *lse_out, int32_t *argmax_out,
                        void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

/* iq_decode_attention for keys with a RoPE sub-block (RotaryQuant §5, the
 * MLA/RoPE limitation), written by iq_quantize_append_rope: the score of
 * token j is softmax_scale * (q_content . k_j + q_rope . k_rope_j), where k_j
 * is the content key held packed in k (attended in rotated space as in
 * iq_decode_attention) and k_rope_j its fp16 RoPE coordinates, neither
 * rotated nor scaled by the content norm.  Values have no RoPE part.
 *   q:        [batch][Hq][d + rope_dim] of q_dtype, RoPE coordinates last.
 *   k_rope:   DEVICE [batch][H_kv][k->capacity][rope_dim] fp16 bits, 16-B
 *             aligned; k->capacity * rope_dim * 2 below 2^30 bytes.
 *   rope_dim: 64 (IQ_ERR_UNSUPPORTED otherwise), with any head_dim and bit
 *             width except head_dim 512 at 4 bits (IQ_ERR_UNSUPPORTED).
 *   out:      [batch][Hq][d] (the content coordinates).
 * Other arguments, workspace and errors as iq_decode_attention. */
int iq_decode_attention_rope(const iq_config *cfg, const void *q, int32_t q_dtype,
                             int32_t batch, int32_t num_q_heads,
                             const iq_cache *k, const uint16_t *k_rope, int32_t rope_dim,
                             const iq_cache *v, const int32_t *kv_len, int64_t max_kv_len,
                             float softmax_scale, void *out, int32_t out_dtype,
                             float *lse_out, int32_t *argmax_out,
                             void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Split phase of iq_decode_attention (the context is cut into pieces, as in
 * FlashAttention's tiling that RotaryQuant §2 cites): rotates each query once,
 * scores the packed K rows and accumulates the packed V rows in rotated space,
 * and leaves one partial softmax state per (query head, piece) in
 * `workspace`, where the pieces are equal shares of all sequences' 32-token
 * tiles, cut at sequence and KV-head boundaries.  Arguments as for iq_decode_attention; track_argmax != 0 also
 * records the position of the largest score (otherwise the merge reports -1
 * as every argmax).  The workspace content is opaque and valid only for a
 * merge call with the same cfg, batch, num_q_heads and max_kv_len. */
int iq_decode_attention_partial(const iq_config *cfg, const void *q, int32_t q_dtype,
                                int32_t batch, int32_t num_q_heads,
                                const iq_cache *k, const iq_cache *v,
                                const int32_t *kv_len, int64_t max_kv_len,
                                float softmax_scale, int32_t track_argmax,
                                void *workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* Merge phase: combines the partial states a preceding
 * iq_decode_attention_partial left in `workspace`, divides by the softmax
 * denominator and applies R^T once (RotaryQuant §3.4: the inverse rotation
 * acts on the aggregated output, not per token).  Writes out, lse_out and
 * argmax_out as iq_decode_attention does. */
int iq_decode_attention_merge(const iq_config *cfg, int32_t batch, int32_t num_q_heads,
                              int64_t max_kv_len, void *out, int32_t out_dtype,
                              float *lse_out, int32_t *argmax_out,
                              const void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* iq_decode_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and results without the workspace, which
 * comes from a fixed array of 64 MiB inside this library, one per GPU,
 * held from the library's load until the process ends (its device address is
 * looked up on the first call on each device).  The call allocates nothing.
 * Sizes whose iq_decode_workspace_bytes exceeds 64 MiB return
 * IQ_ERR_WORKSPACE (64 sequences x 32 query / 4 KV heads at d = 128 need
 * about 20 MiB); other errors as iq_decode_attention, IQ_ERR_HIP if the
 * array's address cannot be found.  All calls on one GPU share the array:
 * calls that overlap on one GPU (on different streams, or from several
 * threads) race and must not be made; calls on one stream run in order.
 * Nothing in the array needs to start at zero. */
int iq_decode_attention_noalloc(const iq_config *cfg, const void *q, int32_t q_dtype,
                                int32_t batch, int32_t num_q_heads,
                                const iq_cache *k, const iq_cache *v,
                                const int32_t *kv_len, int64_t max_kv_len,
                                float softmax_scale, void *out, int32_t out_dtype,
                                float *lse_out, int32_t *argmax_out, hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char *iq_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* IQ_H */
