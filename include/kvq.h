/*
 * kvq.h -- C ABI of libkvq.so: quantized-decode kernels for AMD MI355X
 * (gfx950, CDNA4), written in HIP.
 *
 * Conventions for every call below
 *   - Every pointer is a DEVICE pointer owned by the caller; the library never
 *     allocates, frees or retains memory.  Base pointers must be 16-byte
 *     aligned (checked).  bf16 values travel as uint16_t bit patterns and
 *     E4M3 (OCP E4M3FN) codes as uint8_t.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     default stream).  No call synchronizes.
 *   - Return value: KVQ_OK, or a kvq_status_t error.  Arguments are validated
 *     on the host before any HIP call; on error nothing is launched and
 *     kvq_last_error() describes the first violated condition.  No exception
 *     crosses this boundary.
 *   - Outputs are written in full (no read-modify-write of caller memory).
 *     Workspaces are scratch memory: the calls that use one leave its
 *     counter area (below) at zero and put partial results behind it.
 *
 * Sources (web pages; each declaration names the section it implements):
 *   [KVQ]  boostr, src/ops/wgpu/shaders/cache/kv_cache_quant.wgsl
 *   [W8A8] metrale_model_layers, layers/ops/w8a8_decode.rs
 *   [AWQ]  boostr, src/quant/wgpu/shaders/fused_int4_qkv.rs
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KVQ_OK = 0,
    KVQ_E_INVALID = 1,      /* an argument violates the documented contract   */
    KVQ_E_UNSUPPORTED = 2,  /* no gfx950 code object for the current device   */
    KVQ_E_LAUNCH = 3        /* the HIP runtime rejected a kernel launch        */
} kvq_status_t;

/* Message for the last failing call on this thread ("" if none).  The
 * pointer stays valid until the next failing call on the same thread. */
const char *kvq_last_error(void);

/* Library ABI version (major * 100 + minor). */
int kvq_abi_version(void);

/* Workspaces (w8a8_gemv, w8a8_proj, int4_awq_qkv_gemm): the first
 * KVQ_WORKSPACE_COUNTER_BYTES bytes hold the counters through which the
 * workgroups of one output tile find the last of them; every call leaves
 * them at zero, and partial sums (and the INT4 call's scaled fp16 activations)
 * only ever go behind them, also when a call uses no counters.  One zero-filled
 * buffer can therefore serve calls of all three kinds, in any order, as long
 * as they are ordered on one stream. */
#define KVQ_WORKSPACE_COUNTER_BYTES 4096u

/* ======================================================================== */
/* KV cache, symmetric per-token INT8                                       */
/* [KVQ] sections "INT8 Per-Token Quantization" / "Dequantization".  The
 * page's "FP8 Per-Token" sections compute the same integer code (absmax/127,
 * not an E4M3 encoding); kvq_quant_fp8_token / kvq_dequant_fp8_token are
 * aliases of these two calls.
 *
 *   scale[t] = max(max_d |x[t][d]| / 127, 1e-8)        (fp32, IEEE division)
 *   codes[t][d] = clamp(rint_half_even(x[t][d] / scale[t]), -128, 127)
 *   y[t][d] = (float)codes[t][d] * scale[t]
 *
 * x / scale is the correctly rounded fp32 quotient: the kernels form it from
 * the scale's reciprocal plus one fused correction, which gives the IEEE
 * quotient's bits wherever a code depends on it (the same holds for every
 * quantizer below).
 *
 * x, y: fp32 [num_tokens][head_dim] row-major; codes: int8, same shape;
 * scales: fp32 [num_tokens].  num_tokens >= 1, head_dim >= 1.  Inputs must be
 * finite (NaN/Inf are outside the contract). */
int kvq_quant_int8_token(const float *x, int8_t *codes, float *scales,
                         uint32_t num_tokens, uint32_t head_dim, void *stream);
int kvq_dequant_int8_token(const int8_t *codes, const float *scales, float *y,
                           uint32_t num_tokens, uint32_t head_dim, void *stream);
int kvq_quant_fp8_token(const float *x, int8_t *codes, float *scales,
                        uint32_t num_tokens, uint32_t head_dim, void *stream);
int kvq_dequant_fp8_token(const int8_t *codes, const float *scales, float *y,
                          uint32_t num_tokens, uint32_t head_dim, void *stream);

/* KV codecs with 16-bit values (the page's kernels carry an _f32 suffix;
 * these are the same codecs for fp16/bf16 caches).  dtype: KVQ_DT_F32,
 * KVQ_DT_F16 or KVQ_DT_BF16.  A 16-bit input is widened exactly to fp32 and
 * coded by the fp32 rule above (codes and scales equal those of the fp32
 * call on the widened values); a 16-bit output is the fp32 dequantized value
 * rounded to nearest even.  x / y hold num_tokens*head_dim values of that
 * type; every other argument, layout and rule is that of the fp32 call.
 * KVQ_DT_F32 gives exactly the fp32 calls. */
typedef enum { KVQ_DT_F32 = 0, KVQ_DT_F16 = 1, KVQ_DT_BF16 = 2 } kvq_dtype_t;
int kvq_quant_int8_token_dt(const void *x, int x_dtype, int8_t *codes,
                            float *scales, uint32_t num_tokens,
                            uint32_t head_dim, void *stream);
int kvq_dequant_int8_token_dt(const int8_t *codes, const float *scales,
                              void *y, int y_dtype, uint32_t num_tokens,
                              uint32_t head_dim, void *stream);
int kvq_quant_int4_group_dt(const void *x, int x_dtype, uint8_t *packed,
                            float *scales, float *zeros, uint32_t num_tokens,
                            uint32_t head_dim, uint32_t group_size,
                            void *stream);
int kvq_dequant_int4_group_dt(const uint8_t *packed, const float *scales,
                              const float *zeros, void *y, int y_dtype,
                              uint32_t num_tokens, uint32_t head_dim,
                              uint32_t group_size, void *stream);

/* KV cache INT8, one scale for the whole tensor.
 * [KVQ] the parameter block's declared mode 0 ("per_tensor"); the page shows
 * only per-token kernels, so this is the per-token rule above with the
 * absmax taken over all num_tokens*head_dim values:
 *
 *   scale = max(max |x| / 127, 1e-8);   codes = clamp(rint(x / scale), -128, 127)
 *   y = (float)codes * scale
 *
 * x, y: fp32 [num_tokens*head_dim]; codes: int8, same size; scale: fp32 [1].
 * The quantizer runs two launches (partial absmax per workgroup into the
 * workspace, then encode) and needs a device workspace of at least
 * KVQ_INT8_TENSOR_WORKSPACE_BYTES (16-byte aligned); it writes only behind
 * the counter area, so the workspace of the other calls can be shared. */
#define KVQ_INT8_TENSOR_WORKSPACE_BYTES (KVQ_WORKSPACE_COUNTER_BYTES + 2048u)
int kvq_quant_int8_tensor(const float *x, int8_t *codes, float *scale,
                          uint32_t num_tokens, uint32_t head_dim,
                          void *workspace, size_t workspace_bytes, void *stream);
int kvq_dequant_int8_tensor(const int8_t *codes, const float *scale, float *y,
                            uint32_t num_tokens, uint32_t head_dim, void *stream);

/* ======================================================================== */
/* KV cache, asymmetric per-group INT4                                      */
/* [KVQ] sections "INT4 Per-Group Quantization" / "Dequantization".  Groups
 * are group_size consecutive elements of the flattened [num_tokens*head_dim]
 * array (a group may span tokens when head_dim % group_size != 0).
 *
 *   mn, mx = min, max of the group;   scale = (mx - mn) / 15  (stored as is)
 *   sf = max(scale, 1e-8);   zero = -mn / sf
 *   code = clamp(rint_half_even((x - mn) / sf), 0, 15)
 *   packed[e / 2] = code[e even] | code[e odd] << 4      (low nibble first)
 *   y = (float)code * scale - zero * scale     (two roundings, then subtract)
 *
 * x, y: fp32 [num_tokens*head_dim]; packed: uint8 [num_tokens*head_dim/2];
 * scales, zeros: fp32 [G], G = num_tokens*head_dim/group_size.  The page
 * stores the zeros after the scales in one buffer; here they are a separate
 * array.  group_size >= 2, even, and divides num_tokens*head_dim.  A constant
 * group stores scale 0 and dequantizes to +0 (the page's behaviour). */
int kvq_quant_int4_group(const float *x, uint8_t *packed, float *scales,
                         float *zeros, uint32_t num_tokens, uint32_t head_dim,
                         uint32_t group_size, void *stream);
int kvq_dequant_int4_group(const uint8_t *packed, const float *scales,
                           const float *zeros, float *y, uint32_t num_tokens,
                           uint32_t head_dim, uint32_t group_size, void *stream);

/* ======================================================================== */
/* W8A8 FP8 decode (OCP E4M3FN activations and weights)                     */
/* [W8A8] items W8a8Scale, W8a8Weight, W8a8Scratch, w8a8_act_quant,
 * w8a8_act_quant_silu, w8a8_gemv, w8a8_proj. */

typedef enum {
    W8A8_ROWSCALE = 0,  /* W8a8Scale::PerRow: one weight scale per output row,
                           one activation scale per token row               */
    W8A8_BLK128 = 1     /* W8a8Scale::Block128: one weight scale per 128x128
                           block, one activation scale per 128 columns       */
} w8a8_scale_t;

#define W8A8_MAX_ROWS 256u   /* largest token-row count per call            */
#define W8A8_K_UNIT 128u     /* K must be a positive multiple of this       */

/* Activation quantization (w8a8_act_quant; with silu, w8a8_act_quant_silu).
 *   v = f32(x)                       silu == 0 (up must be NULL)
 *   v = silu(f32(x))                 silu != 0, up == NULL
 *   v = silu(f32(x)) * f32(up)       silu != 0, up != NULL (gate = x)
 * silu(v) = v / (1 + e^-v) with a fixed fp32 exponential (Cody-Waite
 * reduction + degree-7 Taylor polynomial), so results are reproducible bits.
 * Per row (ROWSCALE) or per 128-column group (BLK128):
 *   s = max(amax / 448, 1e-8);   q = E4M3_rne_satfinite(v / s)
 * x, up: bf16 [rows][ldx]; q: uint8 [rows][k]; a_scales: fp32 [rows]
 * (ROWSCALE) or [rows][k/128] (BLK128).  1 <= rows <= 256, k % 128 == 0,
 * ldx >= k, ldx % 8 == 0.  Inputs must be finite. */
int w8a8_act_quant(w8a8_scale_t kind, int silu, const uint16_t *x,
                   const uint16_t *up, uint32_t ldx, uint32_t rows, uint32_t k,
                   uint8_t *q, float *a_scales, void *stream);

/* Sizes of the two activation buffers w8a8_act_quant writes and w8a8_gemv
 * reads (W8a8Scratch): q_bytes = rows*k, scale_bytes = rows*max(k/128,1)*4
 * for BLK128 and rows*4 for ROWSCALE. */
int w8a8_scratch_bytes(w8a8_scale_t kind, uint32_t rows, uint32_t k,
                       size_t *q_bytes, size_t *scale_bytes);

/* One weight segment (a Fp8Weight): E4M3 codes [n][k] row-major, and scales
 * fp32 [n] (ROWSCALE) or [ceil(n/128)][k/128] (BLK128). */
typedef struct {
    const uint8_t *w;
    const float *scale;
    uint32_t n;
} w8a8_segment_t;

/* GEMV/GEMM over 1..3 concatenated weight segments (w8a8_gemv):
 *   out[m][j] = bf16_rne( sum_k dec(q[m][k]) * sa * dec(W[j][k]) * sw )
 * where W is the concatenation of the segments along n (output column j
 * belongs to segment 0 below n0, segment 1 below n0+n1, else segment 2) and
 * the scales are the row scales (ROWSCALE: sa[m] * sw[j]) or the block
 * scales applied per 128-wide K block (BLK128: sa[m][kb] * sw[j/128][kb]).
 * Accumulation is fp32.  Every segment but the last must have n % 16 == 0
 * (ROWSCALE) or n % 128 == 0 (BLK128); all share k.
 * q, a_scales: as written by w8a8_act_quant; out: bf16 [rows][ldc], ldc >=
 * sum n; columns >= sum n of each row are not touched.
 * workspace: NULL, or device memory of at least w8a8_gemv_workspace_bytes(),
 * zero-filled before its first use.  Split-K partial sums go behind its
 * counter area (KVQ_WORKSPACE_COUNTER_BYTES), which the call leaves as it
 * found it, so calls ordered on one stream can reuse the buffer.
 * Without it the call still works, with less parallelism for large rows.
 * Concurrent calls must not share a workspace. */
int w8a8_gemv(w8a8_scale_t kind, const uint8_t *q, const float *a_scales,
              uint32_t rows, uint32_t k, const w8a8_segment_t *segs,
              uint32_t nseg, uint16_t *out, uint32_t ldc, void *workspace,
              size_t workspace_bytes, void *stream);

/* Workspace size that lets w8a8_gemv use its full parallelism (may be 0). */
int w8a8_gemv_workspace_bytes(w8a8_scale_t kind, uint32_t rows, uint32_t k,
                              uint32_t n_total, size_t *bytes);

/* w8a8_proj: act_quant into (q, a_scales) then gemv, on one stream.  With
 * rows <= 8 (and, for ROWSCALE, k <= 4096) it is ONE launch: the GEMV kernel
 * quantizes the activations itself, writes the same codes and scales to
 * (q, a_scales) and returns the same output bits as the two-step form;
 * otherwise two launches.  The workspace is used only by the two-launch
 * form (see w8a8_gemv). */
int w8a8_proj(w8a8_scale_t kind, int silu, const uint16_t *x,
              const uint16_t *up, uint32_t ldx, uint32_t rows, uint32_t k,
              const w8a8_segment_t *segs, uint32_t nseg, uint16_t *out,
              uint32_t ldc, uint8_t *q, float *a_scales, void *workspace,
              size_t workspace_bytes, void *stream);

/* Offline weight preparation with the activation rule: w fp32 [n][k] ->
 * codes [n][k] and scales [n] (ROWSCALE) or [ceil(n/128)][k/128] (BLK128),
 * amax taken per weight row or per 128x128 block.  k % 128 == 0.  (The page
 * receives weights already quantized; this supplies them.) */
int w8a8_weight_quant(w8a8_scale_t kind, const float *w, uint32_t n,
                      uint32_t k, uint8_t *q, float *scales, void *stream);

/* Plain conversion fp32 -> E4M3FN (round to nearest even, saturating to
 * +-448, sign kept), the encoder every W8A8 quantizer above uses. */
int kvq_f32_to_e4m3(const float *x, uint8_t *q, uint64_t n, void *stream);

/* ======================================================================== */
/* INT4 AWQ weight-only, fused Q/K/V                                        */
/* [AWQ] QKV_AWQ_SHIFTS, unpack_awq_qkv, fused_int4_qkv_q / _k / _v.
 *
 *   code(k, j) = (qweight[k][j/8] >> SHIFTS[j % 8]) & 0xF,
 *                SHIFTS = {0, 16, 4, 20, 8, 24, 12, 28}
 *   out[m][j]  = sum_k x[m][k] * (code(k, j) - zeros[k/gs][j]) * scales[k/gs][j]
 *
 * One projection: qweight uint32 [k][n/8]; scales, zeros fp32 [k/gs][n];
 * out fp32 [m][n].  n % 8 == 0. */
typedef struct {
    const uint32_t *qweight;
    const float *scales;
    const float *zeros;
    float *out;
    uint32_t n;
} int4_awq_proj_t;

/* Q, K and V in one launch (the page dispatches three kernels).  k_proj and
 * v_proj are both NULL (a single projection) or both set with equal n.
 * x: fp32 [m][k], m >= 1, k % group_size == 0.  group_size is 32, 64, 128
 * or 256.
 * m < 16: every product and sum is fp32, as on the page (a weight-streaming
 * GEMV on the vector ALUs: codes unpacked to exact floats, x unrounded, s
 * and z applied once per group as s * (sum x q - z * sum x)); 9..15 rows run
 * as two launches of at most 8.
 * m >= 16: the matrix cores take fp16 activations and the exact codes,
 * accumulating in fp32.  fp32 (and bf16) rows are first scaled by the power
 * of two 2^E that puts the row's absmax in [2^14, 2^15) and rounded to fp16
 * (nearest even); each output row is multiplied by 2^-E (exact).  Every term
 * thus keeps 2^-11 relative precision at any fp32 activation scale (rows of
 * 1e-6 or 1e5 alike; zero rows and rows holding inf or NaN are left
 * unscaled).  When a wave's K range fits its LDS ring the wave takes the
 * absmax over its own K range and scales in registers; otherwise one extra
 * launch writes the scaled fp16 rows and their 2^-E into the workspace.
 * Without a workspace, such shapes round x to fp16 unscaled inside the
 * product kernel: then |x| must stay below 65504 (a larger value becomes
 * inf) and terms below 2^-14 lose relative precision (fp16 subnormals).
 * workspace: NULL, or at least int4_awq_workspace_bytes(), zero-filled before
 * its first use; the call leaves its counter area at zero and writes partial
 * tiles behind it, and for m >= 16 the scaled fp16 activations and their
 * row scales behind those.  Without it, one workgroup per tile (less
 * parallelism) and the unscaled rounding above.  The workspace arguments
 * extend the page's call (which has none): split-K partial sums and the
 * scaled copy need device scratch the library does not allocate.
 * Concurrent calls must not share a workspace. */
int int4_awq_qkv_gemm(const float *x, uint32_t m, uint32_t k,
                      uint32_t group_size, const int4_awq_proj_t *q_proj,
                      const int4_awq_proj_t *k_proj,
                      const int4_awq_proj_t *v_proj, void *workspace,
                      size_t workspace_bytes, void *stream);

int int4_awq_workspace_bytes(uint32_t m, uint32_t k, uint32_t group_size,
                             uint32_t n_total, size_t *bytes);

/* The same call with 16-bit activations (kvq_dtype_t: KVQ_DT_F32, KVQ_DT_F16
 * or KVQ_DT_BF16; x holds m*k values of that type).  m < 16: the values are
 * widened exactly to fp32 (the same results as the fp32 call on the widened
 * values).  m >= 16: fp16 values go to the matrix cores unchanged (exact);
 * bf16 values are widened exactly and then scaled and rounded like fp32
 * input.  Outputs stay fp32.  KVQ_DT_F32 is exactly int4_awq_qkv_gemm. */
int int4_awq_qkv_gemm_dt(const void *x, int x_dtype, uint32_t m, uint32_t k,
                         uint32_t group_size, const int4_awq_proj_t *q_proj,
                         const int4_awq_proj_t *k_proj,
                         const int4_awq_proj_t *v_proj, void *workspace,
                         size_t workspace_bytes, void *stream);

/* int4_awq_qkv_gemm for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, hosts that forbid hipMalloc.  Same
 * arguments, rules and results as int4_awq_qkv_gemm with a sufficient
 * workspace (fp32 activations), but the workspace is a device array inside
 * the library: KVQ_INT4_NOALLOC_SCRATCH_BYTES on each GPU, held while the
 * library's code is loaded there (until the process ends).  The call
 * allocates and frees nothing.  Shapes whose plan needs more scratch than
 * that return KVQ_E_INVALID (use int4_awq_qkv_gemm with a workspace).
 * Every call on a GPU uses that GPU's one array: calls that overlap on one
 * GPU (different streams, or host threads) race and must be ordered by the
 * caller. */
#define KVQ_INT4_NOALLOC_SCRATCH_BYTES (4u << 20)
int int4_awq_qkv_gemm_noalloc(const float *x, uint32_t m, uint32_t k,
                              uint32_t group_size,
                              const int4_awq_proj_t *q_proj,
                              const int4_awq_proj_t *k_proj,
                              const int4_awq_proj_t *v_proj, void *stream);

/* ======================================================================== */
/* Decode attention over the INT8 per-token cache                           */
/* The consumer of the [KVQ] "INT8 Per-Token Quantization" cache.  The pages
 * define the cache and its dequantization (value = code * scale) but no
 * attention; this is textbook scaled-dot-product attention for one new token
 * per query head, query head h reading KV head h / (num_q_heads /
 * num_kv_heads):
 *   s_t = softmax_scale * (q_h . k_t),  p = softmax(s),  out_h = sum_t p_t v_t
 * with k_t, v_t the dequantized cache rows.  Arithmetic is fp32: the scales
 * multiply the integer dot products and the softmax weights; within
 * 1e-3 * sum_t p_t |v_t| of the exact result for moderate scores.
 *   q:        fp32 [num_q_heads][head_dim]
 *   k_codes, v_codes: int8 [num_tokens][num_kv_heads][head_dim] (the
 *             per-token quantizer's output for num_tokens*num_kv_heads rows)
 *   k_scales, v_scales: fp32 [num_tokens][num_kv_heads]
 *   out:      fp32 [num_q_heads][head_dim]
 * head_dim is 64, 128 or 256; num_q_heads is 1..8 times num_kv_heads;
 * num_tokens >= 1.
 * All pointers are device memory, 16-byte aligned, owned by the caller.
 * workspace: NULL, or at least kvq_attn_decode_workspace_bytes() (the
 * shared workspace of the calls above: the per-chunk partial results go
 * behind its counter area, which this call does not touch; a second kernel
 * on the stream merges them).  Without it one workgroup walks each KV
 * head's tokens (less parallelism, same definition).
 * Concurrent calls must not share a workspace.  Errors: KVQ_E_INVALID for
 * shapes, null or misaligned pointers, a non-finite softmax_scale. */
int kvq_attn_decode_int8(const float *q, uint32_t num_q_heads,
                         uint32_t num_kv_heads, uint32_t num_tokens,
                         uint32_t head_dim, const int8_t *k_codes,
                         const float *k_scales, const int8_t *v_codes,
                         const float *v_scales, float softmax_scale,
                         float *out, void *workspace, size_t workspace_bytes,
                         void *stream);

int kvq_attn_decode_workspace_bytes(uint32_t num_q_heads, uint32_t num_kv_heads,
                                    uint32_t num_tokens, uint32_t head_dim,
                                    size_t *bytes);

/* The same attention over the [KVQ] "INT4 Per-Group Quantization" cache:
 * each (token, KV head) row of head_dim values holds head_dim / group_size
 * groups (group_size 32, 64 or 128, at most head_dim), dequantized as
 * code * scale - zero *
 * scale.  k_packed, v_packed: uint8 [num_tokens][num_kv_heads][head_dim/2],
 * two codes per byte, even element in the low nibble (the quantizer's output
 * for num_tokens*num_kv_heads rows); scales and zeros: fp32
 * [num_tokens][num_kv_heads][head_dim/group_size].  Per group the scale
 * multiplies sum q*code - zero * sum q, and the softmax weight times the
 * scale multiplies the value codes.  Everything else (layout, workspace,
 * tolerance, errors) as kvq_attn_decode_int8. */
int kvq_attn_decode_int4(const float *q, uint32_t num_q_heads,
                         uint32_t num_kv_heads, uint32_t num_tokens,
                         uint32_t head_dim, uint32_t group_size,
                         const uint8_t *k_packed, const float *k_scales,
                         const float *k_zeros, const uint8_t *v_packed,
                         const float *v_scales, const float *v_zeros,
                         float softmax_scale, float *out, void *workspace,
                         size_t workspace_bytes, void *stream);

/* A batch of sequences of different lengths, one new token each (the same
 * attention per sequence).
 *   q, out:    fp32 [batch][num_q_heads][head_dim]
 *   seq_start: device uint32 [batch + 1]: sequence b's cache rows are tokens
 *              seq_start[b] .. seq_start[b+1]-1 of the cache (packed:
 *              [total_tokens][num_kv_heads][...] as in the calls above).
 *              Non-decreasing, seq_start[batch] <= total_tokens, every
 *              length <= max_seq_tokens (the host's bound, used to plan the
 *              work).  The kernels read it on the device: longer sequences
 *              are cut at max_seq_tokens, rows past total_tokens read as zero
 *              codes and scales (no fault), a sequence with no tokens gets a
 *              zero output.
 * Workspace as above, sized by kvq_attn_decode_varlen_workspace_bytes.
 * Errors: KVQ_E_INVALID for batch == 0, head shapes as above,
 * max_seq_tokens > total_tokens, a null or misaligned seq_start. */
int kvq_attn_decode_int8_varlen(const float *q, uint32_t batch,
                                uint32_t num_q_heads, uint32_t num_kv_heads,
                                uint32_t head_dim, const uint32_t *seq_start,
                                uint32_t total_tokens, uint32_t max_seq_tokens,
                                const int8_t *k_codes, const float *k_scales,
                                const int8_t *v_codes, const float *v_scales,
                                float softmax_scale, float *out,
                                void *workspace, size_t workspace_bytes,
                                void *stream);

int kvq_attn_decode_int4_varlen(const float *q, uint32_t batch,
                                uint32_t num_q_heads, uint32_t num_kv_heads,
                                uint32_t head_dim, uint32_t group_size,
                                const uint32_t *seq_start, uint32_t total_tokens,
                                uint32_t max_seq_tokens, const uint8_t *k_packed,
                                const float *k_scales, const float *k_zeros,
                                const uint8_t *v_packed, const float *v_scales,
                                const float *v_zeros, float softmax_scale,
                                float *out, void *workspace,
                                size_t workspace_bytes, void *stream);

int kvq_attn_decode_varlen_workspace_bytes(uint32_t batch, uint32_t num_q_heads,
                                           uint32_t num_kv_heads,
                                           uint32_t max_seq_tokens,
                                           uint32_t head_dim, size_t *bytes);

/* ======================================================================== */
/* Measurement helper (not part of the method)                              */
/* kvq_stream_read: reads `bytes` (a positive multiple of 16) at `src` (16-
 * byte aligned device memory) with 16-byte loads across the whole GPU and
 * writes almost nothing (sink: one device uint32, written only for an
 * impossible data pattern).  Its rate is the empirical read ceiling the
 * benchmark reports beside each kernel's bandwidth. */
int kvq_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
