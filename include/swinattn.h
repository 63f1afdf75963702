/*
 * swinattn.h -- C ABI of libswinattn: fused shifted-window multi-head
 * attention forward (Swin Transformer) for AMD Instinct MI355X (gfx950).
 *
 * One call computes, for every image of a batch:
 *   cyclic shift by (-shift, -shift) -> cut into window x window tiles ->
 *   per tile and head: softmax(Q K^T / sqrt(head_dim) + bias + mask) V ->
 *   put the tiles back -> shift by (+shift, +shift).
 * Passages that define it:
 *   - NVIDIA talk "Swin Transformer training and inference optimization"
 *     (uticex.com article 1598), section 1: attention restricted to windows,
 *     the window shift, the relative position bias, multi-head attention, and
 *     the block's split into window shift/partition/reverse plus attention.
 *   - same talk, section 2: shift, partition and merge are pure index mapping
 *     (here folded into the kernel's loads and stores); the fused attention
 *     takes the mask and the bias as tensors.
 *   - same talk, section 3: the position-bias lookup is moved out of the
 *     forward to a one-time step (here it is a closed form of the token
 *     coordinates, resolved when the kernel is compiled;
 *     swin_wattn_precompute materialises the index and mask tensors); batch
 *     GEMM, softmax and batch GEMM run as one kernel whose loads and stores
 *     absorb the transposes.
 *   - Baidu AIAK-Training talk (jxzklqfsx.com article 743345), section 2,
 *     WindowAttention case: the whole module as one kernel, tiles staged
 *     through the memory hierarchy, two matrix products and a softmax.
 *
 * Conventions shared by every call:
 *   - every int return value is a swin_status_t; no call aborts or prints;
 *   - arguments are checked before any device work is queued;
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream);
 *     work is queued on it and the call returns without waiting;
 *   - device pointers are owned by the caller unless stated otherwise;
 *   - the calls act on the HIP device that is current on the calling thread.
 *
 * Mask semantics: after the shift, the last `window` rows (columns) of the
 * shifted image hold two strips that were not adjacent in the image; the
 * shifted frame is split into bands [0,H-window), [H-window,H-shift),
 * [H-shift,H) per axis, and a query and a key in different band pairs get
 * -100 added to their score (natural-log units).  With shift == 0 there is
 * no mask.  Relative position index of query (yi,xi) and key (yj,xj) inside a
 * window: (yi-yj+window-1)*(2*window-1) + (xi-xj+window-1).
 */
#ifndef SWINATTN_H
#define SWINATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SWIN_OK = 0,
  SWIN_ERR_INVALID_ARG = -1,  /* null or misaligned pointer, bad size, shift, divisibility */
  SWIN_ERR_UNSUPPORTED = -2,  /* valid but not built: head_dim != 32, window > 12, too many heads (fp32) */
  SWIN_ERR_NOT_PREPARED = -3, /* copy calls: no swin_wattn_precompute for the key */
  SWIN_ERR_HIP = -4           /* the HIP runtime reported an error (allocation, launch) */
} swin_status_t;

/* Materialises, once per (device, H, W, window, shift), in library-owned
 * device memory: the relative position index [N][N] int32 (N = window^2),
 * the shift mask [nW][N][N] float32 (0 or -100, nW = (H/window)*(W/window))
 * and the per-window region labels [nW][N] uint8, for callers that keep
 * these tensors (a Swin block's index and mask buffers) and for
 * verification through the copy calls.  The forward calls do not need it:
 * they evaluate the index and the mask from token coordinates.
 * May allocate device memory (hipMalloc); the fill is queued on `stream`.
 * Calling it again for a prepared key is a no-op returning SWIN_OK.
 * Requires H, W > 0, 1 <= window <= 12, H % window == 0, W % window == 0,
 * 0 <= shift < window. */
int swin_wattn_precompute(int H, int W, int window, int shift, void* stream);

/* Hot path, bfloat16.
 *   qkv            [B][H][W][3][heads][head_dim] bf16, contiguous, image
 *                  (un-shifted) order; index 0 = query, 1 = key, 2 = value.
 *                  Device pointer, 16-byte aligned.
 *   rel_bias_table [(2*window-1)^2][heads] float32, contiguous; device
 *                  pointer, 4-byte aligned.
 *   out            [B][H][W][heads*head_dim] bf16, contiguous, image order;
 *                  device pointer, 16-byte aligned; must not overlap qkv.
 * Scores and softmax in float32, products on bf16 inputs with float32
 * accumulation, attention weights rounded to bf16 before the value product,
 * output rounded to nearest-even bf16.  B == 0 queues nothing and returns
 * SWIN_OK.  head_dim must be 32; any number of heads.  No setup call
 * needed, no allocation, no host synchronisation; safe to call concurrently
 * from several threads. */
int swin_wattn_fwd(const void* qkv, const float* rel_bias_table, void* out, int B, int H, int W,
                   int heads, int head_dim, int window, int shift, void* stream);

/* Same operation with float32 qkv and out (products and accumulation in
 * float32).  Same layouts, alignment and error behaviour, except that the
 * bias tables of all heads, heads * (2*window-1)^2 * 4 bytes, must fit in
 * 160 KiB (they are staged in LDS together; else SWIN_ERR_UNSUPPORTED). */
int swin_wattn_fwd_f32(const float* qkv, const float* rel_bias_table, float* out, int B, int H,
                       int W, int heads, int head_dim, int window, int shift, void* stream);

/* INT8 variant of swin_wattn_fwd (NVIDIA talk, section 3, INT8
 * quantization: a tensor quantized to INT8 carries a scale, products of
 * INT8 values are summed as integers and the sums are dequantized; the
 * other operations stay in floating point, with INT8 input and output).
 *   qkv       [B][H][W][3][heads][head_dim] int8 codes, contiguous, image
 *             order; 16-byte aligned device pointer.  Code c of part p
 *             (0 = query, 1 = key, 2 = value) stands for c * scale_p
 *             (symmetric per-tensor quantization; every code -128..127 is
 *             accepted).
 *   scale_q, scale_k, scale_v   the three scales, host values.  scale_v must
 *             lie in (0, 2^100] and scale_q * scale_k / sqrt(head_dim) in
 *             [2^-100, 2^100], else SWIN_ERR_INVALID_ARG (NaN included).
 *   out_scale 0: out is bf16, as swin_wattn_fwd.  > 0: out is int8 codes
 *             [B][H][W][heads*head_dim], code = clamp(rne(o / out_scale),
 *             -127, 127) (rne = round half to even) of the float32 output
 *             o, for an INT8 output projection to read; scale_v / out_scale
 *             must lie in [2^-100, 2^100].  Negative or NaN:
 *             SWIN_ERR_INVALID_ARG.
 *   rel_bias_table, out   as swin_wattn_fwd (out must not overlap qkv).
 * The scores are the exact integer sums of code products (float32 holds
 * them exactly) times scale_q * scale_k / sqrt(head_dim), plus bias and
 * mask; softmax and value product as in swin_wattn_fwd, with the value
 * codes taken exactly as bf16 and scale_v (scale_v / out_scale) applied
 * with the normaliser.  Shapes, errors and guarantees otherwise as
 * swin_wattn_fwd. */
int swin_wattn_fwd_i8(const void* qkv, float scale_q, float scale_k, float scale_v,
                      float out_scale, const float* rel_bias_table, void* out, int B, int H,
                      int W, int heads, int head_dim, int window, int shift, void* stream);

/* Backward of swin_wattn_fwd, for training (the NVIDIA talk, section 2,
 * fuses the window attention's backward too).  Given dout = dL/d(out), with
 * S = Q K^T / sqrt(d) + bias + mask, P = softmax(S) per window and head:
 *   dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,  dS = P o (dP - D),
 *   dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d),
 *   d(table)[rel(i,j)][h] = sum over every window and image of dS_ij,
 * where dO is dout gathered through the same shift and partition, and
 * dQ, dK, dV go back through the reverse maps.  P is recomputed (exact
 * float32 softmax) from qkv and the table; nothing of the forward is read.
 *   qkv, rel_bias_table  as swin_wattn_fwd
 *   dout    [B][H][W][heads*head_dim] bf16, image order, 16-byte aligned
 *   dqkv    [B][H][W][3][heads][head_dim] bf16, written (q, k, v gradients);
 *           16-byte aligned; must not overlap qkv, dout or dtable
 *   dtable  [(2*window-1)^2][heads] float32, written (zeroed on the stream,
 *           then accumulated with atomics: the order of the sum varies)
 * head_dim must be 32 and window <= 12 (else SWIN_ERR_UNSUPPORTED); any
 * number of heads.  B == 0 zeroes dtable.  No allocation, no host
 * synchronisation. */
int swin_wattn_bwd(const void* qkv, const float* rel_bias_table, const void* dout, void* dqkv,
                   float* dtable, int B, int H, int W, int heads, int head_dim, int window,
                   int shift, void* stream);

/* Linear layer on either side of the attention, bf16 with fp32 accumulation:
 *   y[t][j] = sum_c x[t][c] * W[j][c] + bias[j]  (+ residual[t][j])
 *  - QKV GEMM + bias (K = C, N = 3C): the output token row is [3][heads][d],
 *    the qkv row swin_wattn_fwd reads (NVIDIA talk, section 3: the QKV GEMM
 *    fused with its bias, the weight put in a kernel-friendly format once).
 *  - Output projection + bias + residual (K = N = C): the same talk,
 *    section 3, adds a bias and then the residual in one kernel.
 *
 * swin_linear_pack_weight: W [N][K] bf16 (out_features x in_features, the
 * nn.Linear layout), device pointer, 16-byte aligned -> packed, N*K bf16 in
 * the operand order swin_linear_fwd reads; caller-owned device memory that
 * must not overlap W.  Once per weight; queued on `stream`.
 *
 * swin_linear_fwd:
 *   x         [T][K] bf16, contiguous, 16-byte aligned (device)
 *   packed    the output of swin_linear_pack_weight for this W
 *   bias      [N] float32, 16-byte aligned, or NULL (no bias)
 *   residual  [T][N] bf16, 16-byte aligned, or NULL (no residual); may be y
 *             itself (in-place add), otherwise must not overlap y
 *   y         [T][N] bf16, 16-byte aligned; must not overlap x, packed, bias
 * Products of bf16 inputs accumulate in float32; bias and residual are added
 * in float32; y is rounded to nearest-even bf16.  K and N must be positive
 * multiples of 32 (else SWIN_ERR_INVALID_ARG); K <= 384 (else
 * SWIN_ERR_UNSUPPORTED).  T == 0 queues nothing.  No allocation, no host
 * synchronisation. */
int swin_linear_pack_weight(const void* weight, void* packed, int N, int K, void* stream);
int swin_linear_fwd(const void* x, const void* packed_weight, const float* bias,
                    const void* residual, void* y, long long T, int K, int N, void* stream);

/* INT8 linear layer (NVIDIA talk, section 3, INT8 quantization: input and
 * weight quantized to INT8, products accumulated in INT32 and the sums
 * dequantized; bias, residual and layer norm stay in floating point; the
 * INT8-output form, which the talk takes for Swin, quantizes the result
 * again so that the next kernel reads INT8):
 *   acc[t][j] = sum_c xq[t][c] * wq[j][c]                    (exact, int32)
 *   bf16 output: y[t][j] = acc * (x_scale * w_scale[j]) + bias[j] (+ residual)
 *                in float32, rounded to nearest-even bf16
 *   int8 output: y[t][j] = clamp(rne(fma(acc, a_j, b_j)), -127, 127), with
 *                a_j = x_scale * w_scale[j] / out_scale[j] and
 *                b_j = bias[j] / out_scale[j] (float32 operations, each
 *                rounded to nearest; rne = round half to even)
 *
 * swin_linear_i8_pack_weight: W [N][K] int8 codes (16-byte aligned device
 * pointer) -> packed, N * ceil(K/64) * 64 bytes (zero where K is not a
 * multiple of 64), caller-owned, 16-byte aligned, not overlapping W.  Once
 * per weight; queued on `stream`.
 *
 * swin_linear_i8_fwd:
 *   x          [T][K] int8 codes, contiguous, 16-byte aligned (device)
 *   x_scale    scale of the x codes (host value, finite and > 0)
 *   packed     the output of swin_linear_i8_pack_weight for this W
 *   w_scale    [N] float32 scales of the rows of W (per output channel);
 *              16-byte aligned device pointer, not NULL
 *   bias       [N] float32, 16-byte aligned, or NULL (no bias)
 *   residual   [T][N] bf16, 16-byte aligned, or NULL; bf16 output only; may
 *              be y itself (in-place add), otherwise must not overlap y
 *   out_scale  [N] float32 scales of the output columns (16-byte aligned;
 *              finite and nonzero), or NULL for bf16 output; for the QKV
 *              projection, columns [0,C) [C,2C) [2C,3C) carry the query,
 *              key and value scales of swin_wattn_fwd_i8
 *   y          [T][N] bf16, or int8 with out_scale; 16-byte aligned; must not
 *              overlap x, packed, bias, w_scale or out_scale
 * K and N must be positive multiples of 32 (else SWIN_ERR_INVALID_ARG);
 * K <= 768 (else SWIN_ERR_UNSUPPORTED).  A residual with int8 output is
 * SWIN_ERR_INVALID_ARG.  T == 0 queues nothing.  No allocation, no host
 * synchronisation. */
int swin_linear_i8_pack_weight(const void* weight, void* packed, int N, int K, void* stream);
int swin_linear_i8_fwd(const void* x, float x_scale, const void* packed_weight,
                       const float* w_scale, const float* bias, const void* residual,
                       const float* out_scale, void* y, long long T, int K, int N, void* stream);

/* Layer normalisation fused into the QKV projection:
 *   xn[t][c] = (x[t][c] - mean_t) / sqrt(var_t + eps) * gamma[c] + beta[c]
 *   y = xn W^T + bias
 * (mean and biased variance of each token row over its K channels, in
 * float32).  The NVIDIA talk, section 3, fuses the layer norm with the
 * window shift and partition that follow it, and prepares the QKV weight
 * and bias in advance; here the shift and partition are part of
 * swin_wattn_fwd's loads, and the layer norm folds into the weight:
 *   y_j = (sum_c x_c W'_jc - mean_t s_j) / sigma_t + b'_j,
 *   W' = gamma o W (bf16), s_j = sum_c W'_jc, b'_j = bias_j + sum_c beta_c W_jc,
 * so one pass reads raw x and writes the qkv the attention reads.
 *
 * swin_ln_linear_pack_weight: W [N][K] bf16 (16-byte aligned), gamma and
 * beta [K] float32, bias [N] float32 or NULL -> packed (N*K bf16, caller-
 * owned, 16-byte aligned, must not overlap W) and consts [2][N] float32
 * (s, then b'; caller-owned, 16-byte aligned, overlapping no input).  Once
 * per weight; queued on `stream`.
 * swin_ln_linear_fwd: x [T][K] bf16 raw (not normalised); packed and consts
 * from swin_ln_linear_pack_weight; eps >= 0.  Other arguments, layouts and
 * errors as swin_linear_fwd (no residual). */
int swin_ln_linear_pack_weight(const void* weight, const float* gamma, const float* beta,
                               const float* bias, void* packed, float* consts, int N, int K,
                               void* stream);
int swin_ln_linear_fwd(const void* x, const void* packed_weight, const float* consts, float eps,
                       void* y, long long T, int K, int N, void* stream);

/* Layer norm + QKV projection + shifted-window attention in one pass: the
 * attention half of a Swin block before its output projection,
 *   out = swin_wattn_fwd( layer_norm(x) W_qkv^T + b_qkv )
 * with q, k and v formed per window on the chip instead of being written to
 * memory and read back.  The NVIDIA talk, section 3, fuses the layer norm
 * with the window shift and partition, fuses the QKV GEMM with its bias and
 * prepares its weight to suit the fused attention.
 *   x        [B][H][W][C] bf16 raw token rows (C = heads * head_dim), image
 *            order, 16-byte aligned
 *   packed_qkv, consts  from swin_ln_linear_pack_weight of the QKV weight
 *            [3C][C] (rows ordered [3][heads][head_dim]), gamma, beta and
 *            bias, with N = 3C and K = C
 *   eps      layer-norm epsilon, >= 0
 *   rel_bias_table, out, B, H, W, heads, head_dim, window, shift: as
 *            swin_wattn_fwd, with out [B][H][W][C]; out must overlap none of
 *            the inputs
 * Arithmetic: the layer norm and the projection as swin_ln_linear_fwd, q, k
 * and v rounded to bf16, then the attention as swin_wattn_fwd.  head_dim
 * must be 32, 5 <= window <= 8 and C <= 192 (else SWIN_ERR_UNSUPPORTED).
 * B == 0 queues nothing.  No allocation, no host synchronisation. */
int swin_ln_qkv_wattn_fwd(const void* x, const void* packed_qkv, const float* consts, float eps,
                          const float* rel_bias_table, void* out, int B, int H, int W, int heads,
                          int head_dim, int window, int shift, void* stream);

/* Copies of the precomputed tensors into caller-owned device memory, queued
 * on `stream` (for verification).  SWIN_ERR_NOT_PREPARED without a prior
 * swin_wattn_precompute for the key.  `stream` may differ from the
 * precompute's stream: the copy is queued behind the precompute's fill (an
 * event recorded at setup), never ahead of it.
 *   index  [N][N] int32;  mask [nW][N][N] float32;
 *   region [nW][N] uint8 region labels (label = 3*band_y + band_x).
 * The index depends on the window only, but the cache is keyed by
 * (device, H, W, window, shift) like the mask and the labels, so the index
 * copy names the same key; each copy takes the caller's stream so that it
 * is ordered with the caller's other work. */
int swin_wattn_copy_index(int H, int W, int window, int shift, int32_t* dst, void* stream);
int swin_wattn_copy_mask(int H, int W, int window, int shift, float* dst, void* stream);
int swin_wattn_copy_region(int H, int W, int window, int shift, uint8_t* dst, void* stream);

/* Frees every precomputed buffer on every device (synchronises each device
 * first).  Afterwards the copy calls return SWIN_ERR_NOT_PREPARED until the
 * next precompute; the forward calls are unaffected.  Must not run
 * concurrently with other calls.  Returns SWIN_OK, or SWIN_ERR_HIP when a
 * device could not be synchronised or a buffer not freed (the cache is
 * emptied either way), so that a failure is not silent. */
int swin_wattn_release(void);

/* Static, human-readable name of a status code. */
const char* swin_wattn_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* SWINATTN_H */
