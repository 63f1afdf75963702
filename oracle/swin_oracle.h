/*
 * swin_oracle.h -- plain, slow, fp64 CPU oracle for shifted-window
 * multi-head attention (Swin Transformer window attention with cyclic shift).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this library: only the tests, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code, header, table or
 * constant with the HIP implementation.
 *
 * What it computes, and where the pages state it:
 *  - NVIDIA talk "Swin Transformer training and inference optimization"
 *    (uticex.com article 1598), section 1 "Swin Transformer introduction":
 *    attention is taken only among the patches of one window; a window shift
 *    fixes the window-boundary problem; a relative position bias is added
 *    inside attention; query and key through softmax give the attention map
 *    that weights value; several heads form multi-head attention; a block is
 *    window shift/partition/reverse, then attention, then FFN.
 *  - same talk, section 2 "training optimization": the window shift is a roll,
 *    the partition/shift/merge operations are pure index mapping, and the
 *    fused attention receives the mask and the bias as tensors.
 *  - same talk, section 3 "inference optimization": the position-bias lookup
 *    is moved to preprocessing; batch GEMM, softmax, batch GEMM form the
 *    attention.
 *  - Baidu AIAK-Training talk (jxzklqfsx.com article 743345), section 2,
 *    WindowAttention fusion case: two matrix products and a softmax.
 * The formula figure of the WindowAttention case did not survive extraction;
 * the oracle takes softmax(Q K^T / sqrt(d) + bias + mask) V.  Where the
 * pages are silent (shift direction, mask value -100, relative index as
 * query minus key, scale 1/sqrt(d)) it takes the plainest reading that the
 * rest of the pages supports, stated at each function below.
 *
 * Conventions (all arrays dense, row-major, no padding):
 *   image tensors  [B][H][W][Cx]
 *   qkv            [B][H][W][3][nh][d]     (0 = query, 1 = key, 2 = value)
 *   table          [(2M-1)^2][nh]          relative position bias, fp32
 *   rel_index      [N][N], N = M*M         int32
 *   mask           [nW][N][N]              0 or -100 (natural-log units)
 *   windows        [B][nWy][nWx][N][Cx]    token t = ty*M + tx in a window
 *   out            [B][H][W][nh*d]
 */
#ifndef SWIN_ORACLE_H
#define SWIN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element type codes of the qkv input accepted by the forward functions */
enum { ORACLE_F64 = 0, ORACLE_F32 = 1, ORACLE_BF16 = 2 /* raw 16-bit patterns */ };

/* cyclic roll with torch.roll semantics on dims (1,2) of [B][H][W][C]:
 * y[b][(i+sy) mod H][(j+sx) mod W][c] = x[b][i][j][c] */
void oracle_roll(const double* x, int B, int H, int W, int C, int sy, int sx, double* y);

/* window partition: win[b][wy][wx][ty*M+tx][c] = x[b][wy*M+ty][wx*M+tx][c] */
void oracle_window_partition(const double* x, int B, int H, int W, int C, int M, double* win);

/* window reverse, the inverse map of oracle_window_partition */
void oracle_window_reverse(const double* win, int B, int H, int W, int C, int M, double* x);

/* relative position index of query i and key j inside an M x M window */
void oracle_rel_index(int M, int32_t* idx);

/* region label image [H][W] of the shifted frame: three bands per axis,
 * [0,H-M), [H-M,H-s), [H-s,H); label = 3*band_y + band_x; all zero if s == 0 */
void oracle_region_labels(int H, int W, int M, int s, int32_t* lab);

/* shifted-window mask [nW][N][N]: 0 where query and key carry the same
 * region label, -100 elsewhere (all zero when s == 0) */
void oracle_shift_mask(int H, int W, int M, int s, double* mask);

/* attention inside windows.  win_qkv [nWin][N][3][nh][d]; window n uses
 * mask[n mod nW] (mask may be NULL = no mask).  npad >= N pads every window
 * to npad tokens: padded keys get score -inf, padded tokens are zero and
 * padded query rows are dropped.  win_out [nWin][N][nh*d].
 * nthreads <= 0 uses every online CPU.  Returns the thread count used. */
int oracle_window_attention(const double* win_qkv, const float* table, const double* mask,
                            long nWin, int nW, int M, int nh, int d, int npad, int nthreads,
                            double* win_out);

/* the whole forward: roll(-s,-s) -> partition -> window attention with bias
 * and mask -> reverse -> roll(+s,+s).  qkv of type dtype, out fp64
 * [B][H][W][nh*d].  Returns the thread count used, or -1 on bad arguments. */
int oracle_swin_wattn_fwd(const void* qkv, int dtype, const float* table, int B, int H, int W,
                          int nh, int d, int M, int s, int npad, int nthreads, double* out);

/* the same forward restricted to selected windows, for spot checks at sizes
 * too large for the whole forward.  sel[k] = b*nW + w.  out [nsel][N][nh*d]
 * in window token order; pos[k*N+t] = (b*H + y)*W + x is the image position
 * that token t of window sel[k] is read from and written back to.
 * Returns the thread count used, or -1 on bad arguments. */
int oracle_swin_wattn_windows(const void* qkv, int dtype, const float* table, int B, int H,
                              int W, int nh, int d, int M, int s, long nsel, const int64_t* sel,
                              int nthreads, double* out, int64_t* pos);

/* Linear layer with bias and optional residual, the operations on either
 * side of the attention:
 *   y[t][j] = sum_c x[t][c] * w[j][c] + bias[j]  (+ residual[t][j])
 * x [T][K] of type xdtype; w [N][K] of type wdtype (out_features x
 * in_features); bias [N] fp32 or NULL (no bias); residual [T][N] of type
 * rdtype or NULL (no residual); y [T][N] fp64.
 *  - QKV GEMM + bias: K = C, N = 3C, output columns in [3][nh][d] order,
 *    which is the qkv token row the attention reads (NVIDIA talk, section 3
 *    "inference optimization": the QKV GEMM is fused with its bias, in a
 *    format prepared for the attention kernel).
 *  - Output projection + bias + residual: K = N = C (same section: the
 *    add-bias-then-add-residual kernel).
 * Returns the thread count used, or -1 on bad arguments. */
int oracle_linear(const void* x, int xdtype, long T, int K, const void* w, int wdtype, int N,
                  const float* bias, const void* residual, int rdtype, int nthreads, double* y);

/* INT8 quantized q, k and v (NVIDIA talk, section 3, INT8 quantization:
 * tensors quantized to INT8 carry a scale, and dequantizing multiplies the
 * code by it).  codes [tokens][3][C] int8, one scale per part (query, key,
 * value): out[t][p][c] = codes[t][p][c] * scales[p], fp64.  The INT8
 * attention is the forward of these dequantized values. */
void oracle_dequant_qkv_i8(const int8_t* codes, long tokens, int C, const float* scales,
                           double* out);

/* INT8 linear layer (NVIDIA talk, section 3, INT8 quantization: input and
 * weight quantized to INT8, products accumulated in INT32, the sum
 * dequantized; bias and residual stay in floating point).  xq [T][K] int8
 * codes with one scale sx; wq [N][K] int8 codes with one scale per output
 * channel sw[N]; bias [N] fp32 or NULL:
 *   acc[t][j] = sum_c xq[t][c] * wq[j][c]                        exact, 64-bit
 *   y[t][j]   = acc[t][j] * sx * sw[j] + bias[j] (+ residual[t][j])      fp64
 * INT8 output (so != NULL, the form the talk takes for Swin): y is quantized
 * again with the scale so[j] of its column, a decision taken in fp32 as one
 * fused multiply-add per output (fl = round to nearest fp32):
 *   yq[t][j] = clamp(round_half_even(fma(fl(acc), fl(fl(sx*sw[j]) / so[j]),
 *                                        fl(bias[j] / so[j]))), -127, 127)
 * No residual with INT8 output.  acc, y and yq may each be NULL (not
 * computed).  Returns the thread count used, or -1 on bad arguments. */
int oracle_linear_i8(const int8_t* xq, long T, int K, float sx, const int8_t* wq, int N,
                     const float* sw, const float* bias, const void* residual, int rdtype,
                     const float* so, int nthreads, int64_t* acc, double* y, int8_t* yq);

/* Layer normalisation over the last dimension, fp64:
 *   mu[t] = mean_c x[t][c],  var[t] = mean_c (x[t][c] - mu[t])^2
 *   y[t][c] = (x[t][c] - mu[t]) / sqrt(var[t] + eps) * gamma[c] + beta[c]
 * x [T][C] of type xdtype; gamma, beta [C] fp32; y [T][C] fp64.  In a Swin
 * block it precedes the window attention; the pages fuse it with the window
 * shift and partition into one kernel (NVIDIA talk, section 3).
 * Returns 0, or -1 on bad arguments. */
int oracle_layernorm(const void* x, int xdtype, long T, int C, const float* gamma,
                     const float* beta, double eps, double* y);

/* Backward of oracle_swin_wattn_fwd: given dout = dL/d(out) [B][H][W][nh*d]
 * (type dout_dtype), the gradients with respect to qkv, dqkv [B][H][W][3][nh][d]
 * fp64, and to the bias table, dtable [(2M-1)^2][nh] fp64.  Per window and
 * head, with S = Q K^T / sqrt(d) + bias + mask, P = softmax(S), O = P V:
 *   dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,  dS = P o (dP - D),
 *   dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d),  dtable[rel(i,j)][h] += dS_ij
 * (summed over every window and image); dO is dout gathered through the
 * same roll and partition as qkv, and dqkv goes back through the reverse
 * maps.  The NVIDIA talk, section 2, fuses this backward for training.
 * Returns the thread count used, or -1 on bad arguments. */
int oracle_swin_wattn_bwd(const void* qkv, int dtype, const float* table, const void* dout,
                          int dout_dtype, int B, int H, int W, int nh, int d, int M, int s,
                          int nthreads, double* dqkv, double* dtable);

#ifdef __cplusplus
}
#endif
#endif
