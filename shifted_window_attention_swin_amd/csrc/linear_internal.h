// Internal interface between the C-ABI front (swinattn_api.hip) and the
// linear-layer kernels (linear_gemm.hip).  Not installed, not part of the ABI.
#pragma once

#include "wattn_internal.h"

namespace swinattn {

// Linear layer y = x W^T + bias (+ residual), bf16 in and out, fp32 bias
// (linear_gemm.hip).  K and N are multiples of 32, K <= kMaxLinearK.  The
// int8 layer (w_scale set) takes K <= kMaxLinearKI8.
constexpr int kMaxLinearK = 384;
constexpr int kMaxLinearKI8 = 768;
constexpr long long kMaxLinearTokens = 1LL << 30;  // tokens per launch (32-bit indices)
struct LinearParams {
  const void* x;      // [T][K] bf16
  const void* wp;     // packed weight [N/32][K/32][2][64][8] bf16
  const float* bias;  // [N] or null
  const void* res;    // [T][N] bf16 or null
  const float* colsum;  // layer norm: [N] row sums of the packed weight, or null
  float eps;            // layer norm epsilon
  void* y;            // [T][N] bf16 (int8 with out_scale)
  long long T;
  int K, N;
  int ncb;     // N / 32 column blocks
  int ncg;     // column groups, one per workgroup (set by launch_linear)
  int blocks;  // row blocks (set by launch_linear)
  float x_scale;            // int8: scale of the x codes
  const float* w_scale;     // int8: [N] scales of the weight rows; null for bf16
  const float* out_scale;   // int8 output: [N] scales of the output columns, or null
  int half_step;  // int8, K % 64 == 32: the last k-step is half (set by launch_linear)
};
// gamma null: plain packing; else the packed weight is gamma o W.
hipError_t launch_linear_pack(const void* w, const float* gamma, void* wp, int N, int K,
                              hipStream_t stream);
// consts [2][N]: row sums of gamma o W (as packed), bias + W beta.
hipError_t launch_linear_ln_consts(const void* w, const float* gamma, const float* beta,
                                  const float* bias, float* consts, int N, int K,
                                  hipStream_t stream);
// int8 weight [N][K] -> packed [N/32][ceil(K/64)][2][64][16] int8
hipError_t launch_linear_pack_i8(const void* w, void* wp, int N, int K, hipStream_t stream);
hipError_t launch_linear(const LinearParams& p, int dev, int cus, hipStream_t stream);

}  // namespace swinattn
