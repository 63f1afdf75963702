// Internal interface between the C-ABI front (swinattn_api.hip) and the
// fused layer norm + QKV projection + window attention kernel
// (ln_qkv_wattn.hip).  Not installed, not part of the ABI.
#pragma once

#include "wattn_internal.h"

namespace swinattn {

// windows of 5 to 8 tokens a side (4 token tiles), C = 32 .. 192 channels
constexpr int kMinLnAttnWindow = 5, kMaxLnAttnWindow = 8, kMaxLnAttnC = 192;
struct LnAttnParams {
  const void* x;        // [B][H][W][C] bf16, raw token rows of this launch's images
  const void* wp;       // packed gamma o W_qkv, [3C/32][C/32][2][64][8] bf16
  const float* consts;  // [2][3C]: row sums of the packed weight, then bias + W beta
  const float* table;   // [(2M-1)^2][nh]
  void* out;            // [B][H][W][C] bf16
  float eps;
  int B, H, W, nh, C, N, shift;  // N = 3C
  int nWy, nWx, nW;
  int windows;          // B * nW
  int streams;          // streams of windows (set by the launcher)
  float score_scale;    // log2(e) / sqrt(head_dim)
  float inv_scale;      // sqrt(head_dim)
  float mask_pieces[3];
};
hipError_t launch_ln_qkv_wattn(int M, const LnAttnParams& p, int dev, int cus,
                               hipStream_t stream);

}  // namespace swinattn
