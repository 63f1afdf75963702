// Internal interface between the C-ABI front (swinattn_api.hip) and the
// attention backward kernel (wattn_backward.hip).  Not installed, not part of the ABI.
#pragma once

#include "wattn_internal.h"

namespace swinattn {

// Backward of the window attention, bf16 (wattn_backward.hip); windows up
// to kMaxBwdWindow.
constexpr int kMaxBwdWindow = 12;
struct BwdParams {
  const void* qkv;     // [B][H][W][3][nh][32] of this launch's images
  const float* table;  // [(2M-1)^2][nh]
  const void* dout;    // [B][H][W][nh*32]
  void* dqkv;          // [B][H][W][3][nh][32]
  float* dtable;       // [(2M-1)^2][nh], accumulated with atomics (zeroed by the host)
  int B, H, W, nh, shift;
  int nWy, nWx, nW;
  int windows;         // B * nW
  int xcd_streams;     // 1: grid a multiple of 8 * nh / HP, the head groups of a run on one
                       // XCD; 2 (one head per workgroup, even nh): the two heads of each
                       // 128-byte line of a run on one XCD
  int runs;            // runs of windows (the grid holds runs * nh / HP workgroups, and in
                       // mode 2 up to 7 idle pairs of workgroups)
  unsigned dqkv_bytes; // bytes of dqkv in this launch (at most 2^31)
  float scale;         // 1 / sqrt(head_dim)
  float score_scale;   // log2(e) / sqrt(head_dim)
  float inv_scale;     // sqrt(head_dim)
  float mask_pieces[3];
};
size_t bwd_lds_bytes(int M);
hipError_t launch_bwd_bf16(int M, const BwdParams& p, int dev, int cus, hipStream_t stream);
hipError_t launch_fill(float* dst, long long n, float v, hipStream_t stream);

}  // namespace swinattn
