// Internal interface between the C-ABI front (swinattn_api.hip) and the
// kernels (wattn_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swinattn {

constexpr int kHeadDim = 32;    // one MFMA K-step (16x16x32 bf16) per score tile
constexpr int kMaxWindow = 12;  // N = 144 = 9 tiles of 16 tokens
constexpr int kMaxTableLds = 64 * 1024;

struct FwdParams {
  const void* qkv;          // [B][H][W][3][nh][32]
  const float* table;       // [(2M-1)^2][nh]
  void* out;                // [B][H][W][nh*32]
  const int32_t* rel_index; // [N][N] precomputed
  const uint8_t* region;    // [nW][N] precomputed region labels
  const uint8_t* has_mask;  // [nW] precomputed: 1 if the window's labels differ
  int B, H, W, nh, shift;
  int nWx, nW;
  int total_windows;        // B * nW (grid size)
  float score_scale;        // log2(e) / sqrt(head_dim)
  float inv_scale;          // sqrt(head_dim): bias and mask are pre-divided by the scale
  float mask_value;         // -100 * sqrt(head_dim)
};

// Queues the precompute kernel.  rel_index [N*N], mask [nW*N*N],
// region [nW*N], has_mask [nW].
hipError_t launch_precompute(int H, int W, int M, int s, int32_t* rel_index, float* mask,
                             uint8_t* region, uint8_t* has_mask, hipStream_t stream);

// Queue the forward kernels; M in [1, kMaxWindow].  `waves` = waves per
// workgroup (heads are dealt round-robin to waves).
hipError_t launch_fwd_bf16(int M, const FwdParams& p, int waves, hipStream_t stream);
hipError_t launch_fwd_f32(int M, const FwdParams& p, int waves, hipStream_t stream);

}  // namespace swinattn
