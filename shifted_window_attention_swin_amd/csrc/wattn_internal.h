// Internal interface between the C-ABI front (swinattn_api.hip) and the
// forward attention kernels, and the limits the kernel families share.
// Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swinattn {

constexpr int kHeadDim = 32;    // one MFMA K-step (16x16x32 bf16) per score tile
constexpr int kMaxWindow = 12;  // N = 144 = 9 tiles of 16 tokens
// bias tables of every head staged by one persistent forward workgroup, at
// most (beyond it the workgroup stages one head group's tables)
constexpr int kMaxTableLds = 64 * 1024;
constexpr int kMaxLds = 160 * 1024;  // LDS of one workgroup on gfx950
// In-kernel token offsets are 32-bit: one launch covers at most this many
// bytes of qkv; larger batches are split into several launches.
constexpr long long kMaxChunkBytes = 1LL << 31;
constexpr int kMaxDevices = 64;  // devices with cached launch properties

struct FwdParams {
  const void* qkv;          // [B][H][W][3][nh][32], B = images of this launch
  const float* table;       // [(2M-1)^2][nh]
  void* out;                // [B][H][W][nh*32]
  int B, H, W, nh, shift;
  int nWy, nWx, nW;         // window grid: rows, columns, rows * columns
  int total_windows;        // B * nW (grid size of the per-window kernels)
  int units;                // B * nW * nhg (work units of the persistent kernel)
  int nhg;                  // head groups per window (persistent kernel)
  int xcd_ranges;           // persistent kernel: one contiguous unit range per XCD
  int own_bias;             // persistent kernel: 0 every head's tables, 1 the workgroup's head
                            // group's, 2 the current unit's head group's (restaged)
  float score_scale;        // log2(e) * scale; scale = 1 / sqrt(head_dim) (times the query
                            // and key scales for int8 codes)
  float inv_scale;          // 1 / scale: bias and mask are pre-divided by the scale
  float mask_value;         // -100 * sqrt(head_dim)
  float mask_pieces[3];     // bf16-exact parts summing to 100 * inv_scale in fp32
  float v_scale;            // int8 forward: scale of the value codes (over the output scale
                            // for int8 output)
  int out_i8;               // int8 forward: int8 output codes instead of bf16
};

// Queues the precompute kernel.  rel_index [N*N], mask [nW*N*N],
// region [nW*N].
hipError_t launch_precompute(int H, int W, int M, int s, int32_t* rel_index, float* mask,
                             uint8_t* region, hipStream_t stream);

// Queue the fp32 forward kernel; M in [1, kMaxWindow].  `waves` = waves per
// workgroup (heads are dealt round-robin to waves).
hipError_t launch_fwd_f32(int M, const FwdParams& p, int waves, hipStream_t stream);
// Dynamic LDS of one fp32 forward workgroup (every head's bias table plus
// slack); at most kMaxLds.
size_t fwd_lds_bytes(int M, int nh);

// Persistent LDS-staged bf16 forward (every window up to kMaxWindow, any
// number of heads): heads are processed in groups of HG (1..4, HG divides nh;
// 1 for windows of more than 4 tiles); `dev` = current device, `cus` = its
// compute units (the grid fills them at the kernel's occupancy, cached per
// device).
hipError_t launch_fwd_bf16_persistent(int M, int HG, const FwdParams& p, int dev, int cus,
                                      hipStream_t stream);
// The same kernel for int8 q, k, v codes (bf16 output); p.score_scale,
// p.inv_scale and p.mask_pieces carry the query and key scales, p.v_scale the
// value scale.
hipError_t launch_fwd_i8_persistent(int M, int HG, const FwdParams& p, int dev, int cus,
                                    hipStream_t stream);

}  // namespace swinattn
