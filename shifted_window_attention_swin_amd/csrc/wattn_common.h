// Device-side building blocks shared by the forward kernels of libswinattn
// (gfx950).  Internal: included by the .hip sources of the library only.
#pragma once

#include "wattn_internal.h"

namespace swinattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#define SWA_INLINE __device__ __forceinline__

template <int M>
struct Win {
  static constexpr int Q = (M + 3) / 4;        // 4-token quads per row and 4-row groups
  static constexpr int P = 4 * Q;              // padded window side
  static constexpr int NT = Q * Q;             // 16-token tiles
  static constexpr int NK = (NT + 1) / 2;      // 32-key steps of the value product
  static constexpr int D = 2 * M - 1;          // side of the relative position table
  static constexpr int T = D * D;              // table rows
  static constexpr int C0 = (M - 1) * D + (M - 1);  // index of offset (0, 0)
  static constexpr int LG = M - 4 * (Q - 1);   // window rows present in the last row group
  static constexpr int TAIL = 2 * M * (P - M); // LDS slack read by padded keys
  // key row r of tile t: window column 4*(t%Q) + r exists
  static constexpr bool col_ok(int t, int r) { return 4 * (t % Q) + r < M; }
  // every lane group of tile t is a window row
  static constexpr bool rows_all(int t) { return 4 * (t / Q) + 3 < M; }
  // code (2M-1)*row + col of in-tile token 0 of tile t
  static constexpr int E(int t) { return 4 * D * (t / Q) + 4 * (t % Q); }
};

// Workgroups are dealt round-robin to the 8 XCDs; renumber them so that each
// XCD (and its L2) works on one contiguous run of windows.
SWA_INLINE int xcd_window(int id, int G) {
  const int per = G >> 3, rem = G & 7, x = id & 7, k = id >> 3;
  return x * per + (x < rem ? x : rem) + k;
}

// Region of a shifted-frame position (yy, xx): three bands per axis,
// [0, L-M), [L-M, L-s), [L-s, L); label = 3*band_y + band_x (0 without shift).
SWA_INLINE int band_of(int pos, int L, int M, int s) {
  return pos < L - M ? 0 : (pos < L - s ? 1 : 2);
}
SWA_INLINE int region_label(int yy, int xx, int H, int W, int M, int s) {
  return s == 0 ? 0 : 3 * band_of(yy, H, M, s) + band_of(xx, W, M, s);
}
// Whether window (wy, wx) of an nWy x nWx grid holds more than one region.
// With 0 < s < M every window off the last window row and column lies inside
// band 0 of both axes; a window on the last row (column) holds rows
// (columns) of bands 1 and 2, each at least one wide.  So the mask is needed
// exactly there, and no per-window flag has to be read from memory.
SWA_INLINE bool window_masked(int s, int wy, int wx, int nWy, int nWx) {
  return s > 0 && (wy == nWy - 1 || wx == nWx - 1);
}

// Channel that column c of a value-transpose tile of channel half hf
// carries.  With this order, row 4g+r of output tile hf is channel
// 8g + 4hf + r: each lane ends up with 8 consecutive channels of its query
// token (one 16-byte store) instead of two 4-channel pieces 32 bytes apart.
SWA_INLINE int out_channel(int hf, int c) { return 8 * (c / 4) + 4 * hf + c % 4; }

// ds_read_b64_tr_b16: transposing 8-byte LDS read (see its use for the lane
// mapping).  `p` points into LDS.
SWA_INLINE bf16x4 lds_read_tr(const char* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(__attribute__((address_space(3))) char*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

SWA_INLINE float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
SWA_INLINE float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// max / sum over the four lane groups (lanes c, c+16, c+32, c+48)
SWA_INLINE float max_groups(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Softmax numerators of one query column block: s[jt][r] holds D of key row
// (jt, 4g+r) for the lane's query.  Replaces s by exp2(D*scale - max*scale);
// rows outside the window become 0.
template <int M>
SWA_INLINE void softmax_numerators(f32x4 (&s)[Win<M>::NT], float score_scale) {
  using S = Win<M>;
  float m = -__builtin_inff();
#pragma unroll
  for (int jt = 0; jt < S::NT; ++jt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (S::col_ok(jt, r)) m = fmaxf(m, s[jt][r]);
  m = max_groups(m);
  const float nms = -m * score_scale;
#pragma unroll
  for (int jt = 0; jt < S::NT; ++jt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      s[jt][r] = S::col_ok(jt, r) ? fast_exp2(fmaf(s[jt][r], score_scale, nms)) : 0.f;
}

// bias table -> LDS: per head, reversed, divided by the score scale; then a
// zero tail that padded keys may read
template <int M>
SWA_INLINE void stage_bias(float* s_bias, const float* table, int nh, float inv_scale) {
  using S = Win<M>;
  const int n = nh * S::T;
  for (int e = threadIdx.x; e < n + S::TAIL; e += blockDim.x) {
    float v = 0.f;
    if (e < n) {
      const int h = e / S::T, k = e - h * S::T;
      v = table[(S::T - 1 - k) * nh + h] * inv_scale;
    }
    s_bias[e] = v;
  }
}

}  // namespace
}  // namespace swinattn
