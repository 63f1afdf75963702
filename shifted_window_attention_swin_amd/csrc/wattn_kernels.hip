// fp32 forward and setup precompute of libswinattn (gfx950, wave64).
//
// fp32 forward (the tight correctness check): one workgroup per (image,
// window), its waves taking the heads round-robin; a wave holds one head's
// query, key and value tiles in registers and runs the math described in
// wattn_persistent.hip on v_mfma_f32_16x16x4f32 (K = 4 per step: lane group g
// supplies channel 8g + st at step st, for Q and K alike), with the shift
// mask as per-element selects and V^T from MFMAs against 0/1 selectors.
// The tiles are loaded straight from HBM in operand layout: the cyclic shift
// and the window partition are the address arithmetic of these loads (talk
// "Swin Transformer training and inference optimization", uticex.com 1598,
// section 2: the window ops are index mapping; section 3: transposes folded
// into the kernel's loads and stores).  Windows of more than 4 tiles read
// key and value tiles again (from cache) for every query tile, which keeps
// the kernel within its registers.
//
// Setup precompute: the relative position index, the shift mask and the
// region labels as tensors, for callers that keep them and for
// verification; the forward and backward kernels evaluate the same closed
// forms from token coordinates instead of reading these tensors.

#include "wattn_common.h"

namespace swinattn {
namespace {

// Everything a lane needs about its tokens, built once per workgroup.
template <int M>
struct LaneWindow {
  using S = Win<M>;
  unsigned in_off[S::NT];   // byte offset of this lane's slice of token (t, c) in the qkv chunk
  unsigned out_off[S::NT];  // byte offset of this lane's slice of token (t, c) in the out chunk
  int qbase[S::NT];         // reversed-table index base of query (t, c) for lane group g
  bool ok[S::NT];           // token (t, c) lies inside the window
  int li[S::NT];            // region label of query (t, c)            (masked windows)
  int lj[S::NT][4];         // region label of key row (t, 4g + r)     (masked windows)

  SWA_INLINE void init(const FwdParams& p, int b, int w, int g, int c, int elem) {
    const int wy = w / p.nWx, wx = w - wy * p.nWx;
    const unsigned C = (unsigned)p.nh * kHeadDim;
#pragma unroll
    for (int t = 0; t < S::NT; ++t) {
      const int ty = 4 * (t / S::Q) + c / 4, tx = 4 * (t % S::Q) + c % 4;
      ok[t] = ty < M && tx < M;
      // query code (2M-1)*row + col; padded queries borrow token (0, 0)
      const int a = ok[t] ? S::D * ty + tx : 0;
      qbase[t] = S::T - 1 - S::C0 - a + S::D * g;
      // shifted-frame (wy*M+ty, wx*M+tx) holds image position + shift (mod H, W)
      int y = wy * M + (ok[t] ? ty : 0) + p.shift, x = wx * M + (ok[t] ? tx : 0) + p.shift;
      y -= y >= p.H ? p.H : 0;
      x -= x >= p.W ? p.W : 0;
      const unsigned pix = ((unsigned)b * p.H + y) * p.W + x;
      in_off[t] = (pix * 3u * C + 8u * g) * elem;
      out_off[t] = (pix * C + 8u * g) * elem;
    }
  }

  SWA_INLINE void init_labels(const FwdParams& p, int w, int g, int c) {
    const int wy = w / p.nWx, wx = w - wy * p.nWx;
#pragma unroll
    for (int t = 0; t < S::NT; ++t) {
      const int ty = 4 * (t / S::Q) + c / 4, tx = 4 * (t % S::Q) + c % 4;
      li[t] = region_label(wy * M + ty, wx * M + tx, p.H, p.W, M, p.shift);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        lj[t][r] = region_label(wy * M + 4 * (t / S::Q) + g, wx * M + 4 * (t % S::Q) + r, p.H, p.W,
                                M, p.shift);
    }
  }

  // accumulator initialisation of score tile (key tile jt, query tile it):
  // (bias + mask) / scale, -inf for keys outside the window
  SWA_INLINE f32x4 score_init(const float* s_bias, int hbase, int it, int jt, bool g_ok,
                              bool select_mask, float mask_value) const {
    f32x4 acc;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (!S::col_ok(jt, r)) {
        acc[r] = -__builtin_inff();
        continue;
      }
      float v = s_bias[hbase + qbase[it] + S::E(jt) + r];
      if (!S::rows_all(jt)) v = g_ok ? v : -__builtin_inff();
      if (select_mask) v = (li[it] == lj[jt][r]) ? v : v + mask_value;
      acc[r] = v;
    }
    return acc;
  }
};

// ---------------------------------------------------------------------------
// fp32 forward: the same layout with v_mfma_f32_16x16x4_f32 (K = 4 per step;
// lane group g supplies channel 8g+st at step st, for Q and K alike)

template <int M>
SWA_INLINE void head_f32(const FwdParams& p, const LaneWindow<M>& lw, const float* s_bias,
                         const char* in, char* out, int h, int g, int c, bool g_ok, bool masked) {
  using S = Win<M>;
  constexpr int NT = S::NT;
  // windows of up to 4 tiles hold every key tile and V^T for all query
  // tiles; larger windows re-read them (from cache) per query tile, which
  // keeps the kernel within its registers
  constexpr bool HOLD = NT <= 4;
  constexpr int NH = HOLD ? NT : 1;
  const unsigned Cb = (unsigned)p.nh * kHeadDim * 4;
  const char* in_h = in + h * kHeadDim * 4;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  // key tile t (its two 4-channel halves) and V^T of tile t
  auto load_k = [&](int t, f32x4 (&k)[2]) {
    k[0] = z;
    k[1] = z;
    if (lw.ok[t]) {
      const char* src = in_h + lw.in_off[t] + Cb;
      k[0] = *reinterpret_cast<const f32x4*>(src);
      k[1] = *reinterpret_cast<const f32x4*>(src + 16);
    }
  };
  auto load_vt = [&](int t, f32x4 (&vt)[2]) {
    f32x4 v0 = z, v1 = z;
    if (lw.ok[t]) {
      const char* src = in_h + lw.in_off[t] + 2 * Cb;
      v0 = *reinterpret_cast<const f32x4*>(src);
      v1 = *reinterpret_cast<const f32x4*>(src + 16);
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x4 acc = z;
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const float sv = (8 * g + st == out_channel(hf, c)) ? 1.f : 0.f;
        const float vv = st < 4 ? v0[st] : v1[st - 4];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(vv, sv, acc, 0, 0, 0);
      }
      vt[hf] = acc;
    }
  };
  f32x4 kk[NH][2], vt[NH][2];
  if constexpr (HOLD) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      load_k(t, kk[t]);
      load_vt(t, vt[t]);
    }
  }
  const int hbase = h * S::T;
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    // re-read tiles: an address opaque to the compiler per query tile, so
    // the loads of different query tiles are not merged (and held)
    if constexpr (!HOLD) asm volatile("" : "+v"(in_h));
    f32x4 q0 = z, q1 = z;
    if (lw.ok[it]) {
      const char* src = in_h + lw.in_off[it];
      q0 = *reinterpret_cast<const f32x4*>(src);
      q1 = *reinterpret_cast<const f32x4*>(src + 16);
    }
    f32x4 s[NT];
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
      f32x4 acc = lw.score_init(s_bias, hbase, it, jt, g_ok, masked, p.mask_value);
      f32x4 kj[2];
      if constexpr (HOLD) {
        kj[0] = kk[jt][0];
        kj[1] = kk[jt][1];
      } else {
        load_k(jt, kj);
      }
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const float ka = st < 4 ? kj[0][st] : kj[1][st - 4];
        const float qb = st < 4 ? q0[st] : q1[st - 4];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka, qb, acc, 0, 0, 0);
      }
      s[jt] = acc;
    }
    softmax_numerators<M>(s, p.score_scale);
    f32x4 o0 = z, o1 = z, l4 = z;
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
      f32x4 vj[2];
      if constexpr (HOLD) {
        vj[0] = vt[jt][0];
        vj[1] = vt[jt][1];
      } else {
        load_vt(jt, vj);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (!S::col_ok(jt, r)) continue;
        o0 = __builtin_amdgcn_mfma_f32_16x16x4f32(vj[0][r], s[jt][r], o0, 0, 0, 0);
        o1 = __builtin_amdgcn_mfma_f32_16x16x4f32(vj[1][r], s[jt][r], o1, 0, 0, 0);
        l4 = __builtin_amdgcn_mfma_f32_16x16x4f32(1.f, s[jt][r], l4, 0, 0, 0);
      }
    }
    if (lw.ok[it]) {
      const float inv = fast_rcp(l4[0]);
      char* dst = out + h * kHeadDim * 4 + lw.out_off[it];
      *reinterpret_cast<f32x4*>(dst) = o0 * inv;
      *reinterpret_cast<f32x4*>(dst + 16) = o1 * inv;
    }
    // keep query tiles apart: interleaving them only raises register pressure
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int M>
__global__ __launch_bounds__(256) void wattn_fwd_f32_kernel(FwdParams p) {
  using S = Win<M>;
  extern __shared__ float s_bias[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int win = xcd_window(blockIdx.x, p.total_windows);
  const int b = win / p.nW, w = win - b * p.nW;
  const char* in = static_cast<const char*>(p.qkv);
  char* out = static_cast<char*>(p.out);

  stage_bias<M>(s_bias, p.table, p.nh, p.inv_scale);
  LaneWindow<M> lw;
  lw.init(p, b, w, g, c, 4);
  const bool g_ok = g < S::LG;
  __syncthreads();
  const bool masked = window_masked(p.shift, w / p.nWx, w % p.nWx, p.nWy, p.nWx);
  if (masked) lw.init_labels(p, w, g, c);
  for (int h = wave; h < p.nh; h += nwaves) head_f32<M>(p, lw, s_bias, in, out, h, g, c, g_ok, masked);
}

// ---------------------------------------------------------------------------
// setup: relative position index, shift mask, region labels

__global__ void precompute_kernel(int H, int W, int M, int s, int32_t* rel_index, float* mask,
                                  uint8_t* region) {
  const int N = M * M, nWx = W / M, nW = (H / M) * nWx;
  const long long total = (long long)nW * N * N;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
    const int j = (int)(e % N);
    const long long rest = e / N;
    const int i = (int)(rest % N), w = (int)(rest / N);
    const int wy = w / nWx, wx = w - wy * nWx;
    const int li = region_label(wy * M + i / M, wx * M + i % M, H, W, M, s);
    const int lj = region_label(wy * M + j / M, wx * M + j % M, H, W, M, s);
    mask[e] = li == lj ? 0.f : -100.f;
    if (w == 0) {
      const int dy = i / M - j / M, dx = i % M - j % M;
      rel_index[i * N + j] = (dy + M - 1) * (2 * M - 1) + (dx + M - 1);
    }
    if (j == 0) region[(long long)w * N + i] = (uint8_t)li;
  }
}

template <int M>
size_t lds_bytes(int nh) {
  return ((size_t)Win<M>::T * nh + Win<M>::TAIL) * sizeof(float);
}

template <int M>
hipError_t launch_f32_m(const FwdParams& p, int waves, hipStream_t st) {
  hipLaunchKernelGGL(wattn_fwd_f32_kernel<M>, dim3(p.total_windows), dim3(64 * waves),
                     lds_bytes<M>(p.nh), st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_precompute(int H, int W, int M, int s, int32_t* rel_index, float* mask,
                             uint8_t* region, hipStream_t stream) {
  const long long total = (long long)(H / M) * (W / M) * M * M * M * M;
  long long blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(precompute_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, H, W, M, s,
                     rel_index, mask, region);
  return hipGetLastError();
}

size_t fwd_lds_bytes(int M, int nh) {
  switch (M) {
#define SWA_LDS_CASE(m) \
  case m: return lds_bytes<m>(nh);
    SWA_LDS_CASE(1) SWA_LDS_CASE(2) SWA_LDS_CASE(3) SWA_LDS_CASE(4) SWA_LDS_CASE(5)
    SWA_LDS_CASE(6) SWA_LDS_CASE(7) SWA_LDS_CASE(8) SWA_LDS_CASE(9) SWA_LDS_CASE(10)
    SWA_LDS_CASE(11) SWA_LDS_CASE(12)
#undef SWA_LDS_CASE
    default: return 0;
  }
}

#define SWA_DISPATCH(FN)                                \
  switch (M) {                                          \
    case 1: return FN<1>(p, waves, stream);             \
    case 2: return FN<2>(p, waves, stream);             \
    case 3: return FN<3>(p, waves, stream);             \
    case 4: return FN<4>(p, waves, stream);             \
    case 5: return FN<5>(p, waves, stream);             \
    case 6: return FN<6>(p, waves, stream);             \
    case 7: return FN<7>(p, waves, stream);             \
    case 8: return FN<8>(p, waves, stream);             \
    case 9: return FN<9>(p, waves, stream);             \
    case 10: return FN<10>(p, waves, stream);           \
    case 11: return FN<11>(p, waves, stream);           \
    case 12: return FN<12>(p, waves, stream);           \
    default: return hipErrorInvalidValue;               \
  }

hipError_t launch_fwd_f32(int M, const FwdParams& p, int waves, hipStream_t stream) {
  SWA_DISPATCH(launch_f32_m)
}

}  // namespace swinattn
