// Kernels of libswinattn for gfx950 (MI355X, CDNA4, wave64).
//
// Forward: one workgroup per (image, window); the workgroup's waves take the
// heads round-robin.  For one head a wave holds the whole window in VGPRs:
//
//   Q, K, V   16-token tiles loaded straight from HBM in MFMA operand layout
//             (lane = token 16t + lane%16, 16 bytes of head_dim each); the
//             cyclic shift and window partition are the address arithmetic of
//             these loads (talk "Swin Transformer training and inference
//             optimization", uticex.com 1598, section 2: the window ops are
//             index mapping; section 3: transposes folded into the kernel's
//             loads and stores).
//   S^T = K Q^T + C   v_mfma_f32_16x16x32_bf16, K = head_dim = 32 exactly.
//             The accumulator C is initialised with the relative position bias
//             (gathered from a head-major copy of the table in LDS) plus the
//             shift mask, both divided by the score scale, so one fma later
//             turns D into a base-2 logit.  Transposing S puts one query per
//             lane column: the softmax over keys is an in-lane reduction plus
//             two cross-lane steps.
//   P^T       exp2, row sums in fp32, P rounded to bf16; the C/D layout of S^T
//             is directly the B-operand layout of the next MFMA.
//   O^T = V^T P^T   V^T in operand layout comes from an MFMA against a 0/1
//             selector (an exact transpose inside the matrix core).
//   store     lane writes 4 consecutive channels of one token: the window
//             reverse and the roll back are the store addresses.
//
// Tiles: N = window^2 tokens padded to NT*16.  Padded keys get -inf in the
// accumulator initialisation (weight exactly 0); padded tokens load as zero
// (0 * finite = 0 in the value product); padded queries are not stored.

#include "wattn_internal.h"

namespace swinattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define SWA_INLINE __device__ __forceinline__

template <int M>
struct Win {
  static constexpr int N = M * M;
  static constexpr int NT = (N + 15) / 16;      // 16-token tiles
  static constexpr int LV = N - 16 * (NT - 1);  // valid tokens of the last tile (1..16)
  static constexpr int T = (2 * M - 1) * (2 * M - 1);
  static constexpr int NK = (NT + 1) / 2;       // 32-key steps of the bf16 value product
  // row r of key tile t holds key 16t + 4g + r, g = lane / 16
  static constexpr bool row_empty(int t, int r) { return t == NT - 1 && r >= LV; }
  static constexpr bool row_full(int t, int r) { return t < NT - 1 || 12 + r < LV; }
};

// Workgroups are dealt round-robin to the 8 XCDs; renumber them so that each
// XCD (and its L2) works on one contiguous run of windows.
SWA_INLINE int xcd_window(int id, int G) {
  const int per = G >> 3, rem = G & 7, x = id & 7, k = id >> 3;
  return x * per + (x < rem ? x : rem) + k;
}

SWA_INLINE float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
SWA_INLINE float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Everything a lane needs about its tokens, built once per workgroup.
template <int M>
struct LaneWindow {
  using S = Win<M>;
  int rc[S::NT];      // query code  rel_index[i][0] - rel_index[0][0], i = 16t + c
  int cc[S::NT][4];   // key code    rel_index[0][j], j = 16t + 4g + r
  int li[S::NT];      // region label of query i (masked windows only)
  int lj[S::NT][4];   // region label of key j
  long long pix[S::NT];  // flattened image position of token 16t + c
  bool ok[S::NT];     // token 16t + c exists

  SWA_INLINE void init(const FwdParams& p, int b, int w, int g, int c, bool masked) {
    constexpr int N = S::N;
    const int wy = w / p.nWx, wx = w - wy * p.nWx;
    const int r00 = p.rel_index[0];
#pragma unroll
    for (int t = 0; t < S::NT; ++t) {
      const int i = 16 * t + c;
      ok[t] = i < N;
      const int ti = ok[t] ? i : 0;
      rc[t] = p.rel_index[ti * N] - r00;
      // shifted frame position (wy*M+ty, wx*M+tx) holds image position +shift (mod H, W)
      const int ty = ti / M, tx = ti - ty * M;
      int y = wy * M + ty + p.shift, x = wx * M + tx + p.shift;
      y -= y >= p.H ? p.H : 0;
      x -= x >= p.W ? p.W : 0;
      pix[t] = ((long long)b * p.H + y) * p.W + x;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * t + 4 * g + r;
        cc[t][r] = p.rel_index[j < N ? j : 0];
      }
    }
    if (masked) {
      const uint8_t* reg = p.region + (long long)w * N;
#pragma unroll
      for (int t = 0; t < S::NT; ++t) {
        li[t] = reg[ok[t] ? 16 * t + c : 0];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * t + 4 * g + r;
          lj[t][r] = reg[j < N ? j : 0];
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < S::NT; ++t) {
        li[t] = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) lj[t][r] = 0;
      }
    }
  }

  // accumulator initialisation of score tile (key tile jt, query tile it):
  // bias/scale (+ mask/scale), -inf for keys past N
  SWA_INLINE f32x4 score_init(const float* s_bias, int hoff, int it, int jt, int g, bool masked,
                              float mask_value) const {
    f32x4 acc;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v;
      if (S::row_empty(jt, r)) {
        v = -__builtin_inff();
      } else {
        v = s_bias[hoff + rc[it] + cc[jt][r]];
        if (!S::row_full(jt, r)) v = (4 * g + r < S::LV) ? v : -__builtin_inff();
        if (masked) v = (li[it] == lj[jt][r]) ? v : v + mask_value;
      }
      acc[r] = v;
    }
    return acc;
  }
};

// Row softmax of one query column block: s[jt][r] holds D for key 16jt+4g+r
// of the lane's query.  Replaces s by exp2(D*scale - max) and returns the
// (cross-lane complete) sum.
template <int M>
SWA_INLINE float softmax_cols(f32x4 (&s)[Win<M>::NT], float score_scale) {
  using S = Win<M>;
  float m = -__builtin_inff();
#pragma unroll
  for (int jt = 0; jt < S::NT; ++jt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (!S::row_empty(jt, r)) m = fmaxf(m, s[jt][r]);
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  const float nms = -m * score_scale;
  float l = 0.f;
#pragma unroll
  for (int jt = 0; jt < S::NT; ++jt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (S::row_empty(jt, r)) {
        s[jt][r] = 0.f;
      } else {
        const float e = fast_exp2(fmaf(s[jt][r], score_scale, nms));
        s[jt][r] = e;
        l += e;
      }
    }
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  return l;
}

// ---------------------------------------------------------------------------
// bf16 forward

template <int M>
SWA_INLINE void load_head_bf16(const __bf16* qkv, const LaneWindow<M>& lw, int C, int h, int g,
                               bf16x8 (&q)[Win<M>::NT], bf16x8 (&k)[Win<M>::NT],
                               bf16x8 (&v)[Win<M>::NT]) {
  using S = Win<M>;
#pragma unroll
  for (int t = 0; t < S::NT; ++t) {
    if (lw.ok[t]) {
      const __bf16* src = qkv + lw.pix[t] * (3LL * C) + h * kHeadDim + 8 * g;
      q[t] = *reinterpret_cast<const bf16x8*>(src);
      k[t] = *reinterpret_cast<const bf16x8*>(src + C);
      v[t] = *reinterpret_cast<const bf16x8*>(src + 2 * C);
    } else {
      q[t] = bf16x8{};
      k[t] = bf16x8{};
      v[t] = bf16x8{};
    }
  }
}

template <int M>
SWA_INLINE void head_bf16(const FwdParams& p, const LaneWindow<M>& lw, const float* s_bias,
                          __bf16* out, int C, int h, int g, bool masked, const bf16x8 (&sel)[2],
                          const bf16x8 (&q)[Win<M>::NT], const bf16x8 (&k)[Win<M>::NT],
                          const bf16x8 (&v)[Win<M>::NT]) {
  using S = Win<M>;
  constexpr int NT = S::NT, NK = S::NK;
  // V^T in A-operand layout: MFMA of each value tile against the selector of
  // channel half `hf` gives D[4g+r][c] = V[16t+4g+r][16hf+c] exactly
  bf16x8 va[2][NK];
#pragma unroll
  for (int kt = 0; kt < NK; ++kt)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      const f32x4 d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v[2 * kt], sel[hf], z, 0, 0, 0);
      f32x4 d1 = z;
      if (2 * kt + 1 < NT)
        d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v[2 * kt + 1], sel[hf], z, 0, 0, 0);
      bf16x8 a;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        a[r] = (__bf16)d0[r];
        a[4 + r] = (__bf16)d1[r];
      }
      va[hf][kt] = a;
    }

  const int hoff = h * S::T;
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    f32x4 s[NT];
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
      s[jt] = lw.score_init(s_bias, hoff, it, jt, g, masked, p.mask_value);
      s[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k[jt], q[it], s[jt], 0, 0, 0);
    }
    const float l = softmax_cols<M>(s, p.score_scale);
    // P^T as B operand: slots 0-3 = key tile 2kt, slots 4-7 = key tile 2kt+1
    bf16x8 pb[NK];
#pragma unroll
    for (int kt = 0; kt < NK; ++kt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pb[kt][r] = (__bf16)s[2 * kt][r];
        pb[kt][4 + r] = (2 * kt + 1 < NT) ? (__bf16)s[2 * kt + 1][r] : (__bf16)0.f;
      }
    }
    f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < NK; ++kt) {
      o0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[0][kt], pb[kt], o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[1][kt], pb[kt], o1, 0, 0, 0);
    }
    if (lw.ok[it]) {
      const float inv = fast_rcp(l);
      bf16x4 w0, w1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        w0[r] = (__bf16)(o0[r] * inv);
        w1[r] = (__bf16)(o1[r] * inv);
      }
      __bf16* dst = out + lw.pix[it] * C + h * kHeadDim + 4 * g;
      *reinterpret_cast<bf16x4*>(dst) = w0;
      *reinterpret_cast<bf16x4*>(dst + 16) = w1;
    }
  }
}

template <int M>
__global__ __launch_bounds__(256) void wattn_fwd_bf16_kernel(FwdParams p) {
  using S = Win<M>;
  constexpr int NT = S::NT, T = S::T;
  extern __shared__ float s_bias[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int win = xcd_window(blockIdx.x, p.total_windows);
  const int b = win / p.nW, w = win - b * p.nW;
  const int nh = p.nh, C = nh * kHeadDim;
  const __bf16* qkv = static_cast<const __bf16*>(p.qkv);
  __bf16* out = static_cast<__bf16*>(p.out);

  // bias table -> LDS, head-major, divided by the score scale
  for (int e = tid; e < T * nh; e += blockDim.x) {
    const int idx = e / nh, h = e - idx * nh;
    s_bias[h * T + idx] = p.table[e] * p.inv_scale;
  }
  const bool masked = p.has_mask[w] != 0;
  LaneWindow<M> lw;
  lw.init(p, b, w, g, c, masked);

  bf16x8 sel[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int s = 0; s < 8; ++s) sel[hf][s] = (8 * g + s == c + 16 * hf) ? (__bf16)1.f : (__bf16)0.f;

  bf16x8 q[NT], k[NT], v[NT];
  int h = wave;
  if (h < nh) load_head_bf16<M>(qkv, lw, C, h, g, q, k, v);
  __syncthreads();
  for (; h < nh; h += nwaves) {
    const bool more = h + nwaves < nh;
    bf16x8 qn[NT], kn[NT], vn[NT];
    if (more) load_head_bf16<M>(qkv, lw, C, h + nwaves, g, qn, kn, vn);
    head_bf16<M>(p, lw, s_bias, out, C, h, g, masked, sel, q, k, v);
    if (more) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        q[t] = qn[t];
        k[t] = kn[t];
        v[t] = vn[t];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 forward: the same structure with v_mfma_f32_16x16x4_f32 (K = 4 per
// step; lane group g supplies channel 8g+st at step st, for Q and K alike)

template <int M>
__global__ __launch_bounds__(256) void wattn_fwd_f32_kernel(FwdParams p) {
  using S = Win<M>;
  constexpr int NT = S::NT, T = S::T;
  extern __shared__ float s_bias[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int win = xcd_window(blockIdx.x, p.total_windows);
  const int b = win / p.nW, w = win - b * p.nW;
  const int nh = p.nh, C = nh * kHeadDim;
  const float* qkv = static_cast<const float*>(p.qkv);
  float* out = static_cast<float*>(p.out);

  for (int e = tid; e < T * nh; e += blockDim.x) {
    const int idx = e / nh, h = e - idx * nh;
    s_bias[h * T + idx] = p.table[e] * p.inv_scale;
  }
  const bool masked = p.has_mask[w] != 0;
  LaneWindow<M> lw;
  lw.init(p, b, w, g, c, masked);
  __syncthreads();

  for (int h = wave; h < nh; h += nwaves) {
    // V^T through the selector: vt[t][hf][r] = V[16t+4g+r][16hf+c]
    f32x4 vt[NT][2];
    f32x4 kk[NT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = v0, k0 = v0, k1 = v0;
      if (lw.ok[t]) {
        const float* src = qkv + lw.pix[t] * (3LL * C) + h * kHeadDim + 8 * g;
        k0 = *reinterpret_cast<const f32x4*>(src + C);
        k1 = *reinterpret_cast<const f32x4*>(src + C + 4);
        v0 = *reinterpret_cast<const f32x4*>(src + 2 * C);
        v1 = *reinterpret_cast<const f32x4*>(src + 2 * C + 4);
      }
      kk[t][0] = k0;
      kk[t][1] = k1;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          const float sv = (8 * g + st == c + 16 * hf) ? 1.f : 0.f;
          const float vv = st < 4 ? v0[st] : v1[st - 4];
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(vv, sv, acc, 0, 0, 0);
        }
        vt[t][hf] = acc;
      }
    }
    const int hoff = h * T;
#pragma unroll
    for (int it = 0; it < NT; ++it) {
      f32x4 q0 = {0.f, 0.f, 0.f, 0.f}, q1 = q0;
      if (lw.ok[it]) {
        const float* src = qkv + lw.pix[it] * (3LL * C) + h * kHeadDim + 8 * g;
        q0 = *reinterpret_cast<const f32x4*>(src);
        q1 = *reinterpret_cast<const f32x4*>(src + 4);
      }
      f32x4 s[NT];
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) {
        f32x4 acc = lw.score_init(s_bias, hoff, it, jt, g, masked, p.mask_value);
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          const float ka = st < 4 ? kk[jt][0][st] : kk[jt][1][st - 4];
          const float qb = st < 4 ? q0[st] : q1[st - 4];
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka, qb, acc, 0, 0, 0);
        }
        s[jt] = acc;
      }
      const float l = softmax_cols<M>(s, p.score_scale);
      f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = o0;
#pragma unroll
      for (int jt = 0; jt < NT; ++jt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (S::row_empty(jt, r)) continue;
          o0 = __builtin_amdgcn_mfma_f32_16x16x4f32(vt[jt][0][r], s[jt][r], o0, 0, 0, 0);
          o1 = __builtin_amdgcn_mfma_f32_16x16x4f32(vt[jt][1][r], s[jt][r], o1, 0, 0, 0);
        }
      if (lw.ok[it]) {
        const float inv = fast_rcp(l);
        float* dst = out + lw.pix[it] * C + h * kHeadDim + 4 * g;
        *reinterpret_cast<f32x4*>(dst) = o0 * inv;
        *reinterpret_cast<f32x4*>(dst + 16) = o1 * inv;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// setup: relative position index, shift mask, region labels, has-mask flags

__device__ int band_of(int pos, int L, int M, int s) {
  return pos < L - M ? 0 : (pos < L - s ? 1 : 2);
}

__device__ int region_of(int w, int t, int H, int W, int M, int s) {
  if (s == 0) return 0;
  const int nWx = W / M, wy = w / nWx, wx = w - wy * nWx, ty = t / M, tx = t - ty * M;
  return 3 * band_of(wy * M + ty, H, M, s) + band_of(wx * M + tx, W, M, s);
}

__global__ void precompute_kernel(int H, int W, int M, int s, int32_t* rel_index, float* mask,
                                  uint8_t* region, uint8_t* has_mask) {
  const int N = M * M, nW = (H / M) * (W / M);
  const long long total = (long long)nW * N * N;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
    const int j = (int)(e % N);
    const long long rest = e / N;
    const int i = (int)(rest % N), w = (int)(rest / N);
    const int li = region_of(w, i, H, W, M, s), lj = region_of(w, j, H, W, M, s);
    mask[e] = li == lj ? 0.f : -100.f;
    if (w == 0) {
      const int dy = i / M - j / M, dx = i % M - j % M;
      rel_index[i * N + j] = (dy + M - 1) * (2 * M - 1) + (dx + M - 1);
    }
    if (j == 0) region[(long long)w * N + i] = (uint8_t)li;
    if (i == 0 && j == 0) {
      int differ = 0;
      for (int t = 1; t < N; ++t) differ |= region_of(w, t, H, W, M, s) != li;
      has_mask[w] = (uint8_t)differ;
    }
  }
}

template <int M>
hipError_t launch_bf16_m(const FwdParams& p, int waves, hipStream_t st) {
  const size_t lds = (size_t)Win<M>::T * p.nh * sizeof(float);
  hipLaunchKernelGGL(wattn_fwd_bf16_kernel<M>, dim3(p.total_windows), dim3(64 * waves), lds, st, p);
  return hipGetLastError();
}

template <int M>
hipError_t launch_f32_m(const FwdParams& p, int waves, hipStream_t st) {
  const size_t lds = (size_t)Win<M>::T * p.nh * sizeof(float);
  hipLaunchKernelGGL(wattn_fwd_f32_kernel<M>, dim3(p.total_windows), dim3(64 * waves), lds, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_precompute(int H, int W, int M, int s, int32_t* rel_index, float* mask,
                             uint8_t* region, uint8_t* has_mask, hipStream_t stream) {
  const long long total = (long long)(H / M) * (W / M) * M * M * M * M;
  long long blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(precompute_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, H, W, M, s,
                     rel_index, mask, region, has_mask);
  return hipGetLastError();
}

#define SWA_DISPATCH(FN)                                                                      \
  switch (M) {                                                                                \
    case 1: return FN<1>(p, waves, stream);                                                   \
    case 2: return FN<2>(p, waves, stream);                                                   \
    case 3: return FN<3>(p, waves, stream);                                                   \
    case 4: return FN<4>(p, waves, stream);                                                   \
    case 5: return FN<5>(p, waves, stream);                                                   \
    case 6: return FN<6>(p, waves, stream);                                                   \
    case 7: return FN<7>(p, waves, stream);                                                   \
    case 8: return FN<8>(p, waves, stream);                                                   \
    case 9: return FN<9>(p, waves, stream);                                                   \
    case 10: return FN<10>(p, waves, stream);                                                 \
    case 11: return FN<11>(p, waves, stream);                                                 \
    case 12: return FN<12>(p, waves, stream);                                                 \
    default: return hipErrorInvalidValue;                                                     \
  }

hipError_t launch_fwd_bf16(int M, const FwdParams& p, int waves, hipStream_t stream) {
  SWA_DISPATCH(launch_bf16_m)
}

hipError_t launch_fwd_f32(int M, const FwdParams& p, int waves, hipStream_t stream) {
  SWA_DISPATCH(launch_f32_m)
}

}  // namespace swinattn
