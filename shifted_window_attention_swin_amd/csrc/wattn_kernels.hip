// Kernels of libswinattn for gfx950 (MI355X, CDNA4, wave64).
//
// Forward: one workgroup per (image, window); the workgroup's waves take the
// heads round-robin.  For one head a wave holds the whole window in VGPRs:
//
//   Q, K, V   16-token tiles loaded straight from HBM in MFMA operand layout
//             (lane = token, 16 bytes of head_dim each); the cyclic shift and
//             the window partition are the address arithmetic of these loads
//             (talk "Swin Transformer training and inference optimization",
//             uticex.com 1598, section 2: the window ops are index mapping;
//             section 3: transposes folded into the kernel's loads/stores).
//   S^T = K Q^T + C   v_mfma_f32_16x16x32_bf16, K = head_dim = 32 exactly.
//             The accumulator C starts as relative position bias (+ shift
//             mask) divided by the score scale, so one fma later turns D into
//             a base-2 logit.  Transposing S puts one query per lane column:
//             the softmax over keys is in-lane plus two permlane swaps.
//   P^T       exp2 of the logits, rounded to bf16: the C/D layout of S^T is
//             directly the B-operand layout of the next MFMA.
//   O^T = V^T P^T   V^T in operand layout comes from an MFMA of each value
//             tile against a 0/1 selector (an exact transpose in the matrix
//             core); the row sums of P come from one more MFMA against a tile
//             of ones, so the normaliser sums exactly the weights applied.
//   store     lane writes 4 consecutive channels of one token: the window
//             reverse and the roll back are the store addresses.
//
// Token layout inside a window ("quad tiles"): with Q = ceil(M/4) the window
// is padded to (4Q) x (4Q) tokens and cut into Q*Q tiles of 4 rows x 4
// columns; in-tile token u sits at row 4*(t/Q) + u/4, column 4*(t%Q) + u%4.
// In the C/D layout row 4g+r of a key tile (g = lane/16) is then window row
// 4*(t/Q)+g, column 4*(t%Q)+r, so the relative position index
// (dy+M-1)(2M-1) + (dx+M-1) of (query, key) splits into a per-lane part and
// a compile-time part: with the bias table stored reversed in LDS, every bias
// gather is one ds_read with an immediate offset and no address arithmetic.
// Padded keys get -inf in the accumulator (weight exactly 0); padded tokens
// load the window's first token as finite stand-in data (weight 0 times
// finite = 0 in the value product); padded queries are not stored.

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
  int li[S::NT];            // region label of query (t, c)            (masked, select path)
  int lj[S::NT][4];         // region label of key row (t, 4g + r)     (masked, select path)
  bf16x8 mask_a[S::NT];     // key-side mask operand of tile t          (masked, MFMA path)
  bf16x8 mask_b[S::NT];     // query-side mask operand of tile t        (masked, MFMA path)

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

  template <bool MFMA_OPERANDS>
  SWA_INLINE void init_labels(const FwdParams& p, int w, int g, int c) {
    const int wy = w / p.nWx, wx = w - wy * p.nWx;
    if (MFMA_OPERANDS) {
      // Inside one window the region labels take at most four values: the
      // window's rows and columns each meet at most two bands, told apart by
      // "position >= L - shift".  Local label l = 2*[row part] + [column
      // part] is owned by lane group g = l.  A score tile MFMA of these
      // operands adds sum_s [l_key == g] x_s * ([l_query == g] - 1)
      // = -(x_0 + x_1 + x_2) = -100/scale exactly when the labels differ.
#pragma unroll
      for (int t = 0; t < S::NT; ++t) {
        const int ty = 4 * (t / S::Q) + c / 4, tx = 4 * (t % S::Q) + c % 4;
        const int loc = 2 * (wy * M + ty >= p.H - p.shift) + (wx * M + tx >= p.W - p.shift);
        const bool mine = loc == g;
        bf16x8 a = {}, q = {};
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          a[k] = mine ? (__bf16)p.mask_pieces[k] : (__bf16)0.f;
          q[k] = mine ? (__bf16)0.f : (__bf16)-1.f;
        }
        mask_a[t] = a;
        mask_b[t] = q;
      }
      return;
    }
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
// bf16 forward

template <int M>
SWA_INLINE void load_head_bf16(const char* base, const LaneWindow<M>& lw, unsigned Cb,
                               bf16x8 (&q)[Win<M>::NT], bf16x8 (&k)[Win<M>::NT],
                               bf16x8 (&v)[Win<M>::NT]) {
  // tokens outside the window read the window's first token instead (their
  // offsets are clamped): padded keys are -inf in the accumulator, padded
  // values meet weight 0 and padded queries are never stored, so finite
  // stand-in data is as good as zeros and needs no masking
#pragma unroll
  for (int t = 0; t < Win<M>::NT; ++t) {
    const char* src = base + lw.in_off[t];
    q[t] = *reinterpret_cast<const bf16x8*>(src);
    k[t] = *reinterpret_cast<const bf16x8*>(src + Cb);
    v[t] = *reinterpret_cast<const bf16x8*>(src + 2 * Cb);
  }
}

struct HeadCtx {
  const float* s_bias;
  char* out;          // out chunk base
  float score_scale;
  float mask_value;
  bool g_ok;          // lane group is a window row in the last row group
  bf16x8 sel[2];      // selectors of channel halves for the transpose MFMA
  bf16x8 ones;
};

template <int M>
SWA_INLINE void head_bf16(const HeadCtx& hc, const LaneWindow<M>& lw, int h, bool masked,
                          const bf16x8 (&q)[Win<M>::NT], const bf16x8 (&k)[Win<M>::NT],
                          const bf16x8 (&v)[Win<M>::NT]) {
  using S = Win<M>;
  constexpr int NT = S::NT, NK = S::NK;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  // V^T in A-operand layout: slots 0-3 from value tile 2kt, 4-7 from 2kt+1;
  // the selector MFMA gives D[4g+r][c] = V[token (t, 4g+r)][16*hf + c]
  bf16x8 va[2][NK];
#pragma unroll
  for (int kt = 0; kt < NK; ++kt)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const f32x4 d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v[2 * kt], hc.sel[hf], z, 0, 0, 0);
      f32x4 d1 = z;
      if (2 * kt + 1 < NT)
        d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v[2 * kt + 1], hc.sel[hf], z, 0, 0, 0);
      bf16x8 a;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        a[r] = (__bf16)d0[r];
        a[4 + r] = (__bf16)d1[r];
      }
      va[hf][kt] = a;
    }

  const int hbase = h * S::T;
  char* out_h = hc.out + h * kHeadDim * 2;
  // The label compares are the same for every head; hoisted out of the head
  // loop they would need 64-bit lane masks by the dozen.  Redo them per head.
  LaneWindow<M> lwh = lw;
  if (!S::MASK_MFMA) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      asm volatile("" : "+v"(lwh.li[t]));
#pragma unroll
      for (int r = 0; r < 4; ++r) asm volatile("" : "+v"(lwh.lj[t][r]));
    }
  }
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    f32x4 s[NT];
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
      s[jt] = lwh.score_init(hc.s_bias, hbase, it, jt, hc.g_ok, masked && !S::MASK_MFMA,
                             hc.mask_value);
      s[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k[jt], q[it], s[jt], 0, 0, 0);
      if (S::MASK_MFMA && masked)
        s[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lwh.mask_a[jt], lwh.mask_b[it], s[jt], 0, 0, 0);
    }
    softmax_numerators<M>(s, hc.score_scale);
    bf16x8 pb[NK];
#pragma unroll
    for (int kt = 0; kt < NK; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pb[kt][r] = (__bf16)s[2 * kt][r];
        pb[kt][4 + r] = (2 * kt + 1 < NT) ? (__bf16)s[2 * kt + 1][r] : (__bf16)0.f;
      }
    f32x4 o0 = z, o1 = z, l4 = z;
#pragma unroll
    for (int kt = 0; kt < NK; ++kt) {
      o0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[0][kt], pb[kt], o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[1][kt], pb[kt], o1, 0, 0, 0);
      l4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hc.ones, pb[kt], l4, 0, 0, 0);
    }
    if (lw.ok[it]) {
      const float inv = fast_rcp(l4[0]);
      bf16x8 wv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        wv[r] = (__bf16)(o0[r] * inv);
        wv[4 + r] = (__bf16)(o1[r] * inv);
      }
      *reinterpret_cast<bf16x8*>(out_h + lw.out_off[it]) = wv;
    }
    // keep query tiles apart: interleaving them only raises register pressure
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Heads h = wave, wave + nwaves, ...: the first head's tiles are loaded by
// the caller, the others here; latency is hidden by the other resident waves.
template <int M>
SWA_INLINE void run_heads_bf16(const HeadCtx& hc, const LaneWindow<M>& lw, const char* in,
                               unsigned Cb, int nh, int wave, int nwaves, bool masked,
                               bf16x8 (&qa)[Win<M>::NT], bf16x8 (&ka)[Win<M>::NT],
                               bf16x8 (&va)[Win<M>::NT]) {
  for (int h = wave; h < nh; h += nwaves) {
    if (h != wave) load_head_bf16<M>(in + h * kHeadDim * 2, lw, Cb, qa, ka, va);
    head_bf16<M>(hc, lw, h, masked, qa, ka, va);
  }
}

template <int M>
__global__ __launch_bounds__(256) void wattn_fwd_bf16_kernel(FwdParams p) {
  using S = Win<M>;
  constexpr int NT = S::NT;
  extern __shared__ float s_bias[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int win = xcd_window(blockIdx.x, p.total_windows);
  const int b = win / p.nW, w = win - b * p.nW;
  const int nh = p.nh;
  const unsigned Cb = (unsigned)nh * kHeadDim * 2;
  const char* in = static_cast<const char*>(p.qkv);

  stage_bias<M>(s_bias, p.table, nh, p.inv_scale);
  LaneWindow<M> lw;
  lw.init(p, b, w, g, c, 2);
  bf16x8 q[NT], k[NT], v[NT];
  if (wave < nh) load_head_bf16<M>(in + wave * kHeadDim * 2, lw, Cb, q, k, v);

  HeadCtx hc;
  hc.s_bias = s_bias;
  hc.out = static_cast<char*>(p.out);
  hc.score_scale = p.score_scale;
  hc.mask_value = p.mask_value;
  hc.g_ok = g < S::LG;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int s = 0; s < 8; ++s)
      hc.sel[hf][s] = (8 * g + s == out_channel(hf, c)) ? (__bf16)1.f : (__bf16)0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s) hc.ones[s] = (__bf16)1.f;
  __syncthreads();

  const bool masked = window_masked(p.shift, w / p.nWx, w % p.nWx, p.nWy, p.nWx);
  if (masked) lw.template init_labels<S::MASK_MFMA>(p, w, g, c);
  run_heads_bf16<M>(hc, lw, in, Cb, nh, wave, nwaves, masked, q, k, v);
}

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
  if (masked) lw.template init_labels<false>(p, w, g, c);
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
hipError_t launch_bf16_m(const FwdParams& p, int waves, hipStream_t st) {
  hipLaunchKernelGGL(wattn_fwd_bf16_kernel<M>, dim3(p.total_windows), dim3(64 * waves),
                     lds_bytes<M>(p.nh), st, p);
  return hipGetLastError();
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

hipError_t launch_fwd_bf16(int M, const FwdParams& p, int waves, hipStream_t stream) {
  SWA_DISPATCH(launch_bf16_m)
}

hipError_t launch_fwd_f32(int M, const FwdParams& p, int waves, hipStream_t stream) {
  SWA_DISPATCH(launch_f32_m)
}

}  // namespace swinattn
