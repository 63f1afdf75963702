// Layer norm + QKV projection + shifted-window attention in one pass
// (gfx950): the attention half of a Swin block before its output projection,
// reading the raw token rows x and writing the attention output, with q, k
// and v never leaving the chip.
//
// The NVIDIA talk "Swin Transformer training and inference optimization"
// (uticex.com 1598), section 3, fuses the layer norm with the window shift
// and partition, fuses the QKV GEMM with its bias and prepares its weight in
// a format that suits the fused attention; here all of these run in the
// attention's own workgroups.  Per window and head:
//
//   xn  = layer norm of each token row of x (over its C channels)
//   qkv = xn W^T + b        (3 x 32 channels of the head)
//   out = softmax(q k^T / sqrt(d) + bias + mask) v   (as swin_wattn_fwd)
//
// The layer norm folds into the packed weight as in swin_ln_linear_fwd:
// y_j = (sum_c x_c W'_jc - mean s_j) / sigma + b'_j, so the products run on
// the raw rows and each token needs only its mean and 1/sigma.
//
//   workgroup  persistent, fixed on one head for the launch, its q, k and v
//              weight blocks (32 channels x C each, MFMA A operands) held in
//              registers for the whole launch.  C <= 96: 4 waves, waves 0-2
//              holding one 32-channel block each and wave 3 taking the
//              token statistics.  C >= 128: 8 waves, waves 0-5 holding one
//              16-channel tile each (half the weight registers, so that two
//              workgroups of 8 waves fit per CU instead of two of 4) and
//              waves 6-7 taking the statistics, two lanes per token.
//              The nh head workgroups of a stream of windows sit on one XCD
//              and walk the same windows in the same order, so a window's x
//              rows come from HBM once and from that XCD's L2 for the other
//              heads.
//   window     the x rows of its 64 padded quad-tile tokens (49 at window 7)
//              are staged in LDS as 1 KB blocks (16 tokens x 32 channels),
//              the next window's rows waiting in registers; the weight
//              waves form D = W' x^T for q, k and v (the head's 96
//              channels), the statistics waves the mean and 1/sigma of
//              every token; then the folded epilogue writes q, k, v in bf16
//              into LDS in the attention's tile layout and waves 0-3 run
//              the attention of one query tile each (the math of
//              wattn_persistent.hip: bias and mask in the accumulator, exp2
//              softmax across lanes, V^T from transposing reads, the
//              normaliser from an MFMA against ones).  4 waves: one window
//              at a time.  8 waves: two windows in flight, the attention of
//              window i - 1 beside the v products and statistics of window
//              i (see the main loop).
//   output     each lane stores 8 channels (16 bytes) of its query token;
//              the two 64-byte halves of a token's line come from the
//              workgroups of two heads on the same XCD and meet in its L2.

#include <atomic>
#include <type_traits>

#include "ln_attn_internal.h"
#include "wattn_common.h"

namespace swinattn {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kLaBlock = 1024;  // 16 tokens x 64 bytes

// waves per workgroup: 8 from 4 k-steps (C >= 128) on, see above
template <int KS>
constexpr int la_waves() {
  return KS >= 4 ? 8 : 4;
}

template <int M, int KS>
struct LaLds {
  using S = Win<M>;
  static constexpr int NT = S::NT;                          // token tiles (4)
  static constexpr int BIAS = ((S::T + S::TAIL) * 4 + 15) / 16 * 16;
  static constexpr int CST = 2 * 96 * 4;                    // s_j and b'_j of the head's channels
  static constexpr int STAT = 16 * NT * 8;                  // (mean, 1/sigma) per token
  static constexpr int OFF_CST = BIAS;
  static constexpr int OFF_STAT = OFF_CST + CST;
  static constexpr int OFF_X = OFF_STAT + STAT;             // NT * KS blocks of x, two
                                                            // windows' with 8 waves
  static constexpr int XBUF = la_waves<KS>() == 8 ? 2 : 1;
  static constexpr int OFF_UNIT = OFF_X + XBUF * NT * KS * kLaBlock;  // q, k, v tiles
  static constexpr int OFF_MASK = OFF_UNIT + 3 * NT * kLaBlock;
  static constexpr int BYTES = OFF_MASK + NT * kLaBlock;
};

// Window coordinates (row, column) of in-tile token u of tile t.
template <int M>
SWA_INLINE void la_token(int t, int u, int& ty, int& tx) {
  ty = 4 * (t / Win<M>::Q) + u / 4;
  tx = 4 * (t % Win<M>::Q) + u % 4;
}

// Flattened image position (within the launch) of window token (ty, tx);
// tokens outside the window stand in for the window's first token.
SWA_INLINE unsigned la_pixel(const LnAttnParams& p, int M, int b, int wy, int wx, int ty, int tx,
                             bool ok) {
  int y = wy * M + (ok ? ty : 0) + p.shift, x = wx * M + (ok ? tx : 0) + p.shift;
  y -= y >= p.H ? p.H : 0;
  x -= x >= p.W ? p.W : 0;
  return ((unsigned)b * p.H + y) * p.W + x;
}

// waves per SIMD the registers must leave room for (the second launch
// bound): 4-wave workgroups, 3 (three per CU) while the weight blocks (8 KS
// VGPRs) and the next window's rows (4 KS) leave the attention enough
// registers; 8-wave workgroups, 4 (two per CU, at most 128 VGPRs)
template <int KS>
constexpr int la_min_waves() {
  return la_waves<KS>() == 8 ? 4 : 3;
}

template <int M, int KS>
__global__ __launch_bounds__(la_waves<KS>() * 64, la_min_waves<KS>()) void ln_qkv_wattn_kernel(LnAttnParams p) {
  using S = Win<M>;
  using L = LaLds<M, KS>;
  constexpr int NT = S::NT, NK = S::NK, T = S::T;
  static_assert(NT == 4, "windows of 5 to 8 tokens a side: 4 token tiles");
  constexpr int kLaWaves = la_waves<KS>();
  constexpr bool W8 = kLaWaves == 8;
  // waves computing the products (0 .. kGemm-1) and the statistics (the rest)
  constexpr int kGemm = W8 ? 6 : 3;
  constexpr int XB = NT * KS;                                  // x blocks of a window
  constexpr int XPW = (XB + kLaWaves - 1) / kLaWaves;          // x blocks loaded per wave
  constexpr int C = KS * 32;
  extern __shared__ char s_lds[];
  float* s_bias = reinterpret_cast<float*>(s_lds);
  float* s_cst = reinterpret_cast<float*>(s_lds + L::OFF_CST);    // [s | b'][96]
  float2* s_stat = reinterpret_cast<float2*>(s_lds + L::OFF_STAT);
  char* s_x = s_lds + L::OFF_X;
  char* s_unit = s_lds + L::OFF_UNIT;
  char* s_mask = s_lds + L::OFF_MASK;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wv >= 0 && wv < kLaWaves);
  const int gq = lane & 3, cq = lane >> 2;  // load layout: 16-byte part, token
  const int g = lane >> 4, c = lane & 15;   // MFMA layout: lane group, token
  // byte offset of 16-byte part `part` of in-tile token u in a 1 KB block:
  // the part is XORed with bits 1-2 of the token (bank-conflict-free reads
  // of tokens 4 apart)
  auto uchunk = [](int u, int part) { return 64 * u + 16 * (part ^ ((u >> 1) & 3)); };
  const int nh = p.nh;
  const char* xb = static_cast<const char*>(p.x);
  char* outb = static_cast<char*>(p.out);
  const unsigned xrow = (unsigned)C * 2;       // bytes of one x (and out) row

  // workgroup -> (head, stream): with 8 streams or more the nh heads of
  // stream 8 (k / nh) + (id & 7) are slots k of XCD id & 7 (workgroups are
  // dealt to XCDs round-robin); fewer streams take consecutive ids
  const int id = blockIdx.x, streams = p.streams;
  int h, stream;
  if (streams % 8 == 0) {
    const int k8 = id >> 3;
    h = k8 % nh;
    stream = (k8 / nh) * 8 + (id & 7);
  } else {
    h = id % nh;
    stream = id / nh;
  }

  // bias table of the head (reversed, divided by the scale) and the folded
  // layer-norm constants of its 96 output channels: s_j, then b'_j
  for (int e = tid; e < T + S::TAIL; e += kLaWaves * 64)
    s_bias[e] = e < T ? p.table[(T - 1 - e) * nh + h] * p.inv_scale : 0.f;
  for (int e = tid; e < 2 * 96; e += kLaWaves * 64) {
    const int half = e / 96, r = e - half * 96;           // r = slice * 32 + channel
    const int ch = (r / 32) * C + h * 32 + (r % 32);      // output channel of the QKV row
    s_cst[e] = p.consts[half * p.N + ch];
  }
  // the wave's weights: slice sl (q, k, v) of head h, column block
  // sl * nh + h of the packed weight, both of its 16-row tiles (4 waves) or
  // tile ti (8 waves: tile ti of a block carries channels 8 j + 4 ti + r,
  // j = 0..3, r = 0..3); the statistics waves hold none
  constexpr int NTI = W8 ? 1 : 2;  // weight tiles per wave
  const int sl = W8 ? wv >> 1 : wv, ti = W8 ? wv & 1 : 0;
  bf16x8 a[KS][NTI];
  if (wv < kGemm) {
    const char* wcb = static_cast<const char*>(p.wp) + (size_t)(sl * nh + h) * KS * 2048 + lane * 16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < NTI; ++i) a[ks][i] = *reinterpret_cast<const bf16x8*>(wcb + (ks * 2 + ti + i) * 1024);
  }

  struct Pos {
    int b, wy, wx;
  };
  auto decode = [&](int bw) {
    Pos q;
    q.b = bw / p.nW;
    const int w = bw - q.b * p.nW;
    q.wy = w / p.nWx;
    q.wx = w - q.wy * p.nWx;
    return q;
  };
  // x rows of a window: block xi = tile * KS + k-step, wave wv loads blocks
  // wv, wv + 4, ...; one token address per lane
  using Regs = u32x4[XPW];
  auto issue = [&](Regs& R, const Pos& q) {
#pragma unroll
    for (int k = 0; k < XPW; ++k) {
      const int xi = wv + kLaWaves * k;
      if (xi < XB) {
        const int t = xi / KS, ks = xi - t * KS;
        int ty, tx;
        la_token<M>(t, cq, ty, tx);
        const bool ok = ty < M && tx < M;
        const unsigned pix = la_pixel(p, M, q.b, q.wy, q.wx, ty, tx, ok);
        R[k] = *reinterpret_cast<const u32x4*>(xb + pix * xrow + ks * 64 + 16 * gq);
      }
    }
  };
  auto write = [&](const Regs& R, char* sx) {
#pragma unroll
    for (int k = 0; k < XPW; ++k) {
      const int xi = wv + kLaWaves * k;
      if (xi < XB) *reinterpret_cast<u32x4*>(sx + xi * kLaBlock + uchunk(cq, gq)) = R[k];
    }
  };
  // key-side shift-mask operands of a masked window (see wattn_persistent.hip)
  auto write_mask = [&](const Pos& q, int t0, int t1) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < t0 || t >= t1) continue;
      int ty, tx;
      la_token<M>(t, c, ty, tx);
      const int loc = 2 * (q.wy * M + ty >= p.H - p.shift) + (q.wx * M + tx >= p.W - p.shift);
      bf16x8 m = {};
#pragma unroll
      for (int j = 0; j < 3; ++j) m[j] = loc == g ? (__bf16)p.mask_pieces[j] : (__bf16)0.f;
      *reinterpret_cast<bf16x8*>(s_mask + t * kLaBlock + lane * 16) = m;
    }
  };

  // (mean, 1/sigma) of every token of the window, one lane per token: the
  // sum and the sum of squares from bf16 dot products (each product exact in
  // fp32), K var = S2 - S1 mean; where that difference would lose more than
  // 8 bits to cancellation (rows whose mean is large against their spread)
  // the wave takes the mean of the squared deviations from the mean in a
  // second pass, as the definition reads
  // 4 waves: wave 3, one lane per token.  8 waves: waves 6 and 7, tokens
  // 32 (wv - 6) .. + 31, two lanes per token (lane and lane + 32), each
  // summing half of the row's 16-byte chunks; the halves are added with a
  // swap of the wave's two 32-lane halves
  auto ln_stats = [&](const char* sx) {
    constexpr float kInvK = 1.f / C;
    constexpr int QH = W8 ? 2 * KS : 4 * KS;  // chunks a lane sums
    const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
    const int t = W8 ? (wv - kGemm) * 32 + (lane & 31) : lane;  // 16 NT = 64 tokens
    const int q0 = W8 ? (lane >> 5) * QH : 0;
    const char* tile = sx + (t >> 4) * KS * kLaBlock;
    auto chunk = [&](int q) {  // chunk q of the row: k-step q / 4, part q % 4
      return *reinterpret_cast<const bf16x8*>(tile + (q >> 2) * kLaBlock + uchunk(t & 15, q & 3));
    };
    auto both_halves = [&](float x) {
      if constexpr (W8) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
      return x;
    };
    // a few chunks at a time: the row's chunks are not held
    float s1 = 0.f, s2 = 0.f;
#pragma unroll 4
    for (int q = 0; q < QH; ++q) {
      const bf16x8 hv = chunk(q0 + q);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2 pr = {hv[2 * e], hv[2 * e + 1]};
        s1 = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, s1, false);
        s2 = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, s2, false);
      }
    }
    s1 = both_halves(s1);
    s2 = both_halves(s2);
    const float mu = s1 * kInvK;
    float kvar = fmaxf(s2 - s1 * mu, 0.f);
    if (__builtin_amdgcn_ballot_w64(kvar < s2 * (1.f / 256.f)) != 0) {  // wave-uniform
      float d2 = 0.f;
#pragma unroll 4
      for (int q = 0; q < QH; ++q) {
        const bf16x8 hv = chunk(q0 + q);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = (float)hv[e] - mu;
          d2 = fmaf(d, d, d2);
        }
      }
      kvar = both_halves(d2);
    }
    if (!W8 || lane < 32) s_stat[t] = make_float2(mu, rsqrtf(kvar * kInvK + p.eps));
  };

  const bool g_ok = g < S::LG;  // lane group is a window row in the last row group
  bf16x8 ones;
#pragma unroll
  for (int s = 0; s < 8; ++s) ones[s] = (__bf16)1.f;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};

  // attention of query tile it of the window (one head, tiles in LDS)
  auto attend = [&](const Pos& pos, int it) {
    const bool masked = window_masked(p.shift, pos.wy, pos.wx, p.nWy, p.nWx);
    auto block = [&](int sl, int t) { return s_unit + (sl * NT + t) * kLaBlock; };
    const bf16x8 q = *reinterpret_cast<const bf16x8*>(block(0, it) + uchunk(c, g));
    int ty, tx;
    la_token<M>(it, c, ty, tx);
    const bool ok = ty < M && tx < M;
    const int qbase = T - 1 - S::C0 - (ok ? S::D * ty + tx : 0) + S::D * g;
    bf16x8 mask_b = {};
    if (masked) {
      const int loc = 2 * (pos.wy * M + ty >= p.H - p.shift) + (pos.wx * M + tx >= p.W - p.shift);
#pragma unroll
      for (int k = 0; k < 3; ++k) mask_b[k] = loc == g ? (__bf16)0.f : (__bf16)-1.f;
    }
    f32x4 sc[NT];
    auto score_tiles = [&](auto masked_c) {
      constexpr bool MASKED = decltype(masked_c)::value;
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) {
        f32x4 acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (!S::col_ok(jt, r)) {
            acc[r] = -__builtin_inff();
            continue;
          }
          float v = s_bias[qbase + S::E(jt) + r];
          if (!S::rows_all(jt)) v = g_ok ? v : -__builtin_inff();
          acc[r] = v;
        }
        const bf16x8 kj = *reinterpret_cast<const bf16x8*>(block(1, jt) + uchunk(c, g));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kj, q, acc, 0, 0, 0);
        if constexpr (MASKED) {
          const bf16x8 mj = *reinterpret_cast<const bf16x8*>(s_mask + jt * kLaBlock + lane * 16);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mj, mask_b, acc, 0, 0, 0);
        }
        sc[jt] = acc;
      }
    };
    if (masked) score_tiles(std::true_type{});
    else score_tiles(std::false_type{});
    softmax_numerators<M>(sc, p.score_scale);
    bf16x8 pb[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pb[kk][r] = (__bf16)sc[2 * kk][r];
        pb[kk][4 + r] = (2 * kk + 1 < NT) ? (__bf16)sc[2 * kk + 1][r] : (__bf16)0.f;
      }
    // V^T: transposing reads of the value tiles (lane i of a group of 16
    // receives element i % 4 of the 8-byte chunks read by lanes i / 4 + 4k)
    f32x4 o0 = z, o1 = z, l4 = z;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const int t1 = 2 * kk + 1 < NT ? 2 * kk + 1 : 2 * kk;
      bf16x8 v[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int own = uchunk(lane >> 2, lane & 3) + 8 * hf;
        const bf16x4 lo = lds_read_tr(block(2, 2 * kk) + own);
        const bf16x4 hi = lds_read_tr(block(2, t1) + own);
        v[hf] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      o0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v[0], pb[kk], o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v[1], pb[kk], o1, 0, 0, 0);
      l4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[kk], l4, 0, 0, 0);
    }
    if (ok) {
      const float inv = fast_rcp(l4[0]);
      bf16x8 ov;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ov[r] = (__bf16)(o0[r] * inv);
        ov[4 + r] = (__bf16)(o1[r] * inv);
      }
      const unsigned pix = la_pixel(p, M, pos.b, pos.wy, pos.wx, ty, tx, true);
      *reinterpret_cast<bf16x8*>(outb + pix * xrow + h * 64 + 16 * g) = ov;
    }
  };

  // D = W'_tiles x^T of the window in sx: rows output channels, columns
  // the window's tokens
  auto gemm = [&](const char* sx, f32x4 (&acc)[NT][NTI]) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < NTI; ++i) acc[t][i] = z;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8 xv = *reinterpret_cast<const bf16x8*>(sx + (t * KS + ks) * kLaBlock + uchunk(c, g));
#pragma unroll
        for (int i = 0; i < NTI; ++i)
          acc[t][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks][i], xv, acc[t][i], 0, 0, 0);
      }
    }
  };
  // folded layer norm and bias: lane (g, c) holds channels 8g + 4 i + r
  // (weight tile i, r = 0..3) of slice sl for token c of every tile; bf16
  // q, k or v into the tile, 8 bytes per weight tile
  auto epilogue = [&](const f32x4 (&acc)[NT][NTI]) {
    const float* cs = s_cst + sl * 32 + 8 * g + 4 * ti;
    f32x4 sv[NTI], bv[NTI];
#pragma unroll
    for (int i = 0; i < NTI; ++i) {
      sv[i] = *reinterpret_cast<const f32x4*>(cs + 4 * i);
      bv[i] = *reinterpret_cast<const f32x4*>(cs + 4 * i + 96);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float2 st = s_stat[t * 16 + c];
      char* dst = s_unit + (sl * NT + t) * kLaBlock + uchunk(c, g) + 8 * ti;
      if constexpr (W8) {
        bf16x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = (__bf16)fmaf(fmaf(-st.x, sv[0][r], acc[t][0][r]), st.y, bv[0][r]);
        *reinterpret_cast<bf16x4*>(dst) = o;
      } else {
        bf16x8 o;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            o[4 * i + r] = (__bf16)fmaf(fmaf(-st.x, sv[i][r], acc[t][i][r]), st.y, bv[i][r]);
        *reinterpret_cast<bf16x8*>(dst) = o;
      }
    }
  };

  Regs R;
  int w = stream;
  if (w < p.windows) issue(R, decode(w));
  __syncthreads();  // tables and constants staged
  if constexpr (!W8) {
    // one window at a time: products and statistics, epilogue, attention
    for (; w < p.windows; w += streams) {
      const Pos cur = decode(w);
      write(R, s_x);
      __syncthreads();  // x rows of the window visible
      if (w + streams < p.windows) {
        // the loads leave ahead of the other workgroups' math on the SIMD
        __builtin_amdgcn_s_setprio(3);
        issue(R, decode(w + streams));
        __builtin_amdgcn_s_setprio(0);
      }
      f32x4 acc[NT][NTI];
      if (wv < kGemm) {
        gemm(s_x, acc);
      } else {
        ln_stats(s_x);
        if (window_masked(p.shift, cur.wy, cur.wx, p.nWy, p.nWx)) write_mask(cur, 0, NT);
      }
      __syncthreads();  // token statistics and mask operands visible
      if (wv < kGemm) epilogue(acc);
      __syncthreads();  // q, k, v of the window visible
      if (wv < NT) attend(cur, wv);
      // the x tile is rewritten only after every wave has passed the second
      // barrier above; the q, k, v tiles, statistics and mask operands only
      // after the next window's first barrier, which every wave reaches
      // after its attention
    }
  } else {
    // two windows in flight: while waves 0-3 run the attention of window
    // i - 1, waves 4-5 form v of window i and waves 6-7 its statistics;
    // then waves 0-3 form q and k of window i (and waves 4-7 finish v and
    // the mask operands).  The x rows of consecutive windows alternate
    // between two buffers, so the rows of window i + 1 are written while
    // waves 0-3 still read those of window i.
    Pos prev = decode(w);
    bool have_prev = false;
    for (int it = 0; w < p.windows; w += streams, ++it) {
      const Pos cur = decode(w);
      char* sx = s_x + (it & 1) * XB * kLaBlock;
      write(R, sx);
      // x rows of window i visible; q, k, v and mask operands of window
      // i - 1 visible
      __syncthreads();
      if (w + streams < p.windows) {
        __builtin_amdgcn_s_setprio(3);
        issue(R, decode(w + streams));
        __builtin_amdgcn_s_setprio(0);
      }
      f32x4 acc[NT][NTI];
      if (wv < NT) {
        if (have_prev) attend(prev, wv);
      } else if (wv < kGemm) {
        gemm(sx, acc);
      } else {
        ln_stats(sx);
      }
      // statistics of window i visible; the attention of window i - 1 is
      // done with the q, k, v tiles and the mask operands
      __syncthreads();
      if (wv < NT) {
        gemm(sx, acc);
        epilogue(acc);
      } else if (wv < kGemm) {
        epilogue(acc);
      } else if (window_masked(p.shift, cur.wy, cur.wx, p.nWy, p.nWx)) {
        write_mask(cur, 2 * (wv - kGemm), 2 * (wv - kGemm) + 2);
      }
      prev = cur;
      have_prev = true;
    }
    if (have_prev) {
      __syncthreads();  // q, k, v and mask operands of the last window visible
      if (wv < NT) attend(prev, wv);
    }
  }
}

template <int M, int KS>
int la_blocks_per_cu(int dev) {
  static std::atomic<int> cache[kMaxDevices];
  const bool cacheable = dev >= 0 && dev < kMaxDevices;
  if (cacheable) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ln_qkv_wattn_kernel<M, KS>,
                                                   la_waves<KS>() * 64, LaLds<M, KS>::BYTES) !=
          hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  if (cacheable) cache[dev].store(per_cu, std::memory_order_relaxed);
  return per_cu;
}

// Grid: streams of windows x heads, a multiple of 8 nh (each XCD holds
// whole streams) when the chip holds that many, at the kernel's occupancy,
// and at most one stream per window.
template <int M, int KS>
hipError_t launch_la(const LnAttnParams& p_in, int dev, int cus, hipStream_t st) {
  LnAttnParams p = p_in;
  const long long slots = (long long)cus * la_blocks_per_cu<M, KS>(dev);
  long long streams = slots / p.nh;
  if (streams > p.windows) streams = p.windows;
  if (streams >= 8) streams -= streams % 8;
  if (streams < 1) streams = 1;
  p.streams = (int)streams;
  const long long grid = streams * p.nh;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((ln_qkv_wattn_kernel<M, KS>), dim3((unsigned)grid), dim3(la_waves<KS>() * 64),
                     (LaLds<M, KS>::BYTES), st, p);
  return hipGetLastError();
}

template <int M>
hipError_t launch_la_m(const LnAttnParams& p, int dev, int cus, hipStream_t st) {
  switch (p.C / 32) {
    case 1: return launch_la<M, 1>(p, dev, cus, st);
    case 2: return launch_la<M, 2>(p, dev, cus, st);
    case 3: return launch_la<M, 3>(p, dev, cus, st);
    case 4: return launch_la<M, 4>(p, dev, cus, st);
    case 5: return launch_la<M, 5>(p, dev, cus, st);
    case 6: return launch_la<M, 6>(p, dev, cus, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_ln_qkv_wattn(int M, const LnAttnParams& p, int dev, int cus,
                               hipStream_t stream) {
  switch (M) {
    case 5: return launch_la_m<5>(p, dev, cus, stream);
    case 6: return launch_la_m<6>(p, dev, cus, stream);
    case 7: return launch_la_m<7>(p, dev, cus, stream);
    case 8: return launch_la_m<8>(p, dev, cus, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace swinattn
