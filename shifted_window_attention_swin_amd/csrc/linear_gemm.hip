// Linear layer with bias and optional residual, the operations on either side
// of the window attention (gfx950):
//
//   y[t][j] = sum_c x[t][c] * W[j][c] + bias[j]  (+ residual[t][j])
//
//  - QKV GEMM + bias: K = C, N = 3C.  The output token row is [3][heads][d],
//    the qkv row the attention kernel reads.  The NVIDIA talk "Swin
//    Transformer training and inference optimization" (uticex.com 1598),
//    section 3, fuses the QKV GEMM with its bias and transforms the weight
//    into a kernel-friendly format ahead of time; here that format is the
//    MFMA operand order of swin_linear_pack_weight.
//  - Output projection + bias + residual: K = N = C (same section: the kernel
//    that adds a bias, then the residual).
//
// At Swin sizes K = C is small (96..384), so the layer moves more bytes than
// it does arithmetic per byte (Swin-L stage 1 QKV: 144 FLOP/B against a bf16
// ridge of about 310): the kernel is built to stream x and y at HBM speed.
//
//   row block  32 tokens x K, staged in LDS as 1 KB blocks of 16 tokens x 64
//              bytes (32 input channels, the 16-byte parts of a token
//              permuted so that the MFMA B operand reads are free of bank
//              conflicts); the next block waits in registers.
//   workgroup  6, 4 or 2 waves (the widest that divides N / 32), persistent,
//              owning one column group (a 32-channel block per wave: whole
//              128-byte lines of every token) for the whole launch and
//              walking row blocks;
//              the column groups of a row block run side by side on one XCD,
//              so x comes from HBM once and from that XCD's L2 after.
//   weight     packed once: column block cb, k-step ks, tile i is one 1 KB
//              MFMA A operand.  Each wave loads its block's tiles into
//              registers once and keeps them.
//   product    D = W_tile * x^T: D rows are output channels, columns tokens.
//              Row m of packed tile i carries channel out_channel(i, m), so a
//              lane ends with 8 consecutive channels of one token.
//   epilogue   the fp32 products go through an LDS tile so that every store
//              instruction writes whole lines (8 tokens x 128 bytes): + bias,
//              + residual (read as whole lines too), round to bf16,
//              non-temporal 16-byte stores.  Halves of a line written by
//              different waves cost a quarter more HBM write traffic.
//
// INT8 (same talk, section 3, INT8 quantization: input and weight in INT8,
// products accumulated in INT32, the sums dequantized, bias and residual in
// floating point; the INT8-output form quantizes the result again).  The
// v_mfma_i32_16x16x64_i8 operands hold 16 bytes per lane at the byte
// positions of the bf16 16x16x32 operands, so the kernel moves the same
// bytes: a 64-byte k-step is 64 int8 input channels (K = 96 ends in half a
// step: those lanes take zeros, and the packed weight is zero there).  The
// int32 sums are converted to fp32 in the product layout: times x_scale *
// w_scale[j], then bias (and residual) as above, rounded to bf16; or, for
// INT8 output, the code clamp(rne(fma(sum, a_j, b_j)), -127, 127) with
// a_j = x_scale * w_scale[j] / out_scale[j], b_j = bias[j] / out_scale[j].

#include <atomic>
#include <type_traits>

#include "linear_internal.h"
#include "wattn_common.h"

namespace swinattn {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kLinRows = 32;               // tokens per row block: 2 tiles of 16
constexpr int kLinTiles = kLinRows / 16;
// bytes per token of the fp32 output tile of a WAVES-wave workgroup (padded)
constexpr int lin_out_stride(int waves) { return waves * 32 * 4 + 16; }

// epilogue / prologue of the linear kernel: bf16 x and weight (0-2); int8
// x and weight with bf16 output (3, 4) or int8 output (5)
enum LinMode {
  kLinPlain = 0,
  kLinResidual = 1,
  kLinLayerNorm = 2,
  kLinI8 = 3,
  kLinI8Residual = 4,
  kLinI8Out = 5
};
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// sum over aligned groups of L = 4 or 8 lanes (DPP: lane ^ 1, lane ^ 2
// within quads, then the mirror of each half row pairs the two quads)
template <int L>
SWA_INLINE float group_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
  if constexpr (L == 8)
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));
  return v;
}

// LDS of the layer norm, after the x and output tiles: (mean, 1/sigma) of
// the row block's tokens
constexpr size_t lin_ln_lds_bytes() { return kLinRows * 8; }

// WAVES waves per workgroup, one 32-column block each: with an even WAVES
// the workgroup's WAVES * 32 channels are WAVES / 2 whole 128-byte lines of
// every bf16 token.
// MODE kLinResidual adds a residual; kLinLayerNorm normalises every token
// row of x (over its K channels) before the product.
template <int KS, int MODE, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void linear_fwd_kernel(LinearParams p) {
  constexpr bool RES = MODE == kLinResidual || MODE == kLinI8Residual, LN = MODE == kLinLayerNorm;
  constexpr bool I8 = MODE >= kLinI8, I8OUT = MODE == kLinI8Out;
  constexpr int kLinWaves = WAVES;
  constexpr int kLinCols = 32 * WAVES;
  constexpr int kOutStride = lin_out_stride(WAVES);
  constexpr int kOut8Stride = kLinCols + 16;  // bytes per token of the int8 output tile
  constexpr int NB = kLinTiles * KS;                      // LDS blocks per row block
  constexpr int BPW = (NB + kLinWaves - 1) / kLinWaves;   // blocks loaded per wave
  constexpr int CPT = kLinCols / 8;                       // 16-byte chunks per token
  extern __shared__ char s_lds[];
  char* s_x = s_lds;              // NB blocks of 1 KB: the row block of x
  char* s_o = s_lds + NB * 1024;  // kLinRows x kOutStride: the fp32 output tile
  float2* s_stat = reinterpret_cast<float2*>(s_o + kLinRows * kOutStride);  // layer norm

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wv >= 0 && wv < kLinWaves);
  const int T = (int)p.T;                   // the host keeps T below 2^31
  const int gq = lane & 3, cq = lane >> 2;  // load layout: 16-byte part, token
  const int g = lane >> 4, c = lane & 15;   // MFMA layout: lane group, token
  // byte offset of 16-byte part `part` of token u in a 1 KB block of x: the
  // part is XORed with bits 1-2 of the token, so that the tokens 4 apart
  // that a lane group reads together sit in different banks
  auto uchunk = [](int u, int part) { return 64 * u + 16 * (part ^ ((u >> 1) & 3)); };
  const char* xb = static_cast<const char*>(p.x);
  const char* rb = static_cast<const char*>(p.res);
  char* yb = static_cast<char*>(p.y);
  const size_t xrow = I8 ? (size_t)p.K : (size_t)KS * 64;  // bytes of one x row
  const size_t yrow = (size_t)p.N * 2;      // bytes of one bf16 y (residual) row

  // This workgroup's column group and row blocks.  The grid is a multiple
  // of the column-group count, so a workgroup keeps one column group for the
  // whole launch.  When the grid also covers the 8 XCDs evenly, each XCD
  // owns a contiguous range of row blocks and the column groups of a row
  // block run side by side on one XCD: x is fetched into its L2 once.
  const int G = gridDim.x, id = blockIdx.x, ncg = p.ncg;
  int cg, r, step, r_end;
  if (G % (8 * ncg) == 0) {
    const int x = id & 7, j = id >> 3, per = G >> 3;
    cg = j % ncg;
    step = per / ncg;
    r = (int)((long long)p.blocks * x / 8) + j / ncg;
    r_end = (int)((long long)p.blocks * (x + 1) / 8);
  } else {
    cg = id % ncg;
    step = G / ncg;
    r = id / ncg;
    r_end = p.blocks;
  }
  const int cb = cg * kLinWaves + wv;  // this wave's column block (product phase)
  const bool active = cb < p.ncb;
  // store phase: the output tile is kLinRows * CPT chunks of 16 bytes (8
  // channels); wave wv stores chunks 128 wv + 64 j + lane, j = 0, 1, in
  // token-major order, so consecutive lanes cover whole lines of a token.
  // int8 output: chunks of 16 channels (16 bytes), chunk 64 wv + lane
  int srow[2], sch[2];
  bool s_active[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if constexpr (I8OUT) {
      const int q = 64 * wv + lane;
      srow[j] = q / (kLinCols / 16);
      sch[j] = cg * kLinCols + 16 * (q - srow[j] * (kLinCols / 16));
      s_active[j] = j == 0 && sch[j] < p.N;
      continue;
    }
    const int q = 128 * wv + 64 * j + lane;
    srow[j] = q / CPT;
    sch[j] = cg * kLinCols + 8 * (q - srow[j] * CPT);
    s_active[j] = sch[j] < p.N;
  }

  // the wave's weight tiles stay in registers for the whole launch
  using AOp = std::conditional_t<I8, i32x4, bf16x8>;
  AOp a[KS][2];
  if (active) {
    const char* wcb = static_cast<const char*>(p.wp) + (size_t)cb * KS * 2048 + lane * 16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      a[ks][0] = *reinterpret_cast<const AOp*>(wcb + (ks * 2) * 1024);
      a[ks][1] = *reinterpret_cast<const AOp*>(wcb + (ks * 2 + 1) * 1024);
    }
  }
  // the bias of the lane's 8 channels in each store slot j (zero without a
  // bias); held for the launch, except with the layer norm (below)
  auto load_bias = [&](f32x4 (&bv)[2][2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bv[j][0] = bv[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (s_active[j] && p.bias) {
        bv[j][0] = *reinterpret_cast<const f32x4*>(p.bias + sch[j]);
        bv[j][1] = *reinterpret_cast<const f32x4*>(p.bias + sch[j] + 4);
      }
    }
  };
  f32x4 bias[2][2];
  if constexpr (!LN && !I8OUT) load_bias(bias);
  // int8: the dequantization constants of the 8 channels 8g + 4i + r of the
  // wave's column block that lane (g, c) holds in the product layout:
  // kq = x_scale * w_scale (bf16 output), or kq = x_scale * w_scale /
  // out_scale and kb = bias / out_scale (int8 output)
  f32x4 kq[I8 ? 2 : 1], kb[I8OUT ? 2 : 1];
  if constexpr (I8) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      kq[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (I8OUT) kb[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int ch = cb * 32 + 8 * g + 4 * i;
      if (active && ch < p.N) {
        const f32x4 sw = *reinterpret_cast<const f32x4*>(p.w_scale + ch);
#pragma unroll
        for (int q = 0; q < 4; ++q) kq[i][q] = p.x_scale * sw[q];
        if constexpr (I8OUT) {
          const f32x4 so = *reinterpret_cast<const f32x4*>(p.out_scale + ch);
          f32x4 bi = f32x4{0.f, 0.f, 0.f, 0.f};
          if (p.bias) bi = *reinterpret_cast<const f32x4*>(p.bias + ch);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            kq[i][q] = kq[i][q] / so[q];  // correctly rounded fp32 division
            kb[i][q] = bi[q] / so[q];
          }
        }
      }
    }
  }
  // layer norm: the folded bias b'_j and row sum s_j of the 8 channels
  // 8g + 4i + r (i = 0, 1, r = 0..3) of the wave's column block that lane
  // (g, c) holds in the product layout, for the launch.  The epilogue is
  // applied there, before the output tile, so that the store phase reads
  // only the tile: applied in the store layout, every row block re-read
  // 64 bytes of these constants per lane and slot from LDS, three times
  // the tile's bytes (Swin-L stage 1: 76.8 against about 80 us)
  f32x4 ln_b[LN ? 2 : 1], ln_s[LN ? 2 : 1];
  if constexpr (LN) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      ln_b[i] = ln_s[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int ch = cb * 32 + 8 * g + 4 * i;
      if (active && ch < p.N) {
        if (p.bias) ln_b[i] = *reinterpret_cast<const f32x4*>(p.bias + ch);
        ln_s[i] = *reinterpret_cast<const f32x4*>(p.colsum + ch);
      }
    }
  }

  // Layer norm, folded into the weights: with z the unit-normalised row,
  //   y_j = sum_c (z_c gamma_c + beta_c) W_jc + b_j
  //       = (sum_c x_c W'_jc - mean s_j) / sigma + b'_j,
  // W' = gamma o W (the packed weight), s_j = sum_c W'_jc, b' = b + W beta
  // (prepared once with the packing).  The products run on the raw row
  // block; the mean and 1/sigma of every token are only needed by the
  // epilogue, so they are computed from LDS while the products are in
  // flight: LL lanes per token, CPL 16-byte chunks of its row per lane
  // (chunk q = ql + LL k: k-step q / 4, part q % 4) held in registers, DPP
  // sums over the group.  One pass of bf16 dot products (each product exact
  // in fp32) gives the sum S1 and the sum of squares S2, and K var = S2 -
  // S1 mean.  That difference loses about log2(S2 / (K var)) bits to
  // cancellation; where more than 8 are at stake (a row whose mean is
  // large against its spread, e.g. mean 40 and spread 1) the wave forms the
  // variance as the definition has it instead, the mean of the squared
  // deviations from the mean, in a second pass over the held chunks.
  constexpr int LL = KS % 2 == 0 ? 8 : 4;                 // lanes per token
  constexpr int CPL = KS * 4 / LL;                        // chunks per lane
  constexpr int TPW_LN = 64 / LL;                         // tokens per wave and pass
  const int ql = lane % LL;
  auto ln_stats = [&]() {
    for (int t0 = wv * TPW_LN; t0 < kLinRows; t0 += kLinWaves * TPW_LN) {  // wave-uniform
      const int t = t0 + lane / LL;
      const char* tile = s_x + (t >> 4) * KS * 1024;
      bf16x8 h[CPL];
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        const int q = ql + LL * k;
        h[k] = *reinterpret_cast<const bf16x8*>(tile + (q >> 2) * 1024 +
                                                uchunk(t & 15, q & 3));
      }
      float s1 = 0.f, s2 = 0.f;
      const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
      for (int k = 0; k < CPL; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 pr = {h[k][2 * e], h[k][2 * e + 1]};
          s1 = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, s1, false);
          s2 = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, s2, false);
        }
      constexpr float kInvK = 1.f / (KS * 32);
      const float S1 = group_sum<LL>(s1), S2 = group_sum<LL>(s2);
      const float mu = S1 * kInvK;
      float kvar = fmaxf(S2 - S1 * mu, 0.f);
      if (__builtin_amdgcn_ballot_w64(kvar < S2 * (1.f / 256.f)) != 0) {  // wave-uniform
        float d2 = 0.f;
#pragma unroll
        for (int k = 0; k < CPL; ++k)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float d = (float)h[k][e] - mu;
            d2 = fmaf(d, d, d2);
          }
        kvar = group_sum<LL>(d2);
      }
      const float rs = rsqrtf(kvar * kInvK + p.eps);
      if (ql == 0) s_stat[t] = make_float2(mu, rs);
    }
  };

  // register-staged loads of row block rr: LDS block bi = tile * KS + k-step;
  // rows past the end load the last row (finite stand-in data, not stored)
  using Regs = u32x4[BPW];
  auto issue = [&](Regs& R, int rr) {
#pragma unroll
    for (int k = 0; k < BPW; ++k) {
      const int bi = wv + kLinWaves * k;
      if (bi < NB) {
        const int tt = bi / KS, ks = bi - tt * KS;
        int tok = rr * kLinRows + tt * 16 + cq;
        if (tok >= T) tok = T - 1;
        // int8 rows of K = 64 KS - 32: the upper half of the last k-step
        // lies past the row, and takes zeros (the packed weight is zero there)
        if (I8 && ks == KS - 1 && p.half_step && gq >= 2)
          R[k] = u32x4{0u, 0u, 0u, 0u};
        else
          R[k] = *reinterpret_cast<const u32x4*>(xb + (size_t)tok * xrow + ks * 64 + 16 * gq);
      }
    }
  };
  auto write = [&](const Regs& R) {
#pragma unroll
    for (int k = 0; k < BPW; ++k) {
      const int bi = wv + kLinWaves * k;
      if (bi < NB) *reinterpret_cast<u32x4*>(s_x + bi * 1024 + uchunk(cq, gq)) = R[k];
    }
  };

  Regs R;
  constexpr bool kEarly = !RES && !I8;
  if (r < r_end) issue(R, r);
  for (; r < r_end; r += step) {
    write(R);
    // bf16 layers without a residual issue the next row block's loads
    // before the barrier, while the other waves still write (Swin-L stage 1
    // QKV 65.7 -> 64.8 us, with the layer norm 77.5 -> 76.3 us; the int8
    // QKV was 1.6% slower that way)
    if (kEarly && r + step < r_end) issue(R, r + step);
    __syncthreads();  // row block visible to every wave
    const int tok0 = r * kLinRows;
    // the residual goes out before the next row block's loads, so waiting
    // for it never waits for them (vector memory returns count in order)
    bf16x8 res[RES ? 2 : 1];
    if constexpr (RES) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (s_active[j]) {
          int tok = tok0 + srow[j];
          if (tok >= T) tok = T - 1;
          res[j] = *reinterpret_cast<const bf16x8*>(rb + (size_t)tok * yrow + sch[j] * 2);
        }
    }
    if (!kEarly && r + step < r_end) issue(R, r + step);
    if (active) {
      f32x4 acc[kLinTiles][2];
      if constexpr (I8) {
        i32x4 iacc[kLinTiles][2];
#pragma unroll
        for (int tt = 0; tt < kLinTiles; ++tt) iacc[tt][0] = iacc[tt][1] = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int tt = 0; tt < kLinTiles; ++tt) {
            const i32x4 b =
                *reinterpret_cast<const i32x4*>(s_x + (tt * KS + ks) * 1024 + uchunk(c, g));
            iacc[tt][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[ks][0], b, iacc[tt][0], 0, 0, 0);
            iacc[tt][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[ks][1], b, iacc[tt][1], 0, 0, 0);
          }
        }
        if constexpr (I8OUT) {
          // the code of every output: one fma, a clamp to +-127, then round
          // half to even (adding 1.5 * 2^23 rounds to an integer and leaves
          // it, in two's complement, in the low byte; the same code as
          // rounding first and clamping after); lane (g, c) packs its 8
          // consecutive channels into the int8 output tile
#pragma unroll
          for (int tt = 0; tt < kLinTiles; ++tt) {
            u32x2 w;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              unsigned word = 0u;
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const float y = __builtin_amdgcn_fmed3f(
                    fmaf((float)iacc[tt][i][q], kq[i][q], kb[i][q]), -127.f, 127.f);
                word |= (__float_as_uint(y + 12582912.f) & 0xFFu) << (8 * q);
              }
              w[i] = word;
            }
            *reinterpret_cast<u32x2*>(s_o + (tt * 16 + c) * kOut8Stride + wv * 32 + 8 * g) = w;
          }
        } else {
          // dequantize in the product layout
#pragma unroll
          for (int tt = 0; tt < kLinTiles; ++tt)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
              for (int q = 0; q < 4; ++q) acc[tt][i][q] = (float)iacc[tt][i][q] * kq[i][q];
        }
      } else {
#pragma unroll
        for (int tt = 0; tt < kLinTiles; ++tt) acc[tt][0] = acc[tt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          // keep each k-step's operand reads next to its products: hoisting
          // every read of the row block would hold 8 * KS registers
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int tt = 0; tt < kLinTiles; ++tt) {
            const bf16x8 b =
                *reinterpret_cast<const bf16x8*>(s_x + (tt * KS + ks) * 1024 + uchunk(c, g));
            acc[tt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks][0], b, acc[tt][0], 0, 0, 0);
            acc[tt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks][1], b, acc[tt][1], 0, 0, 0);
          }
        }
      }
      if constexpr (LN) {
        ln_stats();       // overlaps the products in flight
        __syncthreads();  // every token's (mean, 1/sigma) visible
        // y = (acc - mean s_j) / sigma + b'_j, in the product layout
#pragma unroll
        for (int tt = 0; tt < kLinTiles; ++tt) {
          const float2 st = s_stat[tt * 16 + c];
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[tt][i][q] = fmaf(fmaf(-st.x, ln_s[i][q], acc[tt][i][q]), st.y, ln_b[i][q]);
        }
      }
      // lane (g, c) holds channels 8g + 4i + q of the wave's block for
      // token c of each tile: 8 consecutive floats of the output tile
      if constexpr (!I8OUT) {
#pragma unroll
        for (int tt = 0; tt < kLinTiles; ++tt) {
          char* o = s_o + (tt * 16 + c) * kOutStride + (wv * 32 + 8 * g) * 4;
          *reinterpret_cast<f32x4*>(o) = acc[tt][0];
          *reinterpret_cast<f32x4*>(o + 16) = acc[tt][1];
        }
      }
    } else if constexpr (LN) {
      ln_stats();
      __syncthreads();  // (the barrier of the product waves above)
    }
    __syncthreads();  // output tile complete
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int tok = tok0 + srow[j];
      if (s_active[j] && tok < T) {
        if constexpr (I8OUT) {
          // 16 codes, 16-byte store.  A workgroup of 4 or 6 waves writes
          // whole 128-byte lines of a token, which the output never re-reads
          // (non-temporal); narrower groups write parts of lines that other
          // workgroups complete, which plain stores let meet in L2 (Swin-L
          // stage 1 QKV: 46.2 against 58.6 us with plain stores; Swin-T
          // stage 1, 2 waves: 19.8 against 22.2 us with non-temporal ones)
          const u32x4 w = *reinterpret_cast<const u32x4*>(s_o + srow[j] * kOut8Stride + sch[j] -
                                                          cg * kLinCols);
          u32x4* dst = reinterpret_cast<u32x4*>(yb + (size_t)tok * p.N + sch[j]);
          if constexpr (kLinCols >= 128) __builtin_nontemporal_store(w, dst);
          else *dst = w;
          continue;
        }
        const char* o = s_o + srow[j] * kOutStride + (sch[j] - cg * kLinCols) * 4;
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(o);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(o + 16);
        bf16x8 out;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float y0, y1;
          if constexpr (LN) {  // normalised and biased in the product layout
            y0 = v0[q];
            y1 = v1[q];
          } else {
            y0 = v0[q] + bias[j][0][q];
            y1 = v1[q] + bias[j][1][q];
          }
          if constexpr (RES) {
            y0 += (float)res[j][q];
            y1 += (float)res[j][4 + q];
          }
          out[q] = (__bf16)y0;
          out[4 + q] = (__bf16)y1;
        }
        __builtin_nontemporal_store(out, reinterpret_cast<bf16x8*>(yb + (size_t)tok * yrow + sch[j] * 2));
      }
    }
    __syncthreads();  // every wave is done with both tiles before they are overwritten
  }
}

// packed[cb][ks][i][lane][s] = W[cb*32 + out_channel(i, lane % 16)][ks*32 + 8*(lane/16) + s]
// (times gamma[column], rounded to bf16, when gamma is given)
__global__ void linear_pack_kernel(const uint16_t* w, const float* gamma, uint16_t* wp, int N,
                                   int K) {
  const int KS = K / 32;
  const long long total = (long long)(N / 32) * KS * 2 * 64;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    const int lane = (int)(e & 63);
    const long long t = e >> 6;  // (cb * KS + ks) * 2 + i
    const int i = (int)(t & 1);
    const long long cks = t >> 1;
    const int ks = (int)(cks % KS), cb = (int)(cks / KS);
    const int row = cb * 32 + out_channel(i, lane % 16);
    const int col = ks * 32 + 8 * (lane / 16);
    const u32x4 src = *reinterpret_cast<const u32x4*>(w + (size_t)row * K + col);
    if (gamma) {
      const bf16x8 h = __builtin_bit_cast(bf16x8, src);
      bf16x8 o;
#pragma unroll
      for (int s = 0; s < 8; ++s) o[s] = (__bf16)((float)h[s] * gamma[col + s]);
      *reinterpret_cast<bf16x8*>(wp + e * 8) = o;
    } else {
      *reinterpret_cast<u32x4*>(wp + e * 8) = src;
    }
  }
}

// int8 weight [N][K]: packed[cb][ks][i][lane][s] = W[cb*32 + out_channel(i,
// lane % 16)][ks*64 + 16*(lane/16) + s] for s < 16, zero past K (the bytes
// of the bf16 packing with 64 int8 channels per k-step)
__global__ void linear_pack_i8_kernel(const int8_t* w, int8_t* wp, int N, int K) {
  const int KS = (K + 63) / 64;
  const long long total = (long long)(N / 32) * KS * 2 * 64;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (long long)gridDim.x * blockDim.x) {
    const int lane = (int)(e & 63);
    const long long t = e >> 6;  // (cb * KS + ks) * 2 + i
    const int i = (int)(t & 1);
    const long long cks = t >> 1;
    const int ks = (int)(cks % KS), cb = (int)(cks / KS);
    const int row = cb * 32 + out_channel(i, lane % 16);
    const int col = ks * 64 + 16 * (lane / 16);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (col < K) v = *reinterpret_cast<const u32x4*>(w + (size_t)row * K + col);
    *reinterpret_cast<u32x4*>(wp + e * 16) = v;
  }
}

// layer norm constants of output j: consts[j] = sum_c bf16(gamma_c W_jc)
// (the row sums of the packed weight, rounded as the packing rounds), and
// consts[N + j] = bias_j + sum_c beta_c W_jc; sums in fp64
__global__ void linear_ln_consts_kernel(const uint16_t* w, const float* gamma, const float* beta,
                                        const float* bias, float* consts, int N, int K) {
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < N; j += gridDim.x * blockDim.x) {
    double s = 0.0, b = bias ? (double)bias[j] : 0.0;
    for (int c = 0; c < K; ++c) {
      const float wv = __builtin_bit_cast(float, (unsigned)w[(size_t)j * K + c] << 16);
      s += (double)(float)(__bf16)(wv * gamma[c]);
      b += (double)beta[c] * (double)wv;
    }
    consts[j] = (float)s;
    consts[N + j] = (float)b;
  }
}

// waves per workgroup for N / 32 column blocks: the widest group of 6, 4 or
// 3 that divides them (fewer re-reads of x), else 2.  int8 layers take 9
// first: a group then covers 288-byte spans of a row (Swin-T stage 1 QKV,
// 9 blocks: 15.4 us against 16.7 with 3 waves and 19.8 with 2; Swin-L stage
// 1 QKV, 18 blocks: 44.9-45.4 against 47.0-47.6 us with 6 waves; the bf16
// Swin-T QKV: 16.5 us with 3 waves, 19.3 with 9, 17.8 with 2)
int linear_waves(int ncb, bool i8) {
  if (i8 && ncb % 9 == 0) return 9;
  if (ncb % 6 == 0) return 6;
  return ncb % 4 == 0 ? 4 : ncb % 3 == 0 ? 3 : 2;
}

size_t linear_lds_waves(int K, int waves) {
  return (size_t)kLinTiles * (K / 32) * 1024 + (size_t)kLinRows * lin_out_stride(waves) +
         lin_ln_lds_bytes();
}

template <int KS, int MODE, int WAVES>
int linear_blocks_per_cu(int dev) {
  static std::atomic<int> cache[kMaxDevices];
  const bool cacheable = dev >= 0 && dev < kMaxDevices;
  if (cacheable) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, linear_fwd_kernel<KS, MODE, WAVES>,
                                                   WAVES * 64, linear_lds_waves(KS * 32, WAVES)) !=
          hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  if (cacheable) cache[dev].store(per_cu, std::memory_order_relaxed);
  return per_cu;
}

template <int KS, int MODE, int WAVES>
hipError_t launch_linear_krw(LinearParams p, int dev, int cus, hipStream_t st) {
  p.ncg = (p.ncb + WAVES - 1) / WAVES;
  // a multiple of the column groups (each workgroup keeps one), and of
  // 8 x that when large enough (even XCD shares); never more than the units
  const long long units = (long long)p.blocks * p.ncg;
  long long grid = (long long)cus * linear_blocks_per_cu<KS, MODE, WAVES>(dev);
  if (grid > units) grid = units;
  if (grid >= 8LL * p.ncg) grid -= grid % (8LL * p.ncg);
  else grid -= grid % p.ncg;
  hipLaunchKernelGGL((linear_fwd_kernel<KS, MODE, WAVES>), dim3((unsigned)grid), dim3(WAVES * 64),
                     linear_lds_waves(KS * 32, WAVES), st, p);
  return hipGetLastError();
}

template <int KS, int MODE>
hipError_t launch_linear_kr(const LinearParams& p, int dev, int cus, hipStream_t st) {
  switch (linear_waves(p.ncb, MODE >= kLinI8)) {
    case 9:
      if constexpr (MODE >= kLinI8) return launch_linear_krw<KS, MODE, 9>(p, dev, cus, st);
      return hipErrorInvalidValue;
    case 3: return launch_linear_krw<KS, MODE, 3>(p, dev, cus, st);
    case 6: return launch_linear_krw<KS, MODE, 6>(p, dev, cus, st);
    case 4: return launch_linear_krw<KS, MODE, 4>(p, dev, cus, st);
    default: return launch_linear_krw<KS, MODE, 2>(p, dev, cus, st);
  }
}

template <int KS>
hipError_t launch_linear_ks(const LinearParams& p, int dev, int cus, hipStream_t st) {
  if (p.w_scale) {
    if (p.out_scale) return launch_linear_kr<KS, kLinI8Out>(p, dev, cus, st);
    return p.res ? launch_linear_kr<KS, kLinI8Residual>(p, dev, cus, st)
                 : launch_linear_kr<KS, kLinI8>(p, dev, cus, st);
  }
  if (p.colsum) return launch_linear_kr<KS, kLinLayerNorm>(p, dev, cus, st);
  return p.res ? launch_linear_kr<KS, kLinResidual>(p, dev, cus, st)
               : launch_linear_kr<KS, kLinPlain>(p, dev, cus, st);
}

}  // namespace


hipError_t launch_linear_ln_consts(const void* w, const float* gamma, const float* beta,
                                  const float* bias, float* consts, int N, int K,
                                  hipStream_t stream) {
  hipLaunchKernelGGL(linear_ln_consts_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0,
                     stream, static_cast<const uint16_t*>(w), gamma, beta, bias, consts, N, K);
  return hipGetLastError();
}

hipError_t launch_linear_pack(const void* w, const float* gamma, void* wp, int N, int K,
                              hipStream_t stream) {
  const long long total = (long long)(N / 32) * (K / 32) * 2 * 64;
  long long blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(linear_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(w), gamma, static_cast<uint16_t*>(wp), N, K);
  return hipGetLastError();
}

hipError_t launch_linear_pack_i8(const void* w, void* wp, int N, int K, hipStream_t stream) {
  const long long total = (long long)(N / 32) * ((K + 63) / 64) * 2 * 64;
  long long blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(linear_pack_i8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const int8_t*>(w), static_cast<int8_t*>(wp), N, K);
  return hipGetLastError();
}

hipError_t launch_linear(const LinearParams& q, int dev, int cus, hipStream_t stream) {
  LinearParams p = q;
  p.blocks = (int)((p.T + kLinRows - 1) / kLinRows);
  // k-steps of 64 bytes: 32 bf16 channels, or 64 int8 channels (a last half
  // step when K % 64 == 32)
  p.half_step = p.w_scale && p.K % 64 != 0 ? 1 : 0;
  switch (p.w_scale ? (p.K + 63) / 64 : p.K / 32) {
    case 1: return launch_linear_ks<1>(p, dev, cus, stream);
    case 2: return launch_linear_ks<2>(p, dev, cus, stream);
    case 3: return launch_linear_ks<3>(p, dev, cus, stream);
    case 4: return launch_linear_ks<4>(p, dev, cus, stream);
    case 5: return launch_linear_ks<5>(p, dev, cus, stream);
    case 6: return launch_linear_ks<6>(p, dev, cus, stream);
    case 7: return launch_linear_ks<7>(p, dev, cus, stream);
    case 8: return launch_linear_ks<8>(p, dev, cus, stream);
    case 9: return launch_linear_ks<9>(p, dev, cus, stream);
    case 10: return launch_linear_ks<10>(p, dev, cus, stream);
    case 11: return launch_linear_ks<11>(p, dev, cus, stream);
    case 12: return launch_linear_ks<12>(p, dev, cus, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace swinattn
