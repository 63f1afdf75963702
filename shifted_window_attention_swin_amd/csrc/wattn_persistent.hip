// Persistent, LDS-staged bf16 forward (windows up to 12: 1, 4 or 9 tiles of
// 16 tokens; the Swin windows of 7 and 12 included).
//
// The forward reads every byte once and does little arithmetic per byte, so
// its speed is set by how many bytes are in flight to HBM.  Here that number
// is decoupled from the register budget of the attention math:
//
//   unit       (image, window, group of HG heads): 3*HG slices (q, k, v of
//              each head) x NT tiles, each a 1 KB block of 16 tokens x 64 B
//              staged in LDS.  The Baidu AIAK-Training talk (jxzklqfsx.com
//              743345, section 2, WindowAttention case) describes the fused
//              module as tiles moving through the memory hierarchy of HBM,
//              shared memory and registers; this is that pipeline on gfx950.
//   workgroup  4 waves (3 for 9-tile windows), persistent: the grid walks
//              the units in order, so the units in flight are one compact
//              stretch of the batch; when the units of a window share cache
//              lines, or a launch has at most two units per workgroup, each
//              XCD instead walks its own contiguous range.  A workgroup
//              whose units all belong to one head group stages only that
//              group's bias tables.
//   pipeline   the next unit's 16-byte loads are issued into registers, at
//              raised wave priority, right after the current unit is
//              written to LDS (before the barrier that publishes it, for
//              windows of up to 4 tiles), and stay in flight while the
//              current unit is computed out of LDS.
//   loads      wave w of W loads tiles w, w + W, ... of every slice: a lane
//              owns one token and one 16-byte part of it, so the
//              shift/partition index map is one address per lane per tile.
//              A load instruction covers 16 tokens x 64 contiguous bytes.
//   compute    (head, query tile) items are spread over the waves, a
//              wave's items being all heads of its query tiles; operands
//              come from LDS with ds_read_b128 out of 1 KB blocks whose
//              16-byte parts are swizzled against bank conflicts.  Units of
//              one or two heads re-read key tiles and V^T for every item,
//              which keeps them at 5 workgroups per CU (at most 102 VGPRs);
//              units of 3-4 heads of small windows keep them in registers.
//   stores     the HG heads of a token leave one wave back to back as
//              non-temporal 16-byte stores (whole output lines when HG is
//              even), which the output never re-reads.
//
// The attention math of one item (head h, query tile it):
//
//   S^T = K Q^T + C   v_mfma_f32_16x16x32_bf16 per key tile, K = head_dim =
//             32 exactly.  The accumulator C starts as relative position
//             bias divided by the score scale (and, in masked windows, one
//             more MFMA adds the shift mask, see write_mask), so one fma
//             later turns D into a base-2 logit.  Transposing S puts one
//             query per lane column: the softmax over keys is in-lane plus
//             two permlane swaps.
//   P^T       exp2 of the logits, rounded to bf16: the C/D layout of S^T is
//             directly the B-operand layout of the next MFMA.
//   O^T = V^T P^T   V^T read from LDS with transposing reads; the row sums
//             of P come from one more MFMA against a tile of ones, so the
//             normaliser sums exactly the weights applied.
//   store     each lane writes 8 consecutive channels of one query token:
//             the window reverse and the roll back are the store addresses.
//
// Token layout inside a window ("quad tiles"): with Q = ceil(M/4) the window
// is padded to (4Q) x (4Q) tokens and cut into Q*Q tiles of 4 rows x 4
// columns; in-tile token u sits at row 4*(t/Q) + u/4, column 4*(t%Q) + u%4.
// In the C/D layout row 4g+r of a key tile (g = lane/16) is then window row
// 4*(t/Q)+g, column 4*(t%Q)+r, so the relative position index
// (dy+M-1)(2M-1) + (dx+M-1) of (query, key) splits into a per-lane part and
// a compile-time part: with the bias table stored reversed in LDS, every bias
// gather is one ds_read with an immediate offset.  Padded keys get -inf in
// the accumulator (weight exactly 0); padded tokens load the window's first
// token as finite stand-in data (weight 0 times finite = 0 in the value
// product); padded queries are not stored.

#include <atomic>
#include <type_traits>

#include "wattn_common.h"

namespace swinattn {
namespace {

// waves per workgroup: 4, or 3 for windows of 9 tiles (their 9 query tiles
// then split evenly, and 4 workgroups of 3 waves per CU leave each wave 168
// VGPRs)
template <int M>
constexpr int fwd_waves() {
  return Win<M>::NT > 4 ? 3 : 4;
}
template <int M, int HG>
struct Unit {
  using S = Win<M>;
  static constexpr int kWaves = fwd_waves<M>();
  static constexpr int NT = S::NT;
  static constexpr int SLICES = 3 * HG;                    // q, k, v of HG heads
  static constexpr int TPW = (NT + kWaves - 1) / kWaves;   // tiles loaded per wave
  static constexpr int ITEMS = HG * NT;                    // (head, query tile) items
  static constexpr int IPW = (ITEMS + kWaves - 1) / kWaves;
  // head-inner order: a wave's items are all HG heads of its query tiles, so
  // the HG * 64 output bytes of a token leave the wave together (whole cache
  // lines) instead of 64-byte halves from different waves
  static constexpr bool HEAD_INNER = HG > 1 && IPW % HG == 0;
  // every wave's items belong to one head: key / value tiles load once
  static constexpr bool ONE_HEAD = !HEAD_INNER && ITEMS % kWaves == 0 && NT % IPW == 0;
  // items that do not divide evenly over the waves leave the last wave
  // short; the short wave rotates from unit to unit so that no SIMD sits out
  // all the math.  With 4 waves this applies to units of 1-tile windows (HG
  // items) when HG is not a multiple of 4; the 9 query tiles of a one-head
  // unit of windows 9 to 12 divide evenly over their 3 waves
  static constexpr bool ROTATE = ITEMS % kWaves != 0;
  static constexpr int BLOCK = 1024;                       // 16 tokens x 64 bytes
  // LEAN: windows of up to 4 tiles with units of one or two heads re-read
  // key tiles, V^T and mask operands from LDS for every item, so that 5
  // workgroups fit per CU (at most 102 VGPRs; their one-head-group bias
  // tables keep 5 units within the LDS)
  static constexpr bool LEAN = NT <= 4 && HG <= 2;
  // units of 3 or 4 heads of windows up to 4 tiles keep key tiles, V^T and
  // mask operands in registers for all items of a wave; the others re-read
  // them from LDS
  static constexpr bool HOLD = NT <= 4 && !LEAN;
  static constexpr int MASK_BYTES = HOLD ? 0 : NT * BLOCK;  // key-side mask operands
  static constexpr int BYTES = SLICES * NT * BLOCK + MASK_BYTES;
  static constexpr int block(int s, int t) { return (s * NT + t) * BLOCK; }
  static constexpr int mask_block(int t) { return (SLICES * NT + t) * BLOCK; }
};

// Window coordinates (row, column) of in-tile token u of tile t.
template <int M>
SWA_INLINE void tile_token(int t, int u, int& ty, int& tx) {
  ty = 4 * (t / Win<M>::Q) + u / 4;
  tx = 4 * (t % Win<M>::Q) + u % 4;
}

// Flattened image position (within the launch) of window token (ty, tx);
// tokens outside the window stand in for the window's first token.
SWA_INLINE unsigned token_pixel(const FwdParams& p, int M, int b, int wy, int wx, int ty, int tx,
                                bool ok) {
  int y = wy * M + (ok ? ty : 0) + p.shift, x = wx * M + (ok ? tx : 0) + p.shift;
  y -= y >= p.H ? p.H : 0;
  x -= x >= p.W ? p.W : 0;
  return ((unsigned)b * p.H + y) * p.W + x;
}

// Stages the bias tables of heads h0 .. h0 + count - 1, each reversed and
// divided by the scale, followed by the zero tail read by padded keys.
template <int M>
SWA_INLINE void stage_bias_heads(float* s_bias, const float* table, int nh, int h0, int count,
                                 float inv_scale) {
  using S = Win<M>;
  const int n = count * S::T;
  for (int e = threadIdx.x; e < n + S::TAIL; e += blockDim.x) {
    float v = 0.f;
    if (e < n) {
      const int h = e / S::T, k = e - h * S::T;
      v = table[(S::T - 1 - k) * nh + h0 + h] * inv_scale;
    }
    s_bias[e] = v;
  }
}

// waves per SIMD the register allocation must leave room for
template <int M, int HG>
constexpr int fwd_minw() {
  return fwd_waves<M>() == 3 ? 3 : Unit<M, HG>::LEAN ? 5 : 1;
}

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// 8 int8 codes (two dwords, code k in byte k) as 8 bf16 values in the
// 16-byte layout of a bf16 chunk.  bf16 holds every int8 value exactly.
SWA_INLINE u32x4 widen_chunk(u32x2 v) {
  bf16x8 r;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    r[k] = (__bf16)(float)(int)(signed char)(v[k / 4] >> (8 * (k % 4)));
  return __builtin_bit_cast(u32x4, r);
}
SWA_INLINE u32x4 widen_chunk(u32x4 v) { return v; }

// The persistent forward.  I8: q, k and v arrive as int8 codes with one
// scale per part, and the output is bf16, or int8 codes (out_i8).  A lane
// loads the 8 codes of its token part (8 bytes, in place of 16 bytes of
// bf16) and writes them to LDS as bf16; from there the math is the bf16
// kernel's.  The score MFMA then sums 32 products of codes
// (each at most 2^14 in magnitude) in fp32, which holds every such sum
// exactly: it is the int32 accumulation of an int8 product.  The host folds
// the query and key scales into the score scale (and so into the bias and
// mask, which are pre-divided by it); the value scale multiplies the
// normaliser.
template <int M, int HG, bool I8>
__global__ __launch_bounds__(fwd_waves<M>() * 64, (fwd_minw<M, HG>())) void wattn_fwd_persistent(FwdParams p) {
  using S = Win<M>;
  using U = Unit<M, HG>;
  constexpr int NT = S::NT, NK = S::NK;
  extern __shared__ float s_lds[];
  float* s_bias = s_lds;
  constexpr int kWaves = U::kWaves;
  // bias tables staged: every head (own_bias 0); only the HG heads of the
  // workgroup's head group, which is the same in all its units (1); or
  // only the HG heads of the current unit's head group, staged again
  // between units when it changes (2: head counts whose tables together
  // exceed the LDS budget, on grids that cannot keep one head group per
  // workgroup)
  const int bias_floats = (p.own_bias ? HG : p.nh) * S::T + S::TAIL;
  char* s_unit = reinterpret_cast<char*>(s_lds) + ((bias_floats * 4 + 15) & ~15);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gq = lane & 3, cq = lane >> 2;    // load layout: 16-byte part, token
  // byte offset of 16-byte part `part` of in-tile token u in a 1 KB block:
  // the part is XORed with bits 1-2 of the token, so that the tokens 4
  // apart that a lane group reads together sit in different banks
  auto uchunk = [](int u, int part) {
    return 64 * u + 16 * (part ^ ((u >> 1) & 3));
  };
  const int g = lane >> 4, c = lane & 15;     // MFMA layout: lane group, token
  const int nh = p.nh;
  const unsigned Cb = (unsigned)nh * kHeadDim * 2;  // bytes of one bf16 q (k, v, out) row
  constexpr unsigned EB = I8 ? 1 : 2;                // bytes of one input element
  const unsigned Ci = (unsigned)nh * kHeadDim * EB;  // bytes of one input q (k, v) row
  const char* in = static_cast<const char*>(p.qkv);
  char* out = static_cast<char*>(p.out);
  const int units = p.units;

  // this workgroup's units.  Default: the grid walks the units in order
  // (unit id + k * grid), so the units in flight form one compact stretch of
  // the batch.  Units of one window whose slices share cache lines (64-byte
  // head slices) instead take one contiguous range per XCD, interleaved over
  // the XCD's workgroups: the halves of a line then meet in one L2.
  const int G = gridDim.x, id = blockIdx.x;
  int u, u_step, u_end;
  if (p.xcd_ranges && (G & 7) == 0) {
    const int x = id & 7, per = G >> 3;
    const long long r0 = (long long)units * x / 8, r1 = (long long)units * (x + 1) / 8;
    u = (int)r0 + (id >> 3);
    u_step = per;
    u_end = (int)r1;
  } else {
    u = id;
    u_step = G;
    u_end = units;
  }
  // first head of the workgroup's head group when its bias tables alone are
  // staged (the host sets own_bias only for grids that keep u_step a
  // multiple of the head-group count)
  int hbase = p.own_bias ? (u % p.nhg) * HG : 0;


  // unit u -> (head group, image, window); decoded once, used for the loads
  // and, one iteration later, for the math
  struct Pos {
    int hg, b, wy, wx;
  };
  auto decode = [&](int uu) {
    Pos q;
    q.hg = uu % p.nhg;
    const int bw = uu / p.nhg;
    q.b = bw / p.nW;
    const int w = bw - q.b * p.nW;
    q.wy = w / p.nWx;
    q.wx = w - q.wy * p.nWx;
    return q;
  };

  // register-staged loads of one unit: slice s, tile wv + 4k of this wave,
  // raw chunks of 8 elements (16 bytes of bf16, 8 bytes of int8 codes)
  using Chunk = std::conditional_t<I8, u32x2, u32x4>;
  using Regs = Chunk[U::SLICES][U::TPW];
  auto issue_loads = [&](Regs& R, const Pos& q) {
#pragma unroll
    for (int k = 0; k < U::TPW; ++k) {
      const int t = wv + kWaves * k;
      if (t < NT) {
        int ty, tx;
        tile_token<M>(t, cq, ty, tx);
        const bool ok = ty < M && tx < M;
        const unsigned pix = token_pixel(p, M, q.b, q.wy, q.wx, ty, tx, ok);
        const char* src = in + pix * (3u * Ci) + (unsigned)q.hg * HG * kHeadDim * EB + 8u * EB * gq;
#pragma unroll
        for (int s = 0; s < U::SLICES; ++s)
          R[s][k] = *reinterpret_cast<const Chunk*>(src + (s / HG) * Ci + (s % HG) * kHeadDim * EB);
      }
    }
  };
  // key-side mask operands of a window for large windows: wave w writes
  // tiles w, w+4, ...  (each lane's operand depends on the lane only)
  auto write_mask = [&](const Pos& q) {
    if constexpr (!U::HOLD) {
      if (window_masked(p.shift, q.wy, q.wx, p.nWy, p.nWx)) {
#pragma unroll
        for (int k = 0; k < U::TPW; ++k) {
          const int t = wv + kWaves * k;
          if (t < NT) {
            int ty, tx;
            tile_token<M>(t, c, ty, tx);
            const int loc = 2 * (q.wy * M + ty >= p.H - p.shift) + (q.wx * M + tx >= p.W - p.shift);
            bf16x8 a = {};
#pragma unroll
            for (int j = 0; j < 3; ++j) a[j] = loc == g ? (__bf16)p.mask_pieces[j] : (__bf16)0.f;
            *reinterpret_cast<bf16x8*>(s_unit + U::mask_block(t) + lane * 16) = a;
          }
        }
      }
    }
  };
  auto write_unit = [&](const Regs& R) {
#pragma unroll
    for (int k = 0; k < U::TPW; ++k) {
      const int t = wv + kWaves * k;
      if (t < NT) {
#pragma unroll
        for (int s = 0; s < U::SLICES; ++s)
          *reinterpret_cast<u32x4*>(s_unit + U::block(s, t) + uchunk(lane >> 2, lane & 3)) =
              widen_chunk(R[s][k]);
      }
    }
  };

  const bool g_ok = g < S::LG;  // lane group is a window row in the last row group
  bf16x8 ones;                   // A operand of the row-sum MFMA
#pragma unroll
  for (int s = 0; s < 8; ++s) ones[s] = (__bf16)1.f;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};

  // the math of one unit, out of LDS; `rot` selects which wave takes which
  // share of the items
  auto process = [&](const Pos& pos, int rot) {
    const int hg = pos.hg, b = pos.b, wy = pos.wy, wx = pos.wx;
    const int wq = U::ROTATE ? (wv + rot) % kWaves : wv;
    const bool masked = window_masked(p.shift, wy, wx, p.nWy, p.nWx);
    // key-side mask operand of key tile t for this lane (see
    // LaneWindow::init_labels): it depends on the lane only, not the head
    auto key_mask = [&](int t) {
      int ty, tx;
      tile_token<M>(t, c, ty, tx);
      const int loc = 2 * (wy * M + ty >= p.H - p.shift) + (wx * M + tx >= p.W - p.shift);
      bf16x8 a = {};
#pragma unroll
      for (int k = 0; k < 3; ++k) a[k] = loc == g ? (__bf16)p.mask_pieces[k] : (__bf16)0.f;
      return a;
    };
    bf16x8 mask_a[U::HOLD ? NT : 1];
    if (masked) {
      if constexpr (U::HOLD) {
#pragma unroll
        for (int t = 0; t < NT; ++t) mask_a[t] = key_mask(t);
      }
    }

    // key tiles and the transposed value tiles of local head hl
    constexpr int NH = U::HOLD ? NT : 1, NKH = U::HOLD ? NK : 1;
    bf16x8 kt[NH], va[2][NKH];
    auto key_tile = [&](int hl, int t) {
      return *reinterpret_cast<const bf16x8*>(s_unit + U::block(HG + hl, t) + uchunk(c, g));
    };
    // V^T straight from LDS with the transposing read: in each group of 16
    // lanes, lane i receives element i%4 of the 8-byte chunks read by lanes
    // i/4, i/4+4, i/4+8, i/4+12.  Lane L reading bytes 8*hf.. of its own
    // 16-byte slot of a value tile therefore receives, for k = 0..3, channel
    // out_channel(hf, c) of in-tile token 4g+k: rows 4g..4g+3 of V^T, the
    // A-operand slots of key tile t.
    auto value_t = [&](int hl, int kk, int hf) {
      const int t1 = 2 * kk + 1 < NT ? 2 * kk + 1 : 2 * kk;  // odd tile count: any finite data
      const int own = uchunk(lane >> 2, lane & 3) + 8 * hf;
      const bf16x4 lo = lds_read_tr(s_unit + U::block(2 * HG + hl, 2 * kk) + own);
      const bf16x4 hi = lds_read_tr(s_unit + U::block(2 * HG + hl, t1) + own);
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto load_head = [&](int hl) {
      if constexpr (U::HOLD) {
#pragma unroll
        for (int t = 0; t < NT; ++t) kt[t] = key_tile(hl, t);
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) va[hf][kk] = value_t(hl, kk, hf);
      }
    };
    int cur = -1;
    if (U::ONE_HEAD) {
      cur = wq * U::IPW / NT;
      load_head(cur);
    }
    bf16x8 ovs[HG];  // head-inner: outputs of the query tile's heads, stored together
#pragma unroll
    for (int i = 0; i < U::IPW; ++i) {
      const int item = wq * U::IPW + i;
      if (item >= U::ITEMS) break;
      int hl, it;
      if constexpr (U::HEAD_INNER) {
        hl = i % HG;
        it = wq * (U::IPW / HG) + i / HG;
      } else {
        hl = item / NT;
        it = item - hl * NT;
      }
      const int h = hg * HG + hl;
      if (!U::ONE_HEAD && hl != cur) {
        cur = hl;
        load_head(hl);
      }
      // the query tile and what the lane needs about its query token
      const bf16x8 q = *reinterpret_cast<const bf16x8*>(s_unit + U::block(hl, it) + uchunk(c, g));
      int ty, tx;
      tile_token<M>(it, c, ty, tx);
      const bool ok = ty < M && tx < M;
      int qbase = (h - hbase) * S::T + S::T - 1 - S::C0 - (ok ? S::D * ty + tx : 0) + S::D * g;
      // 9-tile windows: one base register per item for the bias reads,
      // opaque to the compiler, so that it keeps the table constants in the
      // base and the key offsets E(jt) + r (at most 195 words) in the
      // immediate offsets of paired reads instead of an address add per
      // read (window 12: 58.8 -> 57.7 us; smaller windows need no adds)
      if constexpr (NT > 4) asm("" : "+v"(qbase));
      bf16x8 mask_b = {};
      if (masked) {
        const int loc = 2 * (wy * M + ty >= p.H - p.shift) + (wx * M + tx >= p.W - p.shift);
#pragma unroll
        for (int k = 0; k < 3; ++k) mask_b[k] = loc == g ? (__bf16)0.f : (__bf16)-1.f;
      }

      // score tiles.  MASKED: 0 no mask, 1 mask, 2 the window's flag tested
      // per tile.  Nine-tile windows take the flag once per item, outside
      // the tile loop, so that the bias reads and MFMAs of all key tiles are
      // scheduled together (the loop unrolls into one block); smaller
      // windows keep the per-tile test, whose code needs fewer registers
      // and keeps four workgroups per CU
      f32x4 sc[NT];
      auto score_tiles = [&](auto masked_c) {
        constexpr int MASKED = decltype(masked_c)::value;
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
          bf16x8 kj;
          if constexpr (U::HOLD) kj = kt[jt];
          else kj = key_tile(hl, jt);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kj, q, acc, 0, 0, 0);
          if (MASKED == 1 || (MASKED == 2 && masked)) {
            bf16x8 mj;
            if constexpr (U::HOLD) mj = mask_a[jt];
            else mj = *reinterpret_cast<const bf16x8*>(s_unit + U::mask_block(jt) + lane * 16);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mj, mask_b, acc, 0, 0, 0);
          }
          sc[jt] = acc;
        }
      };
      if constexpr (U::HOLD) {
        score_tiles(std::integral_constant<int, 2>{});
      } else {
        if (masked) score_tiles(std::integral_constant<int, 1>{});
        else score_tiles(std::integral_constant<int, 0>{});
      }
      softmax_numerators<M>(sc, p.score_scale);
      bf16x8 pb[NK];
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pb[kk][r] = (__bf16)sc[2 * kk][r];
          pb[kk][4 + r] = (2 * kk + 1 < NT) ? (__bf16)sc[2 * kk + 1][r] : (__bf16)0.f;
        }
      f32x4 o0 = z, o1 = z, l4 = z;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        bf16x8 v0, v1;
        if constexpr (U::HOLD) {
          v0 = va[0][kk];
          v1 = va[1][kk];
        } else {
          v0 = value_t(hl, kk, 0);
          v1 = value_t(hl, kk, 1);
        }
        o0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v0, pb[kk], o0, 0, 0, 0);
        o1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v1, pb[kk], o1, 0, 0, 0);
        l4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[kk], l4, 0, 0, 0);
      }
      if (ok) {
        const float inv = I8 ? fast_rcp(l4[0]) * p.v_scale : fast_rcp(l4[0]);
        if constexpr (I8) {
          if (p.out_i8) {
            // int8 output: v_scale is the value scale over the output
            // scale; the code is clamp(rne(o), -127, 127) (adding 1.5 * 2^23
            // rounds half to even and leaves the code in the low byte), 8
            // codes of the lane's 8 channels in one 8-byte store
            u32x2 w = {0u, 0u};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float y0 = __builtin_amdgcn_fmed3f(o0[r] * inv, -127.f, 127.f) + 12582912.f;
              const float y1 = __builtin_amdgcn_fmed3f(o1[r] * inv, -127.f, 127.f) + 12582912.f;
              w[0] |= (__float_as_uint(y0) & 0xFFu) << (8 * r);
              w[1] |= (__float_as_uint(y1) & 0xFFu) << (8 * r);
            }
            const unsigned pix = token_pixel(p, M, b, wy, wx, ty, tx, true);
            __builtin_nontemporal_store(
                w, reinterpret_cast<u32x2*>(out + pix * (Cb / 2) + h * kHeadDim + 8 * g));
            continue;
          }
        }
        bf16x8 ov;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          ov[r] = (__bf16)(o0[r] * inv);
          ov[4 + r] = (__bf16)(o1[r] * inv);
        }
        const unsigned pix = token_pixel(p, M, b, wy, wx, ty, tx, true);
        bf16x8* dst = reinterpret_cast<bf16x8*>(out + pix * Cb + h * kHeadDim * 2 + 16 * g);
        // the output is not read again: non-temporal stores keep it from
        // displacing cached input lines
        auto store = [&](bf16x8* d, const bf16x8& v) { __builtin_nontemporal_store(v, d); };
        if constexpr (U::HEAD_INNER) {
          ovs[hl] = ov;
          if (hl == HG - 1) {
            // head hl' of the token sits (hl' - hl) * 64 bytes from dst
#pragma unroll
            for (int k = 0; k < HG; ++k) store(dst + 4 * (k - (HG - 1)), ovs[k]);
          }
        } else {
          store(dst, ov);
        }
      }
    }
  };

  // software pipeline: the next unit's loads are in flight while a unit is
  // written to LDS and computed
  Regs R;
  int rot = 0;
  Pos nxt = decode(u);
  if (u < u_end) issue_loads(R, nxt);
  // the bias table (reversed, divided by the scale) is staged while the
  // first unit's loads are in flight
  stage_bias_heads<M>(s_bias, p.table, nh, hbase, p.own_bias ? HG : nh, p.inv_scale);
  __syncthreads();  // bias table visible
  for (; u < u_end; u += u_step) {
    write_unit(R);
    write_mask(nxt);
    if (p.own_bias == 2 && nxt.hg * HG != hbase) {
      // the previous unit's math is done (barrier at the end of the
      // iteration): its tables may be replaced
      hbase = nxt.hg * HG;
      stage_bias_heads<M>(s_bias, p.table, nh, hbase, HG, p.inv_scale);
    }
    // the registers are free once the unit is written: windows of up to 4
    // tiles issue the next unit's loads before the barrier, so they leave
    // while the other waves still write (Swin-L stage 1: 58.3 against
    // 59.0-59.3 us; window 12 keeps them after it: 58.7-58.8 against
    // 59.1-59.7 us)
    constexpr bool kEarly = NT <= 4;
    if (!kEarly) __syncthreads();  // unit (and its bias tables) visible to every wave
    const Pos cur = nxt;
    if (u + u_step < u_end) {
      nxt = decode(u + u_step);
      // the loads leave ahead of the other workgroups' math on the SIMD
      __builtin_amdgcn_s_setprio(3);
      issue_loads(R, nxt);
      __builtin_amdgcn_s_setprio(0);
    }
    if (kEarly) __syncthreads();  // unit (and its bias tables) visible to every wave
    process(cur, rot++);
    __syncthreads();  // every wave is done with the unit before it is overwritten
  }
}

template <int M, int HG>
size_t lds_bytes_mh(int nh) {
  const size_t bias = ((size_t)nh * Win<M>::T + Win<M>::TAIL) * sizeof(float);
  return ((bias + 15) & ~size_t(15)) + Unit<M, HG>::BYTES;
}

// workgroups of wattn_fwd_persistent<M, HG, I8> resident per CU for `lds`
// bytes of dynamic LDS; cached per device as (lds << 8 | blocks)
template <int M, int HG, bool I8>
int blocks_per_cu(int dev, size_t lds, int slot) {
  static std::atomic<long long> cache[kMaxDevices][2];
  const bool cacheable = dev >= 0 && dev < kMaxDevices;
  if (cacheable) {
    const long long c = cache[dev][slot].load(std::memory_order_relaxed);
    if (c > 0 && (size_t)(c >> 8) == lds) return (int)(c & 255);
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, wattn_fwd_persistent<M, HG, I8>,
                                                   Unit<M, HG>::kWaves * 64, lds) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  if (per_cu > 255) per_cu = 255;
  if (cacheable) cache[dev][slot].store(((long long)lds << 8) | per_cu, std::memory_order_relaxed);
  return per_cu;
}

// Grid for `lds` bytes per workgroup: CUs x resident workgroups, at most
// one per unit, whole rounds of the 8 XCDs.
template <int M, int HG, bool I8>
long long fwd_grid(const FwdParams& p, int dev, int cus, size_t lds, int slot) {
  long long grid = (long long)cus * blocks_per_cu<M, HG, I8>(dev, lds, slot);
  if (grid > p.units) grid = p.units;
  if (grid >= 8) grid &= ~7LL;  // whole XCD rounds (equal share per XCD)
  return grid;
}

template <int M, int HG, bool I8>
hipError_t launch_mh(const FwdParams& p_in, int dev, int cus, hipStream_t st) {
  FwdParams p = p_in;
  p.own_bias = 0;
  size_t lds = lds_bytes_mh<M, HG>(p.nh);
  const size_t small = lds_bytes_mh<M, HG>(HG);
  // the tables of every head would take more than the LDS budget (e.g. 48
  // heads at window 12, 101.6 KB): one head group's tables only
  const bool must_own = lds > (size_t)kMaxTableLds;
  long long grid = -1;
  if (Win<M>::NT > 4 || Unit<M, HG>::LEAN || must_own) {
    // 9-tile windows: when a workgroup's units all share one head group it
    // stages only that group's bias tables (one head's table instead of
    // nh), which leaves LDS for one more workgroup per CU.  A workgroup
    // steps through units by the grid (grid order) or by the grid / 8 (XCD
    // ranges), so the grid is cut to a multiple of nhg (8 nhg): at most
    // 8 nhg - 8 workgroups fewer, e.g. 1008 instead of 1024 at 6 heads.
    if (p.nhg > 1) {
      long long g = fwd_grid<M, HG, I8>(p, dev, cus, small, 1);
      const bool xcd = p.xcd_ranges && g % 8 == 0;
      const long long q = xcd || Unit<M, HG>::LEAN ? 8LL * p.nhg : p.nhg;
      if (g >= q) g -= g % q;
      if (g % q == 0) {
        grid = g;
        lds = small;
        p.own_bias = 1;
      } else if (must_own) {
        grid = fwd_grid<M, HG, I8>(p, dev, cus, small, 1);
        lds = small;
        p.own_bias = 2;
      }
    }
  }
  if (grid < 0) grid = fwd_grid<M, HG, I8>(p, dev, cus, lds, 0);
  // launches of at most two units per workgroup walk one contiguous range
  // per XCD (Swin-T stage 3: 10.6 -> 10.0 us); longer ones keep grid order,
  // which keeps the units in flight one compact stretch of the batch
  // (Swin-L stage 1: 58.4 against 61.6 us with XCD ranges).  A one-head-
  // group grid is then a multiple of 8 nhg already, as XCD ranges need.
  if (!p.xcd_ranges && p.nhg > 1 && grid % 8 == 0 && p.units <= 2 * grid &&
      (p.own_bias != 1 || (grid / 8) % p.nhg == 0))
    p.xcd_ranges = 1;
  hipLaunchKernelGGL((wattn_fwd_persistent<M, HG, I8>), dim3((unsigned)grid),
                     dim3(Unit<M, HG>::kWaves * 64), lds, st, p);
  return hipGetLastError();
}

template <int M, bool I8>
hipError_t launch_m(int HG, const FwdParams& p, int dev, int cus, hipStream_t st) {
  if constexpr (Win<M>::NT > 4) {  // larger windows: one head per unit
    return HG == 1 ? launch_mh<M, 1, I8>(p, dev, cus, st) : hipErrorInvalidValue;
  } else {
    switch (HG) {
      case 1: return launch_mh<M, 1, I8>(p, dev, cus, st);
      case 2: return launch_mh<M, 2, I8>(p, dev, cus, st);
      case 3: return launch_mh<M, 3, I8>(p, dev, cus, st);
      case 4: return launch_mh<M, 4, I8>(p, dev, cus, st);
      default: return hipErrorInvalidValue;
    }
  }
}

}  // namespace

#define SWA_PERSISTENT_M(CALL)                                                   \
  switch (M) {                                                                   \
    case 1: return CALL(1);                                                      \
    case 2: return CALL(2);                                                      \
    case 3: return CALL(3);                                                      \
    case 4: return CALL(4);                                                      \
    case 5: return CALL(5);                                                      \
    case 6: return CALL(6);                                                      \
    case 7: return CALL(7);                                                      \
    case 8: return CALL(8);                                                      \
    case 9: return CALL(9);                                                      \
    case 10: return CALL(10);                                                    \
    case 11: return CALL(11);                                                    \
    case 12: return CALL(12);                                                    \
    default: break;                                                              \
  }

hipError_t launch_fwd_bf16_persistent(int M, int HG, const FwdParams& p, int dev, int cus,
                                      hipStream_t stream) {
#define SWA_LAUNCH(m) launch_m<m, false>(HG, p, dev, cus, stream)
  SWA_PERSISTENT_M(SWA_LAUNCH)
#undef SWA_LAUNCH
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_i8_persistent(int M, int HG, const FwdParams& p, int dev, int cus,
                                    hipStream_t stream) {
#define SWA_LAUNCH(m) launch_m<m, true>(HG, p, dev, cus, stream)
  SWA_PERSISTENT_M(SWA_LAUNCH)
#undef SWA_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace swinattn
