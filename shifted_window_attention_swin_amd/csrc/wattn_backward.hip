// Backward of the fused shifted-window attention (bf16, windows up to 12:
// 1, 4 or 9 tiles of 16 tokens), for training.  The NVIDIA talk "Swin
// Transformer training and inference optimization" (uticex.com 1598),
// section 2, fuses the window attention's backward as it fuses the forward.
//
// Per window and head, with S = Q K^T / sqrt(d) + bias + mask, P = softmax(S)
// and dO the output gradient gathered through the same shift and partition:
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,  dS = P o (dP - D),
//   dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d),  dtable[rel(i,j)] += dS_ij.
//
//   unit      (image, window, head or head pair): q, k, v and dO of the
//             heads, each 16-token tile a 1 KB LDS block (16 tokens x 64 B,
//             16-byte parts swizzled against bank conflicts), staged like
//             the forward's (register prefetch of the next unit, issued at
//             raised wave priority).
//   streams   a workgroup keeps one head (or a pair of heads whose 64-byte
//             rows share the 128-byte lines of a token) and walks a
//             contiguous run of at least 8 windows; the head groups of one
//             run sit on one XCD and walk it in step, so the lines that
//             hold several heads of a token are fetched into one L2.
//   waves     one per 16-token tile of the head: 4 per head for windows up
//             to 8 (1 or 4 tiles), 9 for windows of 9 to 12 (whose P and dS
//             blocks, 81 KB, leave room for one workgroup per CU)
//   phase 1   one wave per query tile, in the forward's transposed layout
//             (keys in a lane's accumulator rows, queries across lanes):
//             S^T and P (fp32, exact softmax), dP^T = V dO^T, D, dS^T, and
//             dQ^T = K^T dS^T (K^T from transposing LDS reads, as the
//             forward's V^T).  P and dS go to LDS in bf16 as 16 x 16 blocks
//             [query][key], one per (query tile, key tile), their 8-byte key
//             groups swizzled by query row.
//   phase 2   one wave per key tile: dV^T += dO^T P and dK^T += Q^T dS on
//             16x16x16 MFMAs, their B operands read out of the P and dS
//             blocks with transposing LDS reads (4 queries of a key per
//             lane), dO^T and Q^T from transposing reads of the unit.
//   bias grad the (query, key) pair of a phase-1 accumulator slot of a lane
//             is the same in every window, hence so is its table row: each
//             lane sums the fp32 dS of its 4 x tiles slots in registers over
//             all its workgroup's windows, then adds them once into an LDS
//             copy of the head's table gradient (LDS atomics), which goes to
//             HBM with global atomics.
//   output    head pairs: dQ, dK, dV go through a swizzled LDS tile and leave
//             as whole 128-byte lines; one head: 16-byte stores of 8
//             channels of the lane's token.

#include <atomic>
#include <type_traits>

#include "bwd_internal.h"
#include "wattn_common.h"

namespace swinattn {
namespace {

constexpr int kMinRunWindows = 8;  // windows per run of a workgroup, at least

// waves per head: one per 16-token tile, at least 4 (windows of up to 8
// have 1 or 4 tiles, windows of 9 to 12 have 9)
template <int M>
constexpr int bwd_waves() {
  return Win<M>::NT > 4 ? Win<M>::NT : 4;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

SWA_INLINE f32x4 mfma16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                    __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// sum over the four lane groups (lanes c, c+16, c+32, c+48)
SWA_INLINE float sum_groups(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Window coordinates (row, column) of in-tile token u of tile t.
template <int M>
SWA_INLINE void btile_token(int t, int u, int& ty, int& tx) {
  ty = 4 * (t / Win<M>::Q) + u / 4;
  tx = 4 * (t % Win<M>::Q) + u % 4;
}

// Flattened image position of window token (ty, tx) of window (wy, wx),
// shifted frame to image; tokens outside the window stand in for its first.
SWA_INLINE unsigned bwd_pixel(const BwdParams& p, int M, int b, int wy, int wx, int ty, int tx,
                              bool ok) {
  int y = wy * M + (ok ? ty : 0) + p.shift, x = wx * M + (ok ? tx : 0) + p.shift;
  y -= y >= p.H ? p.H : 0;
  x -= x >= p.W ? p.W : 0;
  return ((unsigned)b * p.H + y) * p.W + x;
}

template <int M, int HP>
struct BwdLds {
  using S = Win<M>;
  static constexpr int TAB = S::T + S::TAIL;    // floats of one head's reversed table
  static constexpr int UNIT = 4 * S::NT * 1024;  // q, k, v, dO tiles of one head
  static constexpr int PBLK = 512;               // 16 x 16 bf16
  static constexpr int PHEAD = S::NT * S::NT * PBLK;  // P (or dS) blocks of one head
  static constexpr int OFF_UNIT = ((HP * TAB + HP * S::T) * 4 + 15) / 16 * 16;
  static constexpr int OFF_P = OFF_UNIT + HP * UNIT;
  static constexpr int OFF_DS = OFF_P + HP * PHEAD;
  static constexpr int BYTES = OFF_DS + HP * PHEAD;
};

// HP = 1: a workgroup of 4 waves keeps one head.  HP = 2: 8 waves keep the
// pair of heads (2k, 2k+1) whose 64-byte rows share the 128-byte lines of
// a token, wave 4 hl + t on tile t of head 2k + hl, and the gradients of both
// heads leave through LDS tiles [tile][16 tokens][128 B] so that every store
// instruction writes whole lines (8 tokens x 128 B): dQ through the k tiles
// (free once the query phase is done), dK and dV through the P and dS blocks
// (free once the key phase is done).
template <int M, int HP>
__global__ __launch_bounds__(bwd_waves<M>() * 64 * HP) void wattn_bwd_bf16_kernel(BwdParams p) {
  using S = Win<M>;
  using L = BwdLds<M, HP>;
  constexpr int NT = S::NT, T = S::T;
  constexpr int WV = bwd_waves<M>();  // waves per head
  static_assert(NT <= WV, "one wave per tile");
  static_assert(HP == 1 || (HP == 2 && NT == 4), "head pairs for 4-tile windows");
  constexpr int BLOCK = 1024;
  constexpr int SLICES = 4;  // q, k, v, dO
  extern __shared__ float s_lds[];
  const int nh = p.nh;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wv >= 0 && wv < WV * HP);
  const int hl = wv / WV;  // head of the wave within the workgroup
  const int tw = wv % WV;  // tile of the wave
  const int gq = lane & 3, cq = lane >> 2;  // load layout: 16-byte part, token
  const int g = lane >> 4, c = lane & 15;   // MFMA layout: lane group, token

  float* s_brev = s_lds + hl * L::TAB;      // reversed table of the wave's head / scale
  float* s_dtab = s_lds + HP * L::TAB;      // bias gradients of the heads [HP][T]
  char* s_base = reinterpret_cast<char*>(s_lds);
  char* s_unit = s_base + L::OFF_UNIT;      // [slice][head][tile] blocks of 1 KB
  auto block = [&](int sl, int t) { return s_unit + ((sl * HP + hl) * NT + t) * BLOCK; };
  // byte offset of 16-byte part `part` of in-tile token u in a 1 KB block:
  // the part is XORed with bits 1-2 of the token, so that the tokens 4
  // apart that a lane group reads together sit in different banks
  auto uchunk = [&](int u, int part) {
    return 64 * u + 16 * (part ^ ((u >> 1) & 3));
  };
  // P and dS of the wave's head, query tile iq and key tile jk: [query 16][key 16] bf16
  auto pblock = [&](int off, int iq, int jk) {
    return s_base + off + hl * L::PHEAD + (iq * NT + jk) * L::PBLK;
  };
  // byte offset of the 8-byte chunk (query row, key group kg) of a block:
  // the key group is XORed with bits 2-3 of the row, so that the 16 rows a
  // lane group writes (32 bytes apart) spread over the banks; the 16 chunks
  // a lane group reads back (4 whole rows) stay one contiguous 128 bytes
  auto pchunk = [&](int row, int kg) {
    return 32 * row + 8 * (kg ^ ((row >> 2) & 3));
  };

  const unsigned Cb = (unsigned)nh * kHeadDim * 2;  // bytes of one q (k, v, dO) row
  const char* in = static_cast<const char*>(p.qkv);
  const char* gin = static_cast<const char*>(p.dout);
  const float scale = p.scale;
  // non-temporal stores (2), except for 9-tile windows, whose one-head
  // workgroups write 64-byte halves of lines: plain stores let L2 join the
  // halves of a line (192.9 against 196.8 us at window 12; at window 7 the
  // one-head path is faster with non-temporal stores, 50.3 against 52.6)
  constexpr int kStorePolicy = NT > 4 ? 0 : 2;
  // gradients leave through raw buffer stores that every lane issues: the
  // lanes of padded tokens aim past the end of the buffer, where the
  // hardware drops the write.  With no branch around the stores, the wait
  // for the next window's loads does not also wait for them to complete.
  const __amdgpu_buffer_rsrc_t out_rs =
      __builtin_amdgcn_make_buffer_rsrc(p.dqkv, 0, (int)p.dqkv_bytes, 0x00020000);
  auto store16 = [&](bool valid, unsigned off, const bf16x8& v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), out_rs,
                                           valid ? (int)off : (int)0xFFFFFFF0u, 0, kStorePolicy);
  };

  // this workgroup's heads and run of windows: workgroup id -> (XCD x, slot
  // k) (workgroups are dealt to the XCDs round-robin).  Mode 1: the nh/HP
  // head groups of run 8 (k / groups) + x are slots groups (k / groups) ..
  // + groups-1 of XCD x.  Mode 2 (one head per workgroup, even head count):
  // slots 2j and 2j+1 of XCD x hold heads 2i and 2i+1 (whose 64-byte rows
  // share the 128-byte lines of a token) of one run, pair unit 8j + x = run
  // * nh/2 + i; only pairs of heads need to meet in one L2, so every run
  // need not fit on one XCD and the grid fills the chip more evenly
  const int groups = nh / HP;
  int grp, run;
  const int id = blockIdx.x;
  if (p.xcd_streams == 2) {
    const int k = id >> 3, npairs = nh >> 1;
    const int pu = (k >> 1) * 8 + (id & 7);
    if (pu >= p.runs * npairs) return;  // idle workgroups of the last slots
    run = pu / npairs;
    grp = 2 * (pu - run * npairs) + (k & 1);
  } else if (p.xcd_streams) {
    const int k = id >> 3;
    grp = k % groups;
    run = (k / groups) * 8 + (id & 7);
  } else {
    grp = id % groups;
    run = id / groups;
  }
  const int h0 = grp * HP;       // first head of the workgroup
  const int head = h0 + hl;      // head of the wave
  const int runs = p.runs;
  const int w_lo = (int)((long long)run * p.windows / runs);
  const int w_hi = (int)((long long)(run + 1) * p.windows / runs);

  for (int e = tid; e < HP * L::TAB; e += blockDim.x) {
    const int eh = e / L::TAB, k = e - eh * L::TAB;
    s_lds[e] = k < T ? p.table[(T - 1 - k) * nh + h0 + eh] * p.inv_scale : 0.f;
  }
  for (int e = tid; e < HP * T; e += blockDim.x) s_dtab[e] = 0.f;

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
  // tile tw of each slice of the wave's head: one token address per lane
  using Regs = u32x4[SLICES];
  auto issue = [&](Regs& R, const Pos& q) {
    if (tw < NT) {
      int uy, ux;
      btile_token<M>(tw, cq, uy, ux);
      const bool uok = uy < M && ux < M;
      const unsigned pix = bwd_pixel(p, M, q.b, q.wy, q.wx, uy, ux, uok);
      const unsigned hoff = (unsigned)head * kHeadDim * 2 + 16u * gq;
      const char* src = in + pix * (3u * Cb) + hoff;
#pragma unroll
      for (int sl = 0; sl < 3; ++sl) R[sl] = *reinterpret_cast<const u32x4*>(src + sl * Cb);
      R[3] = *reinterpret_cast<const u32x4*>(gin + pix * Cb + hoff);
    }
  };
  auto write = [&](const Regs& R) {
    if (tw < NT) {
#pragma unroll
      for (int sl = 0; sl < SLICES; ++sl)
        *reinterpret_cast<u32x4*>(block(sl, tw) + uchunk(lane >> 2, lane & 3)) = R[sl];
    }
  };
  const bool g_ok = g < S::LG;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};

  // local label of shifted-frame position (yy, xx) of a masked window
  auto local_label = [&](int yy, int xx) {
    return 2 * (yy >= p.H - p.shift) + (xx >= p.W - p.shift);
  };
  auto mask_key = [&](int loc) {  // [label == g] x_s
    bf16x8 a = {};
#pragma unroll
    for (int k = 0; k < 3; ++k) a[k] = loc == g ? (__bf16)p.mask_pieces[k] : (__bf16)0.f;
    return a;
  };
  auto mask_query = [&](int loc) {  // [label == g] - 1
    bf16x8 a = {};
#pragma unroll
    for (int k = 0; k < 3; ++k) a[k] = loc == g ? (__bf16)0.f : (__bf16)-1.f;
    return a;
  };
  // 16 bytes of token u (MFMA layout lane) of tile t of slice sl
  auto tok16 = [&](int sl, int t) {
    return *reinterpret_cast<const bf16x8*>(block(sl, t) + uchunk(c, g));
  };
  // transposing read of tile t of slice sl, channel half hf: element k of
  // lane (g, i) is channel out_channel(hf, i) of in-tile token 4g + k
  auto tile_t = [&](int sl, int t, int hf) {
    return lds_read_tr(block(sl, t) + uchunk(lane >> 2, lane & 3) + 8 * hf);
  };
  // 8 consecutive channels of a lane, from two accumulator tiles
  auto pack8 = [&](const f32x4& lo, const f32x4& hi, float mul) {
    bf16x8 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      o[r] = (__bf16)(lo[r] * mul);
      o[4 + r] = (__bf16)(hi[r] * mul);
    }
    return o;
  };
  // head pairs: gradient tile of tile t in LDS ([16 tokens][128 B], this
  // head's half at chunks 4 hl .. 4 hl + 3), written by both heads' waves of
  // tile t.  16-byte chunk k of token row u sits at chunk k ^ (u & 7) of the
  // row, so that the 16 tokens a lane group writes (rows 128 bytes apart)
  // fall in different banks
  auto swz = [&](int u, int k) { return k ^ (u & 7); };
  auto stage_put = [&](char* st, const bf16x8& v) {
    *reinterpret_cast<bf16x8*>(st + c * 128 + 16 * swz(c, 4 * hl + g)) = v;
  };
  // ... and read back by this wave as whole lines: tokens 8 hl .. 8 hl + 7
  // of tile t, 8 lanes per token, to the slice at byte offset `slice` of a
  // token row
  auto stage_store = [&](const char* st, const Pos& pos, unsigned slice) {
    const int u = 8 * hl + (lane >> 3);
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(st + u * 128 + 16 * swz(u, lane & 7));
    int uy, ux;
    btile_token<M>(tw, u, uy, ux);
    const bool uok = uy < M && ux < M;
    const unsigned pix = bwd_pixel(p, M, pos.b, pos.wy, pos.wx, uy, ux, uok);
    store16(uok, pix * (3u * Cb) + slice + (unsigned)h0 * kHeadDim * 2 + 16 * (lane & 7), v);
  };

  // phase-1 lane geometry: query token c of tile tw; its slot (jt, r) is
  // key token 4g + r of tile jt, table row rbase - E(jt) - r
  int ty, tx;
  btile_token<M>(tw < NT ? tw : 0, c, ty, tx);
  const bool ok = ty < M && tx < M;
  const int qbase = T - 1 - S::C0 - (ok ? S::D * ty + tx : 0) + S::D * g;
  const int rbase = T - 1 - qbase;
  f32x4 dta[NT];  // fp32 dS of each slot summed over the windows
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) dta[jt] = z;

  // ---- phase 1: query tile it = tw; returns the lane's dQ ------------------
  auto phase1 = [&](const Pos& pos, bool masked) -> bf16x8 {
    const int it = tw;
    const bf16x8 q = tok16(0, it), go = tok16(3, it);
    bf16x8 mq = {};
    if (masked) mq = mask_query(local_label(pos.wy * M + ty, pos.wx * M + tx));
    // 9-tile windows recompute each dP tile (one MFMA) where it is needed
    // instead of holding all of them next to the scores (36 VGPRs)
    constexpr bool HOLD_DP = NT <= 4;
    f32x4 sc[NT], dp[HOLD_DP ? NT : 1];
    // the window's mask flag is tested once, outside the tile loop: with
    // no branch between tiles, the LDS reads of one tile are issued while
    // the products of the previous ones run
    // 9-tile windows: one base register for the bias reads, opaque to the
    // compiler, so that it keeps the table constants in the base and the
    // key offsets E(jt) + r (at most 195 words) in the immediate offsets of
    // paired reads instead of an address add per read (for head pairs of
    // 4-tile windows it cost registers: 130 instead of 118, one workgroup
    // per CU fewer)
    int qb = qbase;
    if constexpr (NT > 4) asm("" : "+v"(qb));
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
          float v = s_brev[qb + S::E(jt) + r];
          if (!S::rows_all(jt)) v = g_ok ? v : -__builtin_inff();
          acc[r] = v;
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tok16(1, jt), q, acc, 0, 0, 0);
        if constexpr (MASKED) {
          // key-side operand of this lane: key row (jt, 4g + r) is owned by
          // lane group g, the key token is the lane's own token c of tile jt
          int ky, kx;
          btile_token<M>(jt, c, ky, kx);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              mask_key(local_label(pos.wy * M + ky, pos.wx * M + kx)), mq, acc, 0, 0, 0);
        }
        sc[jt] = acc;
        if constexpr (HOLD_DP)
          dp[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tok16(2, jt), go, z, 0, 0, 0);
      }
    };
    if (masked) score_tiles(std::true_type{});
    else score_tiles(std::false_type{});
    // dP tile jt of the lane's query: V_jt dO^T.  The recomputing path's
    // second pass reads the value tiles through a lane offset the compiler
    // cannot see through (one opaque copy per window, so the reads of both
    // passes still schedule freely), so that the two reads and their
    // products are not merged back into nine held tiles.
    const int voff0 = uchunk(c, g);
    int voff1 = voff0;
    if constexpr (!HOLD_DP) asm("" : "+v"(voff1));
    auto dp_tile = [&](int jt, int pass) -> f32x4 {
      if constexpr (HOLD_DP) {
        return dp[jt];
      } else {
        const bf16x8 v =
            *reinterpret_cast<const bf16x8*>(block(2, jt) + (pass == 0 ? voff0 : voff1));
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, go, z, 0, 0, 0);
      }
    };
    // exact softmax in fp32: the max, then e = exp2 about it, its sum l and
    // sum(e dP) in the same pass, so that D = sum(e dP) / l needs no pass of
    // its own (the value tiles are read while the exponentials run)
    float m = -__builtin_inff();
#pragma unroll
    for (int jt = 0; jt < NT; ++jt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (S::col_ok(jt, r)) m = fmaxf(m, sc[jt][r]);
    m = max_groups(m) * p.score_scale;
    float sum = 0.f, dsum = 0.f;
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
      const f32x4 d = dp_tile(jt, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = S::col_ok(jt, r) ? fast_exp2(fmaf(sc[jt][r], p.score_scale, -m)) : 0.f;
        sc[jt][r] = e;
        sum += e;
        dsum += e * d[r];
      }
    }
    sum = sum_groups(sum);
    // padded queries: P = 0, so their dS, P and dQ vanish
    const float inv = ok ? fast_rcp(sum) : 0.f;
    const float Dq = sum_groups(dsum) * inv;
    // dS^T = P o (dP^T - D): fp32 into the table sums; bf16 as the B
    // operand of the key contraction and, with P, into the LDS blocks.
    // dQ^T = K^T dS^T is accumulated as soon as a pair of key tiles has its
    // dS^T, so that only one B operand is live; K^T comes from transposing
    // reads (odd tile counts: any finite data for the missing tile, its dS^T
    // is zero)
    f32x4 o0 = z, o1 = z;
    bf16x8 pb = {};
    // second-pass dP: the value tile of key tile jt + 1 is read before the
    // products of tile jt
    auto vtile = [&](int jt) {
      return *reinterpret_cast<const bf16x8*>(block(2, jt) + voff1);
    };
    bf16x8 vnext = {};
    if constexpr (!HOLD_DP) vnext = vtile(0);
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
      f32x4 d;
      if constexpr (HOLD_DP) {
        d = dp[jt];
      } else {
        const bf16x8 vcur = vnext;
        if (jt + 1 < NT) vnext = vtile(jt + 1);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vcur, go, z, 0, 0, 0);
      }
      bf16x4 pt, st;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pr = sc[jt][r] * inv;
        const float ds = pr * (d[r] - Dq);
        dta[jt][r] += ds;
        st[r] = (__bf16)ds;
        pt[r] = (__bf16)pr;
        pb[4 * (jt % 2) + r] = st[r];
      }
      // P[query c][keys 4g .. 4g+3] of block (it, jt)
      *reinterpret_cast<bf16x4*>(pblock(L::OFF_P, it, jt) + pchunk(c, g)) = pt;
      *reinterpret_cast<bf16x4*>(pblock(L::OFF_DS, it, jt) + pchunk(c, g)) = st;
      if (jt % 2 == 1 || jt == NT - 1) {
        const int kk = jt / 2;
        if (jt % 2 == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) pb[4 + r] = (__bf16)0.f;
        }
        const int t1 = 2 * kk + 1 < NT ? 2 * kk + 1 : 2 * kk;
        const bf16x8 k0 = __builtin_shufflevector(tile_t(1, 2 * kk, 0), tile_t(1, t1, 0), 0, 1, 2,
                                                  3, 4, 5, 6, 7);
        const bf16x8 k1 = __builtin_shufflevector(tile_t(1, 2 * kk, 1), tile_t(1, t1, 1), 0, 1, 2,
                                                  3, 4, 5, 6, 7);
        o0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, pb, o0, 0, 0, 0);
        o1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, pb, o1, 0, 0, 0);
      }
    }
    return pack8(o0, o1, scale);
  };

  // ---- phase 2: key tile jk = tw; dK and dV of the lane's key -----------------
  auto phase2 = [&](bf16x8& dk, bf16x8& dv) {
    const int jk = tw;
    f32x4 dk0 = z, dk1 = z, dv0 = z, dv1 = z;
    if constexpr (HP == 2) {
      // head pairs (two workgroups of 8 waves per CU): reads and products
      // in source order; the pipelined form below was slower here (Swin-L
      // stage 1: 125.3 against 123.5 us)
#pragma unroll
      for (int iq = 0; iq < NT; ++iq) {
        const bf16x4 pb = lds_read_tr(pblock(L::OFF_P, iq, jk) + pchunk(lane >> 2, lane & 3));
        const bf16x4 sb = lds_read_tr(pblock(L::OFF_DS, iq, jk) + pchunk(lane >> 2, lane & 3));
        dv0 = mfma16(tile_t(3, iq, 0), pb, dv0);
        dv1 = mfma16(tile_t(3, iq, 1), pb, dv1);
        dk0 = mfma16(tile_t(0, iq, 0), sb, dk0);
        dk1 = mfma16(tile_t(0, iq, 1), sb, dk1);
      }
    } else {
      // the six operands of query tile iq: P and dS (element k of lane (g, c):
      // query 4g + k of tile iq, key c), dO^T and Q^T halves
      struct Ops {
        bf16x4 pb, sb, o0, o1, q0, q1;
      };
      auto fetch = [&](int iq) {
        Ops o;
        o.pb = lds_read_tr(pblock(L::OFF_P, iq, jk) + pchunk(lane >> 2, lane & 3));
        o.sb = lds_read_tr(pblock(L::OFF_DS, iq, jk) + pchunk(lane >> 2, lane & 3));
        o.o0 = tile_t(3, iq, 0);
        o.o1 = tile_t(3, iq, 1);
        o.q0 = tile_t(0, iq, 0);
        o.q1 = tile_t(0, iq, 1);
        return o;
      };
      // software pipeline: the reads of tile iq + 1 are issued before the
      // products of tile iq, so each product waits for reads issued one step
      // earlier (the scheduling groups keep that order)
      Ops cur = fetch(0);
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
      for (int iq = 0; iq < NT; ++iq) {
        Ops nxt = cur;
        if (iq + 1 < NT) {
          nxt = fetch(iq + 1);
          __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
        }
        dv0 = mfma16(cur.o0, cur.pb, dv0);
        dv1 = mfma16(cur.o1, cur.pb, dv1);
        dk0 = mfma16(cur.q0, cur.sb, dk0);
        dk1 = mfma16(cur.q1, cur.sb, dk1);
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        cur = nxt;
      }
    }
    dk = pack8(dk0, dk1, scale);
    dv = pack8(dv0, dv1, 1.f);
  };
  // this lane's own token (MFMA layout) of tile tw: image offset of its row
  auto own_row = [&](const Pos& pos, bool& vok) {
    int uy, ux;
    btile_token<M>(tw, c, uy, ux);
    vok = uy < M && ux < M;
    return bwd_pixel(p, M, pos.b, pos.wy, pos.wx, uy, ux, vok) * (3u * Cb) +
           (unsigned)head * kHeadDim * 2 + 16 * g;
  };

  // walk over the run's windows, the next window's loads in flight while a
  // window is computed; they go to LDS at the end of the iteration, after
  // the window's stores were issued
  Regs R;
  if (w_lo < w_hi) {
    issue(R, decode(w_lo));
    write(R);
  }
  __syncthreads();  // tables and first unit staged
  for (int bw = w_lo; bw < w_hi; ++bw) {
    const Pos cur = decode(bw);
    if (bw + 1 < w_hi) {
      // the loads leave ahead of the other waves' math on the SIMD
      __builtin_amdgcn_s_setprio(3);
      issue(R, decode(bw + 1));
      __builtin_amdgcn_s_setprio(0);
    }
    bf16x8 dq = {}, dk = {}, dv = {};
    if (tw < NT) dq = phase1(cur, window_masked(p.shift, cur.wy, cur.wx, p.nWy, p.nWx));
    if constexpr (HP == 1) {
      bool vok;
      const unsigned row = own_row(cur, vok);
      if (tw < NT) store16(vok, row, dq);
      __syncthreads();  // P and dS blocks visible
      if (tw < NT) {
        phase2(dk, dv);
        store16(vok, row + Cb, dk);
        store16(vok, row + 2 * Cb, dv);
      }
      __syncthreads();  // every wave is done with the unit before it is overwritten
    } else {
      // dQ tile of tile tw: 2 KB of the k tiles of both heads (slice 1)
      char* st_q = s_unit + (1 * HP * NT) * BLOCK + tw * 2 * BLOCK;
      __syncthreads();  // P and dS blocks visible; the k tiles are free
      stage_put(st_q, dq);
      phase2(dk, dv);
      __syncthreads();  // dQ tiles complete; P and dS blocks are free
      char* st_k = s_base + L::OFF_P + tw * 2 * BLOCK;  // dK tiles, then dV tiles
      char* st_v = st_k + NT * 2 * BLOCK;
      stage_put(st_k, dk);
      stage_put(st_v, dv);
      stage_store(st_q, cur, 0);
      __syncthreads();  // dK and dV tiles complete
      stage_store(st_k, cur, Cb);
      stage_store(st_v, cur, 2 * Cb);
    }
    write(R);         // after the last window: stale data, never read
    __syncthreads();  // next unit visible to every wave
  }
  // this workgroup's bias gradients -> LDS -> HBM
  if (tw < NT && ok) {
#pragma unroll
    for (int jt = 0; jt < NT; ++jt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (S::col_ok(jt, r) && (S::rows_all(jt) || g_ok))
          atomicAdd(&s_dtab[hl * T + rbase - S::E(jt) - r], dta[jt][r]);
  }
  __syncthreads();
  for (int e = tid; e < HP * T; e += blockDim.x) {
    const float v = s_dtab[e];
    const int eh = e / T, k = e - eh * T;
    if (v != 0.f) atomicAdd(p.dtable + k * nh + h0 + eh, v);
  }
}

template <int M, int HP>
int bwd_blocks_per_cu(int dev, size_t lds) {
  static std::atomic<long long> cache[kMaxDevices];
  const bool cacheable = dev >= 0 && dev < kMaxDevices;
  if (cacheable) {
    const long long v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0 && (size_t)(v >> 8) == lds) return (int)(v & 255);
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, wattn_bwd_bf16_kernel<M, HP>,
                                                   bwd_waves<M>() * 64 * HP, lds) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  if (per_cu > 255) per_cu = 255;
  if (cacheable) cache[dev].store(((long long)lds << 8) | per_cu, std::memory_order_relaxed);
  return per_cu;
}

// Grid: nh / HP workgroups (one per head group) per run of windows, as many
// runs as the chip holds at the kernel's occupancy (at most one per
// window); with 8 runs or more, a multiple of 8 runs, laid out per XCD.
struct BwdPlan {
  long long grid;
  int runs, xcd_streams;
};

template <int M, int HP>
BwdPlan plan_bwd(const BwdParams& p, int dev, int cus) {
  const int groups = p.nh / HP;
  const long long slots = (long long)cus * bwd_blocks_per_cu<M, HP>(dev, BwdLds<M, HP>::BYTES);
  long long runs = slots / groups;
  if (runs > p.windows) runs = p.windows;
  // at least kMinRunWindows windows per run: each workgroup adds its table
  // gradient to HBM once with global atomics, and short runs make those adds
  // (and the per-workgroup setup) a large share of a small launch (Swin-T
  // stage 3: 45.2 -> 40.7 us, stage 1: 50.4 -> 46.0 us; 16 windows per run
  // was slower, 55.0 us on stage 3, and 4 windows too, 43.9 us)
  if (runs > p.windows / kMinRunWindows) runs = p.windows / kMinRunWindows;
  if (runs < 1) runs = 1;
  BwdPlan pl;
  pl.xcd_streams = runs >= 8 ? 1 : 0;
  if (pl.xcd_streams) runs -= runs % 8;
  pl.grid = runs * groups;
  // one head per workgroup and an even head count: place pairs of heads,
  // not whole runs, on one XCD (window 12, 6 heads: 42 runs on 252 of 256
  // CUs instead of 40 runs on 240)
  if (HP == 1 && p.nh % 2 == 0 && slots % 16 == 0) {
    const long long npairs = p.nh / 2;
    long long r2 = (slots / 2) / npairs;
    if (r2 > p.windows / kMinRunWindows) r2 = p.windows / kMinRunWindows;
    if (r2 >= 8 && r2 > runs) {
      runs = r2;
      pl.xcd_streams = 2;
      pl.grid = 16 * ((runs * npairs - 1) / 8 + 1);
    }
  }
  pl.runs = (int)runs;  // at most the window count
  return pl;
}

template <int M, int HP>
hipError_t launch_bwd_mh(const BwdParams& p_in, const BwdPlan& pl, hipStream_t st) {
  if (pl.grid > 0x7fffffffLL) return hipErrorInvalidValue;
  BwdParams p = p_in;
  p.runs = pl.runs;
  p.xcd_streams = pl.xcd_streams;
  hipLaunchKernelGGL((wattn_bwd_bf16_kernel<M, HP>), dim3((unsigned)pl.grid),
                     dim3(bwd_waves<M>() * 64 * HP), (BwdLds<M, HP>::BYTES), st, p);
  return hipGetLastError();
}

// head pairs for 4-tile windows (5..8) when the head count is even and the
// pairs' grid covers every CU; a smaller grid takes one head per workgroup,
// twice the workgroups (Swin-T stage 3, 12 heads, 256 windows: 192 head-pair
// workgroups took 40.3 us, 384 one-head workgroups 32.1 us)
template <int M>
hipError_t launch_bwd_m(const BwdParams& p, int dev, int cus, hipStream_t st) {
  if constexpr (Win<M>::NT == 4) {
    if (p.nh % 2 == 0) {
      const BwdPlan pl = plan_bwd<M, 2>(p, dev, cus);
      if (pl.grid >= cus) return launch_bwd_mh<M, 2>(p, pl, st);
    }
  }
  return launch_bwd_mh<M, 1>(p, plan_bwd<M, 1>(p, dev, cus), st);
}

template <int M>
size_t bwd_lds_m() {
  if constexpr (Win<M>::NT == 4) return BwdLds<M, 2>::BYTES;
  return BwdLds<M, 1>::BYTES;
}

__global__ void fill_kernel(float* dst, long long n, float v) {
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (long long)gridDim.x * blockDim.x)
    dst[e] = v;
}

}  // namespace

size_t bwd_lds_bytes(int M) {
  switch (M) {
    case 1: return bwd_lds_m<1>();
    case 2: return bwd_lds_m<2>();
    case 3: return bwd_lds_m<3>();
    case 4: return bwd_lds_m<4>();
    case 5: return bwd_lds_m<5>();
    case 6: return bwd_lds_m<6>();
    case 7: return bwd_lds_m<7>();
    case 8: return bwd_lds_m<8>();
    case 9: return bwd_lds_m<9>();
    case 10: return bwd_lds_m<10>();
    case 11: return bwd_lds_m<11>();
    case 12: return bwd_lds_m<12>();
    default: return 0;
  }
}

hipError_t launch_fill(float* dst, long long n, float v, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, dst, n, v);
  return hipGetLastError();
}

hipError_t launch_bwd_bf16(int M, const BwdParams& p, int dev, int cus, hipStream_t stream) {
  switch (M) {
    case 1: return launch_bwd_m<1>(p, dev, cus, stream);
    case 2: return launch_bwd_m<2>(p, dev, cus, stream);
    case 3: return launch_bwd_m<3>(p, dev, cus, stream);
    case 4: return launch_bwd_m<4>(p, dev, cus, stream);
    case 5: return launch_bwd_m<5>(p, dev, cus, stream);
    case 6: return launch_bwd_m<6>(p, dev, cus, stream);
    case 7: return launch_bwd_m<7>(p, dev, cus, stream);
    case 8: return launch_bwd_m<8>(p, dev, cus, stream);
    case 9: return launch_bwd_m<9>(p, dev, cus, stream);
    case 10: return launch_bwd_m<10>(p, dev, cus, stream);
    case 11: return launch_bwd_m<11>(p, dev, cus, stream);
    case 12: return launch_bwd_m<12>(p, dev, cus, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace swinattn
