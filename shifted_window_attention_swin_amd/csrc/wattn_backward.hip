// Backward of the fused shifted-window attention (bf16, windows up to 8:
// 1 or 4 tiles of 16 tokens), for training.  The NVIDIA talk "Swin
// Transformer training and inference optimization" (uticex.com 1598),
// section 2, fuses the window attention's backward as it fuses the forward.
//
// Per window and head, with S = Q K^T / sqrt(d) + bias + mask, P = softmax(S)
// and dO the output gradient gathered through the same shift and partition:
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,  dS = P o (dP - D),
//   dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d),  dtable[rel(i,j)] += dS_ij.
//
//   unit      (image, window, head): q, k, v and dO of the head, each 16-token
//             tile a 1 KB LDS block (16 tokens x 64 B), staged like the
//             forward's (register prefetch of the next unit).
//   streams   a workgroup keeps one head and walks a contiguous run of
//             windows; the nh workgroups of one run (its nh heads) sit on
//             one XCD and walk it in step, so the 128-byte lines that hold
//             two heads of a token are fetched into one L2.
//   phase 1   one wave per query tile, in the forward's transposed layout
//             (keys in a lane's accumulator rows, queries across lanes):
//             S^T and P (fp32, exact softmax), dP^T = V dO^T, D, dS^T, and
//             dQ^T = K^T dS^T (K^T from transposing LDS reads, as the
//             forward's V^T).  P and dS go to LDS in bf16 as 16 x 16 blocks
//             [query][key], one per (query tile, key tile).
//   phase 2   one wave per key tile: dV^T += dO^T P and dK^T += Q^T dS on
//             16x16x16 MFMAs, their B operands read out of the P and dS
//             blocks with transposing LDS reads (4 queries of a key per
//             lane), dO^T and Q^T from transposing reads of the unit.
//   bias grad the (query, key) pair of a phase-1 accumulator slot of a lane
//             is the same in every window, hence so is its table row: each
//             lane sums the fp32 dS of its 16 slots in registers over all its
//             workgroup's windows (one head), then adds them once into an
//             LDS copy of the head's table gradient (LDS atomics), which goes
//             to HBM with global atomics.
//   output    dQ, dK, dV of a token leave as 16-byte stores of 8 channels.

#include <atomic>

#include "bwd_internal.h"
#include "wattn_common.h"

namespace swinattn {
namespace {

constexpr int kBwdWaves = 4;

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

// bias table of head h -> LDS, divided by the score scale and reversed
// (rows T-1 .. 0), then a zero tail that padded keys may read
template <int M>
SWA_INLINE void stage_head_table(float* s_rev, const float* table, int nh, int h,
                                 float inv_scale) {
  using S = Win<M>;
  for (int e = threadIdx.x; e < S::T + S::TAIL; e += blockDim.x)
    s_rev[e] = e < S::T ? table[(S::T - 1 - e) * nh + h] * inv_scale : 0.f;
}

template <int M>
struct BwdLds {
  using S = Win<M>;
  static constexpr int UNIT = 4 * S::NT * 1024;           // q, k, v, dO tiles
  static constexpr int PBLK = 512;                         // 16 x 16 bf16
  static constexpr int OFF_UNIT = ((2 * S::T + S::TAIL) * 4 + 15) / 16 * 16;
  static constexpr int OFF_P = OFF_UNIT + UNIT;
  static constexpr int OFF_DS = OFF_P + S::NT * S::NT * PBLK;
  static constexpr int BYTES = OFF_DS + S::NT * S::NT * PBLK;
};

template <int M>
__global__ __launch_bounds__(kBwdWaves * 64) void wattn_bwd_bf16_kernel(BwdParams p) {
  using S = Win<M>;
  using L = BwdLds<M>;
  constexpr int NT = S::NT, NK = S::NK, T = S::T;
  static_assert(NT <= kBwdWaves, "one wave per tile");
  constexpr int BLOCK = 1024;
  constexpr int SLICES = 4;  // q, k, v, dO
  extern __shared__ float s_lds[];
  const int nh = p.nh;
  float* s_brev = s_lds;               // reversed table of the head / scale [T + TAIL]
  float* s_dtab = s_brev + T + S::TAIL;  // bias gradient of the head [T]
  char* s_base = reinterpret_cast<char*>(s_lds);
  char* s_unit = s_base + L::OFF_UNIT;   // 4 slices x NT blocks of 1 KB
  auto block = [&](int sl, int t) { return s_unit + (sl * NT + t) * BLOCK; };
  // P and dS of query tile iq and key tile jk: [query 16][key 16] bf16
  auto pblock = [&](int off, int iq, int jk) { return s_base + off + (iq * NT + jk) * L::PBLK; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wv >= 0 && wv < kBwdWaves);
  const int gq = lane & 3, cq = lane >> 2;  // load layout: 16-byte part, token
  const int g = lane >> 4, c = lane & 15;   // MFMA layout: lane group, token
  const unsigned Cb = (unsigned)nh * kHeadDim * 2;  // bytes of one q (k, v, dO) row
  const char* in = static_cast<const char*>(p.qkv);
  const char* gin = static_cast<const char*>(p.dout);
  const float scale = p.scale;
  // gradients leave through raw buffer stores that every lane issues: the
  // lanes of padded tokens aim past the end of the buffer, where the
  // hardware drops the write.  With no branch around the stores, the wait
  // for the next window's loads does not also wait for them to complete.
  const __amdgpu_buffer_rsrc_t out_rs =
      __builtin_amdgcn_make_buffer_rsrc(p.dqkv, 0, (int)p.dqkv_bytes, 0x00020000);
  auto store16 = [&](bool valid, unsigned off, const bf16x8& v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), out_rs,
                                           valid ? (int)off : (int)0xFFFFFFF0u, 0, 2 /* nt */);
  };

  // this workgroup's head and run of windows: workgroup id -> (XCD x, slot
  // k); the nh heads of run 8 (k / nh) + x are slots nh (k / nh) .. + nh-1
  // of XCD x (workgroups are dealt to the XCDs round-robin)
  int head, run;
  const int id = blockIdx.x;
  if (p.xcd_streams) {
    const int k = id >> 3;
    head = k % nh;
    run = (k / nh) * 8 + (id & 7);
  } else {
    head = id % nh;
    run = id / nh;
  }
  const int runs = gridDim.x / nh;
  const int w_lo = (int)((long long)run * p.windows / runs);
  const int w_hi = (int)((long long)(run + 1) * p.windows / runs);

  stage_head_table<M>(s_brev, p.table, nh, head, p.inv_scale);
  for (int e = tid; e < T; e += blockDim.x) s_dtab[e] = 0.f;

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
  // tile wv of each slice: one token address per lane
  using Regs = u32x4[SLICES];
  auto issue = [&](Regs& R, const Pos& q) {
    if (wv < NT) {
      int ty, tx;
      btile_token<M>(wv, cq, ty, tx);
      const bool ok = ty < M && tx < M;
      const unsigned pix = bwd_pixel(p, M, q.b, q.wy, q.wx, ty, tx, ok);
      const char* src = in + pix * (3u * Cb) + (unsigned)head * kHeadDim * 2 + 16u * gq;
#pragma unroll
      for (int sl = 0; sl < 3; ++sl) R[sl] = *reinterpret_cast<const u32x4*>(src + sl * Cb);
      R[3] = *reinterpret_cast<const u32x4*>(gin + pix * Cb + (unsigned)head * kHeadDim * 2 + 16u * gq);
    }
  };
  auto write = [&](const Regs& R) {
    if (wv < NT) {
#pragma unroll
      for (int sl = 0; sl < SLICES; ++sl)
        *reinterpret_cast<u32x4*>(block(sl, wv) + lane * 16) = R[sl];
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
    return *reinterpret_cast<const bf16x8*>(block(sl, t) + (4 * c + g) * 16);
  };
  // transposing read of tile t of slice sl, channel half hf: element k of
  // lane (g, i) is channel out_channel(hf, i) of in-tile token 4g + k
  auto tile_t = [&](int sl, int t, int hf) { return lds_read_tr(block(sl, t) + lane * 16 + 8 * hf); };
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

  // phase-1 lane geometry: query token c of tile wv; its slot (jt, r) is
  // key token 4g + r of tile jt, table row rbase - E(jt) - r
  int ty, tx;
  btile_token<M>(wv < NT ? wv : 0, c, ty, tx);
  const bool ok = ty < M && tx < M;
  const int qbase = T - 1 - S::C0 - (ok ? S::D * ty + tx : 0) + S::D * g;
  const int rbase = T - 1 - qbase;
  f32x4 dta[NT];  // fp32 dS of each slot summed over the windows
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) dta[jt] = z;

  // ---- phase 1: query tile it = wv -----------------------------------------
  auto phase1 = [&](const Pos& pos, bool masked) {
    const int it = wv;
    if (it >= NT) return;
    const bf16x8 q = tok16(0, it), go = tok16(3, it);
    bf16x8 mq = {};
    if (masked) mq = mask_query(local_label(pos.wy * M + ty, pos.wx * M + tx));
    f32x4 sc[NT], dp[NT];
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
      f32x4 acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (!S::col_ok(jt, r)) {
          acc[r] = -__builtin_inff();
          continue;
        }
        float v = s_brev[qbase + S::E(jt) + r];
        if (!S::rows_all(jt)) v = g_ok ? v : -__builtin_inff();
        acc[r] = v;
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tok16(1, jt), q, acc, 0, 0, 0);
      if (masked) {
        // key-side operand of this lane: key row (jt, 4g + r) is owned by
        // lane group g, the key token is the lane's own token c of tile jt
        int ky, kx;
        btile_token<M>(jt, c, ky, kx);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            mask_key(local_label(pos.wy * M + ky, pos.wx * M + kx)), mq, acc, 0, 0, 0);
      }
      sc[jt] = acc;
      dp[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tok16(2, jt), go, z, 0, 0, 0);
    }
    // exact softmax in fp32: max, then the sum of exp2 about it
    float m = -__builtin_inff();
#pragma unroll
    for (int jt = 0; jt < NT; ++jt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (S::col_ok(jt, r)) m = fmaxf(m, sc[jt][r]);
    m = max_groups(m) * p.score_scale;
    float sum = 0.f;
#pragma unroll
    for (int jt = 0; jt < NT; ++jt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = S::col_ok(jt, r) ? fast_exp2(fmaf(sc[jt][r], p.score_scale, -m)) : 0.f;
        sc[jt][r] = e;
        sum += e;
      }
    sum = sum_groups(sum);
    // padded queries: P = 0, so their dS, P and dQ vanish
    const float inv = ok ? fast_rcp(sum) : 0.f;
    float dsum = 0.f;
#pragma unroll
    for (int jt = 0; jt < NT; ++jt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[jt][r] *= inv;
        dsum += sc[jt][r] * dp[jt][r];
      }
    const float Dq = sum_groups(dsum);
    // dS^T = P o (dP^T - D): fp32 into the table sums; bf16 as the B
    // operand of the key contraction and, with P, into the LDS blocks
    bf16x8 pb[NK];
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
      bf16x4 pt, st;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ds = sc[jt][r] * (dp[jt][r] - Dq);
        dta[jt][r] += ds;
        st[r] = (__bf16)ds;
        pt[r] = (__bf16)sc[jt][r];
        pb[jt / 2][4 * (jt % 2) + r] = st[r];
      }
      // P[query c][keys 4g .. 4g+3] of block (it, jt)
      *reinterpret_cast<bf16x4*>(pblock(L::OFF_P, it, jt) + 32 * c + 8 * g) = pt;
      *reinterpret_cast<bf16x4*>(pblock(L::OFF_DS, it, jt) + 32 * c + 8 * g) = st;
    }
    if constexpr (NT % 2 == 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) pb[NK - 1][4 + r] = (__bf16)0.f;
    }
    // dQ^T = K^T dS^T, K^T from transposing reads (odd tile counts: any
    // finite data for the missing tile, its dS^T is zero)
    f32x4 o0 = z, o1 = z;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const int t1 = 2 * kk + 1 < NT ? 2 * kk + 1 : 2 * kk;
      const bf16x8 k0 = __builtin_shufflevector(tile_t(1, 2 * kk, 0), tile_t(1, t1, 0), 0, 1, 2, 3,
                                                4, 5, 6, 7);
      const bf16x8 k1 = __builtin_shufflevector(tile_t(1, 2 * kk, 1), tile_t(1, t1, 1), 0, 1, 2, 3,
                                                4, 5, 6, 7);
      o0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, pb[kk], o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, pb[kk], o1, 0, 0, 0);
    }
    const unsigned pix = bwd_pixel(p, M, pos.b, pos.wy, pos.wx, ty, tx, ok);
    store16(ok, pix * (3u * Cb) + head * kHeadDim * 2 + 16 * g, pack8(o0, o1, scale));
  };

  // ---- phase 2: key tile jk = wv ------------------------------------------
  auto phase2 = [&](const Pos& pos) {
    const int jk = wv;
    if (jk >= NT) return;
    f32x4 dk0 = z, dk1 = z, dv0 = z, dv1 = z;
#pragma unroll
    for (int iq = 0; iq < NT; ++iq) {
      // element k of lane (g, c): P (dS) of query 4g + k of tile iq, key c
      const bf16x4 pb = lds_read_tr(pblock(L::OFF_P, iq, jk) + 8 * lane);
      const bf16x4 sb = lds_read_tr(pblock(L::OFF_DS, iq, jk) + 8 * lane);
      dv0 = mfma16(tile_t(3, iq, 0), pb, dv0);
      dv1 = mfma16(tile_t(3, iq, 1), pb, dv1);
      dk0 = mfma16(tile_t(0, iq, 0), sb, dk0);
      dk1 = mfma16(tile_t(0, iq, 1), sb, dk1);
    }
    int ky, kx;
    btile_token<M>(jk, c, ky, kx);
    const bool kok = ky < M && kx < M;
    const unsigned pix = bwd_pixel(p, M, pos.b, pos.wy, pos.wx, ky, kx, kok);
    const unsigned dst = pix * (3u * Cb) + head * kHeadDim * 2 + 16 * g;
    store16(kok, dst + Cb, pack8(dk0, dk1, scale));
    store16(kok, dst + 2 * Cb, pack8(dv0, dv1, 1.f));
  };

  // walk over the run's windows, the next window's loads in flight while a
  // window is computed; they go to LDS at the end of the iteration, after
  // the window's stores were issued
  Regs R;
  Pos nxt = decode(w_lo);
  if (w_lo < w_hi) {
    issue(R, nxt);
    write(R);
  }
  __syncthreads();  // table and first unit staged
  for (int bw = w_lo; bw < w_hi; ++bw) {
    const Pos cur = nxt;
    const bool more = bw + 1 < w_hi;
    if (more) {
      nxt = decode(bw + 1);
      issue(R, nxt);
    }
    phase1(cur, window_masked(p.shift, cur.wy, cur.wx, p.nWy, p.nWx));
    __syncthreads();  // P and dS blocks visible
    phase2(cur);
    __syncthreads();  // every wave is done with the unit before it is overwritten
    write(R);         // after the last window: stale data, never read
    __syncthreads();  // next unit visible to every wave
  }
  // this workgroup's bias gradient -> LDS -> HBM
  if (wv < NT && ok) {
#pragma unroll
    for (int jt = 0; jt < NT; ++jt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (S::col_ok(jt, r) && (S::rows_all(jt) || g_ok))
          atomicAdd(&s_dtab[rbase - S::E(jt) - r], dta[jt][r]);
  }
  __syncthreads();
  for (int e = tid; e < T; e += blockDim.x) {
    const float v = s_dtab[e];
    if (v != 0.f) atomicAdd(p.dtable + e * nh + head, v);
  }
}

template <int M>
size_t bwd_lds_m() {
  return BwdLds<M>::BYTES;
}

template <int M>
int bwd_blocks_per_cu(int dev, size_t lds) {
  static std::atomic<long long> cache[kMaxDevices];
  const bool cacheable = dev >= 0 && dev < kMaxDevices;
  if (cacheable) {
    const long long v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0 && (size_t)(v >> 8) == lds) return (int)(v & 255);
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, wattn_bwd_bf16_kernel<M>,
                                                   kBwdWaves * 64, lds) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  if (per_cu > 255) per_cu = 255;
  if (cacheable) cache[dev].store(((long long)lds << 8) | per_cu, std::memory_order_relaxed);
  return per_cu;
}

// Grid: nh workgroups (one per head) per run of windows, as many runs as
// the chip holds at the kernel's occupancy (at most one per window); with 8
// runs or more, a multiple of 8 runs, laid out per XCD.
template <int M>
hipError_t launch_bwd_m(const BwdParams& p_in, int dev, int cus, hipStream_t st) {
  BwdParams p = p_in;
  const size_t lds = bwd_lds_m<M>();
  const long long slots = (long long)cus * bwd_blocks_per_cu<M>(dev, lds);
  long long runs = slots / p.nh;
  if (runs > p.windows) runs = p.windows;
  if (runs < 1) runs = 1;
  p.xcd_streams = runs >= 8 ? 1 : 0;
  if (p.xcd_streams) runs -= runs % 8;
  const long long grid = runs * p.nh;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(wattn_bwd_bf16_kernel<M>, dim3((unsigned)grid), dim3(kBwdWaves * 64), lds, st,
                     p);
  return hipGetLastError();
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
    default: return hipErrorInvalidValue;
  }
}

}  // namespace swinattn
