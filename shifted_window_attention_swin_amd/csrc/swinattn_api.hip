// C-ABI front of libswinattn: argument checks, kernel launches on the
// caller's stream, and the per-device cache of materialised index/mask
// tensors.  The talk "Swin Transformer training and inference optimization"
// (uticex.com 1598, section 3) hoists the bias index lookup to a one-time
// preprocessing step; the forward kernels go one step further and evaluate
// the index and the mask as closed forms of the token coordinates, so the
// forward reads no setup state.  The precompute call builds the tensors for
// callers that want them and for verification.

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/swinattn.h"
#include "bwd_internal.h"
#include "ln_attn_internal.h"
#include "linear_internal.h"
#include "wattn_internal.h"

using namespace swinattn;

namespace {

struct Prepared {
  int dev, H, W, M, s;
  void* block;  // one allocation holding the three arrays below
  int32_t* rel_index;
  float* mask;
  uint8_t* region;
  // recorded on the precompute's stream after its fill: a copy on any other
  // stream waits for it, so it never reads the tensors before they are written
  hipEvent_t ready;
};

std::mutex g_mu;
std::vector<Prepared> g_cache;

// compute units per device, looked up on first use (lock-free: a racing
// first use stores the same value twice)
std::atomic<int> g_cus[kMaxDevices];

int compute_units(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return 256;
  int v = g_cus[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    v = 256;
  g_cus[dev].store(v, std::memory_order_relaxed);
  return v;
}

// heads per unit of the persistent kernel.  Windows of up to 4 tiles: 2
// (each wave then owns one head and two query tiles), else 3, else 1.
// Larger windows: 1 (a unit is already 9 tiles per slice).
int head_group(int heads, int M) {
  if ((M + 3) / 4 > 2) return 1;
  if (heads % 2 == 0) return 2;
  if (heads % 3 == 0) return 3;
  return 1;
}

bool shape_ok(int H, int W, int M, int s) {
  return H > 0 && W > 0 && M >= 1 && M <= kMaxWindow && H % M == 0 && W % M == 0 && s >= 0 &&
         s < M;
}

// caller holds g_mu
Prepared* find(int dev, int H, int W, int M, int s) {
  for (auto& e : g_cache)
    if (e.dev == dev && e.H == H && e.W == W && e.M == M && e.s == s) return &e;
  return nullptr;
}

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// The mask value divided by the score scale (100 / scale), as three bf16
// pieces (each the top 8 significant bits of the remainder); their sum is
// the fp32 value exactly, in any order
void mask_pieces(double value, float (&pieces)[3]) {
  float rest = (float)value;
  for (int k = 0; k < 3; ++k) {
    uint32_t u;
    memcpy(&u, &rest, 4);
    u &= 0xFFFF0000u;
    float piece;
    memcpy(&piece, &u, 4);
    pieces[k] = piece;
    rest -= piece;
  }
}

enum FwdKind { kFwdBf16, kFwdF32, kFwdI8 };

// Scales of int8 codes: the score scale scale_q * scale_k / sqrt(head_dim)
// must lie in [2^-100, 2^100] and scale_v in (0, 2^100], so that every
// constant derived from them (the score scale, its inverse, the mask over
// the score scale) is a normal fp32 number; an int8 output scale (so > 0)
// must keep scale_v / so in [2^-100, 2^100].
bool i8_scales_ok(double sq, double sk, double sv, double so, int head_dim) {
  if (!(sq > 0.0) || !(sk > 0.0) || !(sv > 0.0) || !(sv <= 0x1p100)) return false;
  if (!(so >= 0.0)) return false;
  if (so > 0.0 && !(sv / so >= 0x1p-100 && sv / so <= 0x1p100)) return false;
  const double sc = sq * sk / sqrt((double)head_dim);
  return sc >= 0x1p-100 && sc <= 0x1p100;
}

int fwd_common(const void* qkv, const float* table, void* out, int B, int H, int W, int heads,
               int head_dim, int M, int s, void* stream, FwdKind kind, float sq = 1.f,
               float sk = 1.f, float sv = 1.f, float so = 0.f) {
  if (!qkv || !table || !out) return SWIN_ERR_INVALID_ARG;
  if (!aligned(qkv, 16) || !aligned(out, 16) || !aligned(table, 4)) return SWIN_ERR_INVALID_ARG;
  if (B < 0 || H <= 0 || W <= 0 || heads <= 0 || head_dim <= 0 || M <= 0) return SWIN_ERR_INVALID_ARG;
  if (H % M != 0 || W % M != 0 || s < 0 || s >= M) return SWIN_ERR_INVALID_ARG;
  if (kind == kFwdI8 && !i8_scales_ok(sq, sk, sv, so, head_dim)) return SWIN_ERR_INVALID_ARG;
  if (head_dim != kHeadDim || M > kMaxWindow) return SWIN_ERR_UNSUPPORTED;
  // the fp32 kernel stages every head's bias table in LDS; the persistent
  // kernel stages one head group's when every head's would not fit
  if (kind == kFwdF32 && fwd_lds_bytes(M, heads) > (size_t)kMaxLds) return SWIN_ERR_UNSUPPORTED;
  const long long in_elem = kind == kFwdF32 ? 4 : kind == kFwdI8 ? 1 : 2;
  const long long out_elem = kind == kFwdF32 ? 4 : (kind == kFwdI8 && so > 0.f) ? 1 : 2;
  const long long nW = (long long)(H / M) * (W / M);
  const long long C = (long long)heads * head_dim;
  const long long image_bytes = (long long)H * W * 3 * C * in_elem;
  const long long out_image_bytes = (long long)H * W * C * out_elem;
  const long long max_image = image_bytes > out_image_bytes ? image_bytes : out_image_bytes;
  if (max_image > kMaxChunkBytes) return SWIN_ERR_UNSUPPORTED;
  const long long tokens = (long long)B * H * W;
  if (overlap(qkv, (size_t)(tokens * 3 * C * in_elem), out, (size_t)(tokens * C * out_elem)))
    return SWIN_ERR_INVALID_ARG;
  if (B == 0) return SWIN_OK;

  // the relative position index and the shift mask are closed forms of the
  // token coordinates, evaluated in the kernels: no setup state is read
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SWIN_ERR_HIP;
  FwdParams p;
  p.table = table;
  p.H = H;
  p.W = W;
  p.nh = heads;
  p.shift = s;
  p.nWy = H / M;
  p.nWx = W / M;
  p.nW = (int)nW;
  const double sd = sqrt((double)head_dim);
  // the score scale is 1/sqrt(d), times the query and key scales of int8 codes
  const double sqk = kind == kFwdI8 ? (double)sq * (double)sk : 1.0;
  p.score_scale = (float)(1.4426950408889634 * sqk / sd);
  p.inv_scale = (float)(sd / sqk);
  p.mask_value = (float)(-100.0 * sd);
  mask_pieces(100.0 * sd / sqk, p.mask_pieces);
  p.out_i8 = kind == kFwdI8 && so > 0.f ? 1 : 0;
  p.v_scale = kind != kFwdI8 ? 1.f : p.out_i8 ? (float)((double)sv / (double)so) : sv;
  // bf16 and int8: the persistent LDS-staged kernel; fp32: the per-window kernel
  const int hg = head_group(heads, M);
  const bool persistent = kind != kFwdF32;
  const int cus = persistent ? compute_units(dev) : 0;
  p.nhg = heads / hg;
  // a unit's per-token input slice is hg * 32 elements: with several head
  // groups, neighbouring units of a window share 128-byte lines unless the
  // slice is a whole number of lines
  p.xcd_ranges = ((hg * kHeadDim * in_elem) % 128 != 0 && p.nhg > 1) ? 1 : 0;
  p.own_bias = 0;  // chosen per launch by the persistent kernel's launcher
  // fp32 kernel: heads are dealt round-robin to the waves of a workgroup,
  // preferably 2-3 heads per wave
  int waves = 1;
  for (int cand = 4; cand >= 1; --cand)
    if (heads % cand == 0 && heads / cand >= 2) {
      waves = cand;
      break;
    }
  // images per launch: keeps every in-kernel byte offset below 2^31, and the
  // grid (windows of the launch) below 2^31
  long long per = kMaxChunkBytes / max_image;
  if (per * nW * heads > 0x7fffffffLL) per = 0x7fffffffLL / (nW * heads);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const char* in = static_cast<const char*>(qkv);
  char* o = static_cast<char*>(out);
  for (long long b0 = 0; b0 < B; b0 += per) {
    const long long nb = B - b0 < per ? B - b0 : per;
    p.qkv = in + b0 * image_bytes;
    p.out = o + b0 * out_image_bytes;
    p.B = (int)nb;
    p.total_windows = (int)(nb * nW);
    p.units = (int)(nb * nW * p.nhg);
    const hipError_t err = kind == kFwdI8    ? launch_fwd_i8_persistent(M, hg, p, dev, cus, st)
                           : kind == kFwdBf16 ? launch_fwd_bf16_persistent(M, hg, p, dev, cus, st)
                                              : launch_fwd_f32(M, p, waves, st);
    if (err != hipSuccess) return SWIN_ERR_HIP;
  }
  return SWIN_OK;
}

int copy_common(int H, int W, int M, int s, void* dst, int which, void* stream) {
  if (!dst || !shape_ok(H, W, M, s)) return SWIN_ERR_INVALID_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SWIN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  Prepared* e = find(dev, H, W, M, s);
  if (!e) return SWIN_ERR_NOT_PREPARED;
  const size_t N = (size_t)M * M, nW = (size_t)(H / M) * (W / M);
  const void* src = which == 0 ? (const void*)e->rel_index
                    : which == 1 ? (const void*)e->mask
                                 : (const void*)e->region;
  const size_t bytes = which == 0 ? N * N * 4 : which == 1 ? nW * N * N * 4 : nW * N;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipStreamWaitEvent(st, e->ready, 0) != hipSuccess) return SWIN_ERR_HIP;
  const hipError_t err = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st);
  return err == hipSuccess ? SWIN_OK : SWIN_ERR_HIP;
}

}  // namespace

extern "C" {

int swin_wattn_precompute(int H, int W, int window, int shift, void* stream) {
  if (!shape_ok(H, W, window, shift)) return SWIN_ERR_INVALID_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SWIN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (find(dev, H, W, window, shift)) return SWIN_OK;
  const size_t N = (size_t)window * window, nW = (size_t)(H / window) * (W / window);
  const size_t b_idx = align256(N * N * 4), b_mask = align256(nW * N * N * 4),
               b_reg = align256(nW * N);
  void* block = nullptr;
  if (hipMalloc(&block, b_idx + b_mask + b_reg) != hipSuccess) return SWIN_ERR_HIP;
  Prepared e;
  e.dev = dev;
  e.H = H;
  e.W = W;
  e.M = window;
  e.s = shift;
  e.block = block;
  char* base = static_cast<char*>(block);
  e.rel_index = reinterpret_cast<int32_t*>(base);
  e.mask = reinterpret_cast<float*>(base + b_idx);
  e.region = reinterpret_cast<uint8_t*>(base + b_idx + b_mask);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipEventCreateWithFlags(&e.ready, hipEventDisableTiming) != hipSuccess) {
    (void)hipFree(block);
    return SWIN_ERR_HIP;
  }
  if (launch_precompute(H, W, window, shift, e.rel_index, e.mask, e.region, st) != hipSuccess ||
      hipEventRecord(e.ready, st) != hipSuccess) {
    (void)hipStreamSynchronize(st);
    (void)hipEventDestroy(e.ready);
    (void)hipFree(block);
    return SWIN_ERR_HIP;
  }
  g_cache.push_back(e);
  return SWIN_OK;
}

int swin_wattn_fwd(const void* qkv, const float* rel_bias_table, void* out, int B, int H, int W,
                   int heads, int head_dim, int window, int shift, void* stream) {
  return fwd_common(qkv, rel_bias_table, out, B, H, W, heads, head_dim, window, shift, stream,
                    kFwdBf16);
}

int swin_wattn_fwd_i8(const void* qkv, float scale_q, float scale_k, float scale_v,
                      float out_scale, const float* rel_bias_table, void* out, int B, int H,
                      int W, int heads, int head_dim, int window, int shift, void* stream) {
  return fwd_common(qkv, rel_bias_table, out, B, H, W, heads, head_dim, window, shift, stream,
                    kFwdI8, scale_q, scale_k, scale_v, out_scale);
}

int swin_wattn_fwd_f32(const float* qkv, const float* rel_bias_table, float* out, int B, int H,
                       int W, int heads, int head_dim, int window, int shift, void* stream) {
  return fwd_common(qkv, rel_bias_table, out, B, H, W, heads, head_dim, window, shift, stream,
                    kFwdF32);
}

int swin_linear_pack_weight(const void* weight, void* packed, int N, int K, void* stream) {
  if (!weight || !packed || !aligned(weight, 16) || !aligned(packed, 16)) return SWIN_ERR_INVALID_ARG;
  if (N <= 0 || K <= 0 || N % 32 != 0 || K % 32 != 0) return SWIN_ERR_INVALID_ARG;
  if (K > kMaxLinearK) return SWIN_ERR_UNSUPPORTED;
  const size_t bytes = (size_t)N * K * 2;
  if (overlap(weight, bytes, packed, bytes)) return SWIN_ERR_INVALID_ARG;
  return launch_linear_pack(weight, nullptr, packed, N, K, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? SWIN_OK
             : SWIN_ERR_HIP;
}

int swin_linear_i8_pack_weight(const void* weight, void* packed, int N, int K, void* stream) {
  if (!weight || !packed || !aligned(weight, 16) || !aligned(packed, 16)) return SWIN_ERR_INVALID_ARG;
  if (N <= 0 || K <= 0 || N % 32 != 0 || K % 32 != 0) return SWIN_ERR_INVALID_ARG;
  if (K > kMaxLinearKI8) return SWIN_ERR_UNSUPPORTED;
  if (overlap(weight, (size_t)N * K, packed, (size_t)N * ((K + 63) / 64) * 64))
    return SWIN_ERR_INVALID_ARG;
  return launch_linear_pack_i8(weight, packed, N, K, static_cast<hipStream_t>(stream)) == hipSuccess
             ? SWIN_OK
             : SWIN_ERR_HIP;
}

int swin_ln_linear_pack_weight(const void* weight, const float* gamma, const float* beta,
                               const float* bias, void* packed, float* consts, int N, int K,
                               void* stream) {
  if (!weight || !gamma || !beta || !packed || !consts) return SWIN_ERR_INVALID_ARG;
  if (!aligned(weight, 16) || !aligned(packed, 16) || !aligned(consts, 16) || !aligned(gamma, 4) ||
      !aligned(beta, 4) || (bias && !aligned(bias, 4)))
    return SWIN_ERR_INVALID_ARG;
  if (N <= 0 || K <= 0 || N % 32 != 0 || K % 32 != 0) return SWIN_ERR_INVALID_ARG;
  if (K > kMaxLinearK) return SWIN_ERR_UNSUPPORTED;
  const size_t wb = (size_t)N * K * 2, cb = (size_t)N * 8;
  if (overlap(weight, wb, packed, wb) || overlap(consts, cb, packed, wb) ||
      overlap(consts, cb, weight, wb) || overlap(consts, cb, gamma, (size_t)K * 4) ||
      overlap(consts, cb, beta, (size_t)K * 4) || (bias && overlap(consts, cb, bias, (size_t)N * 4)))
    return SWIN_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (launch_linear_pack(weight, gamma, packed, N, K, st) != hipSuccess) return SWIN_ERR_HIP;
  return launch_linear_ln_consts(weight, gamma, beta, bias, consts, N, K, st) == hipSuccess
             ? SWIN_OK
             : SWIN_ERR_HIP;
}

int swin_wattn_bwd(const void* qkv, const float* rel_bias_table, const void* dout, void* dqkv,
                   float* dtable, int B, int H, int W, int heads, int head_dim, int window,
                   int shift, void* stream) {
  if (!qkv || !rel_bias_table || !dout || !dqkv || !dtable) return SWIN_ERR_INVALID_ARG;
  if (!aligned(qkv, 16) || !aligned(dout, 16) || !aligned(dqkv, 16) || !aligned(rel_bias_table, 4) ||
      !aligned(dtable, 4))
    return SWIN_ERR_INVALID_ARG;
  const int M = window, s = shift;
  if (B < 0 || H <= 0 || W <= 0 || heads <= 0 || head_dim <= 0 || M <= 0) return SWIN_ERR_INVALID_ARG;
  if (H % M != 0 || W % M != 0 || s < 0 || s >= M) return SWIN_ERR_INVALID_ARG;
  if (head_dim != kHeadDim || M > kMaxBwdWindow) return SWIN_ERR_UNSUPPORTED;
  const long long nW = (long long)(H / M) * (W / M);
  const long long C = (long long)heads * head_dim;
  const long long image_bytes = (long long)H * W * 3 * C * 2;
  if (image_bytes > kMaxChunkBytes) return SWIN_ERR_UNSUPPORTED;
  const long long tokens = (long long)B * H * W;
  const size_t qb = (size_t)(tokens * 3 * C * 2), gb = (size_t)(tokens * C * 2);
  const size_t tb = (size_t)(2 * M - 1) * (2 * M - 1) * heads * 4;
  if (overlap(dqkv, qb, qkv, qb) || overlap(dqkv, qb, dout, gb) || overlap(dqkv, qb, dtable, tb) ||
      overlap(dtable, tb, qkv, qb) || overlap(dtable, tb, dout, gb) ||
      overlap(dtable, tb, rel_bias_table, tb))
    return SWIN_ERR_INVALID_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SWIN_ERR_HIP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the bias gradient is a sum over every window: zeroed, then accumulated
  if (launch_fill(dtable, (long long)tb / 4, 0.f, st) != hipSuccess) return SWIN_ERR_HIP;
  if (B == 0) return SWIN_OK;
  BwdParams p;
  p.table = rel_bias_table;
  p.dtable = dtable;
  p.H = H;
  p.W = W;
  p.nh = heads;
  p.shift = s;
  p.nWy = H / M;
  p.nWx = W / M;
  p.nW = (int)nW;
  const double sd = sqrt((double)head_dim);
  p.scale = (float)(1.0 / sd);
  p.score_scale = (float)(1.4426950408889634 / sd);
  p.inv_scale = (float)sd;
  mask_pieces(100.0 * sd, p.mask_pieces);
  const int cus = compute_units(dev);
  // images per launch: in-kernel byte offsets stay below 2^31
  const long long per = kMaxChunkBytes / image_bytes;
  const char* in = static_cast<const char*>(qkv);
  const char* gin = static_cast<const char*>(dout);
  char* o = static_cast<char*>(dqkv);
  for (long long b0 = 0; b0 < B; b0 += per) {
    const long long nb = B - b0 < per ? B - b0 : per;
    p.qkv = in + b0 * image_bytes;
    p.dout = gin + b0 * (image_bytes / 3);
    p.dqkv = o + b0 * image_bytes;
    p.B = (int)nb;
    p.windows = (int)(nb * nW);
    p.dqkv_bytes = (unsigned)(nb * image_bytes);
    if (launch_bwd_bf16(M, p, dev, cus, st) != hipSuccess) return SWIN_ERR_HIP;
  }
  return SWIN_OK;
}

namespace {

// The linear layers.  bf16: w_scale null.  int8: x and the packed weight are
// int8 codes, w_scale [N] the weight row scales; out_scale [N] (or null)
// selects int8 output.
int linear_common(const void* x, const float* colsum, float eps, const void* packed_weight,
                  const float* bias, const void* residual, void* y, long long T, int K, int N,
                  void* stream, const float* w_scale = nullptr, float x_scale = 1.f,
                  const float* out_scale = nullptr) {
  const bool i8 = w_scale != nullptr;
  if (!x || !packed_weight || !y) return SWIN_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(packed_weight, 16) || !aligned(y, 16) ||
      (bias && !aligned(bias, 16)) || (residual && !aligned(residual, 16)))
    return SWIN_ERR_INVALID_ARG;
  if (colsum && (!aligned(colsum, 16) || !(eps >= 0.f))) return SWIN_ERR_INVALID_ARG;
  if (i8 && (!aligned(w_scale, 16) || (out_scale && !aligned(out_scale, 16)) ||
             !(x_scale > 0.f) || !(x_scale <= 3.0e38f) || (out_scale && residual)))
    return SWIN_ERR_INVALID_ARG;
  if (T < 0 || N <= 0 || K <= 0 || N % 32 != 0 || K % 32 != 0) return SWIN_ERR_INVALID_ARG;
  if (K > (i8 ? kMaxLinearKI8 : kMaxLinearK)) return SWIN_ERR_UNSUPPORTED;
  const size_t xe = i8 ? 1 : 2, ye = out_scale ? 1 : 2;
  const size_t xb = (size_t)T * K * xe, yb = (size_t)T * N * ye;
  const size_t wb = i8 ? (size_t)N * ((K + 63) / 64) * 64 : (size_t)N * K * 2;
  if (overlap(y, yb, x, xb) || overlap(y, yb, packed_weight, wb) ||
      (bias && overlap(y, yb, bias, (size_t)N * 4)) ||
      (colsum && overlap(y, yb, colsum, (size_t)N * 4)) ||
      (w_scale && overlap(y, yb, w_scale, (size_t)N * 4)) ||
      (out_scale && overlap(y, yb, out_scale, (size_t)N * 4)))
    return SWIN_ERR_INVALID_ARG;
  // the residual may be y itself (in-place residual add), or lie apart from it
  if (residual && residual != y && overlap(y, yb, residual, yb)) return SWIN_ERR_INVALID_ARG;
  if (T == 0) return SWIN_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SWIN_ERR_HIP;
  const int cus = compute_units(dev);
  LinearParams p;
  p.wp = packed_weight;
  p.bias = bias;
  p.colsum = colsum;
  p.eps = eps;
  p.x_scale = x_scale;
  p.w_scale = w_scale;
  p.out_scale = out_scale;
  p.K = K;
  p.N = N;
  p.ncb = N / 32;
  // token indices inside the kernel are 32-bit: at most 2^30 tokens a launch
  for (long long t0 = 0; t0 < T; t0 += kMaxLinearTokens) {
    const long long n = T - t0 < kMaxLinearTokens ? T - t0 : kMaxLinearTokens;
    p.x = static_cast<const char*>(x) + t0 * K * (long long)xe;
    p.res = residual ? static_cast<const char*>(residual) + t0 * N * 2 : nullptr;
    p.y = static_cast<char*>(y) + t0 * N * (long long)ye;
    p.T = n;
    if (launch_linear(p, dev, cus, static_cast<hipStream_t>(stream)) != hipSuccess)
      return SWIN_ERR_HIP;
  }
  return SWIN_OK;
}

}  // namespace

int swin_linear_fwd(const void* x, const void* packed_weight, const float* bias,
                    const void* residual, void* y, long long T, int K, int N, void* stream) {
  return linear_common(x, nullptr, 0.f, packed_weight, bias, residual, y, T, K, N, stream);
}

int swin_linear_i8_fwd(const void* x, float x_scale, const void* packed_weight,
                       const float* w_scale, const float* bias, const void* residual,
                       const float* out_scale, void* y, long long T, int K, int N, void* stream) {
  if (!w_scale) return SWIN_ERR_INVALID_ARG;
  return linear_common(x, nullptr, 0.f, packed_weight, bias, residual, y, T, K, N, stream, w_scale,
                       x_scale, out_scale);
}

int swin_ln_linear_fwd(const void* x, const void* packed_weight, const float* consts, float eps,
                       void* y, long long T, int K, int N, void* stream) {
  if (!consts || !aligned(consts, 16)) return SWIN_ERR_INVALID_ARG;
  return linear_common(x, consts, eps, packed_weight, consts + N, nullptr, y, T, K, N, stream);
}

int swin_ln_qkv_wattn_fwd(const void* x, const void* packed_qkv, const float* consts, float eps,
                          const float* rel_bias_table, void* out, int B, int H, int W, int heads,
                          int head_dim, int window, int shift, void* stream) {
  if (!x || !packed_qkv || !consts || !rel_bias_table || !out) return SWIN_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(packed_qkv, 16) || !aligned(consts, 16) || !aligned(out, 16) ||
      !aligned(rel_bias_table, 4))
    return SWIN_ERR_INVALID_ARG;
  const int M = window, s = shift;
  if (B < 0 || H <= 0 || W <= 0 || heads <= 0 || head_dim <= 0 || M <= 0 || !(eps >= 0.f))
    return SWIN_ERR_INVALID_ARG;
  if (H % M != 0 || W % M != 0 || s < 0 || s >= M) return SWIN_ERR_INVALID_ARG;
  if (head_dim != kHeadDim || M < kMinLnAttnWindow || M > kMaxLnAttnWindow ||
      (long long)heads * head_dim > kMaxLnAttnC)
    return SWIN_ERR_UNSUPPORTED;
  const int C = heads * head_dim, N = 3 * C;
  const long long image_bytes = (long long)H * W * C * 2;
  const long long tokens = (long long)B * H * W;
  const size_t xb = (size_t)(tokens * C * 2), wb = (size_t)N * C * 2, cb = (size_t)N * 8;
  const size_t tb = (size_t)(2 * M - 1) * (2 * M - 1) * heads * 4;
  if (overlap(out, xb, x, xb) || overlap(out, xb, packed_qkv, wb) || overlap(out, xb, consts, cb) ||
      overlap(out, xb, rel_bias_table, tb))
    return SWIN_ERR_INVALID_ARG;
  if (B == 0) return SWIN_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SWIN_ERR_HIP;
  LnAttnParams p;
  p.wp = packed_qkv;
  p.consts = consts;
  p.table = rel_bias_table;
  p.eps = eps;
  p.H = H;
  p.W = W;
  p.nh = heads;
  p.C = C;
  p.N = N;
  p.shift = s;
  p.nWy = H / M;
  p.nWx = W / M;
  p.nW = p.nWy * p.nWx;
  const double sd = sqrt((double)head_dim);
  p.score_scale = (float)(1.4426950408889634 / sd);
  p.inv_scale = (float)sd;
  mask_pieces(100.0 * sd, p.mask_pieces);
  const int cus = compute_units(dev);
  // images per launch: in-kernel byte offsets of x and out stay below 2^31
  const long long per = kMaxChunkBytes / image_bytes;
  if (per < 1) return SWIN_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (long long b0 = 0; b0 < B; b0 += per) {
    const long long nb = B - b0 < per ? B - b0 : per;
    p.x = static_cast<const char*>(x) + b0 * image_bytes;
    p.out = static_cast<char*>(out) + b0 * image_bytes;
    p.B = (int)nb;
    p.windows = (int)(nb * p.nW);
    if (launch_ln_qkv_wattn(M, p, dev, cus, st) != hipSuccess) return SWIN_ERR_HIP;
  }
  return SWIN_OK;
}

int swin_wattn_copy_index(int H, int W, int window, int shift, int32_t* dst, void* stream) {
  return copy_common(H, W, window, shift, dst, 0, stream);
}

int swin_wattn_copy_mask(int H, int W, int window, int shift, float* dst, void* stream) {
  return copy_common(H, W, window, shift, dst, 1, stream);
}

int swin_wattn_copy_region(int H, int W, int window, int shift, uint8_t* dst, void* stream) {
  return copy_common(H, W, window, shift, dst, 2, stream);
}

int swin_wattn_release(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  int status = SWIN_OK;
  int cur = 0;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  for (auto& e : g_cache) {
    if (hipSetDevice(e.dev) != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
        hipEventDestroy(e.ready) != hipSuccess || hipFree(e.block) != hipSuccess)
      status = SWIN_ERR_HIP;
  }
  g_cache.clear();
  if (have_cur) (void)hipSetDevice(cur);
  return status;
}

const char* swin_wattn_status_string(int status) {
  switch (status) {
    case SWIN_OK: return "SWIN_OK";
    case SWIN_ERR_INVALID_ARG: return "SWIN_ERR_INVALID_ARG: invalid argument";
    case SWIN_ERR_UNSUPPORTED: return "SWIN_ERR_UNSUPPORTED: configuration not supported";
    case SWIN_ERR_NOT_PREPARED: return "SWIN_ERR_NOT_PREPARED: swin_wattn_precompute not called for this key";
    case SWIN_ERR_HIP: return "SWIN_ERR_HIP: HIP runtime error";
    default: return "unknown status";
  }
}

}  // extern "C"
