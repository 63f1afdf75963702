/*
 * swin_oracle.c -- fp64 CPU oracle for shifted-window multi-head attention.
 *
 * TEST INFRASTRUCTURE ONLY (see swin_oracle.h): used by the tests, the smoke
 * check and the CPU baseline of the benchmark, never by the product path.
 *
 * Every step is written as its plain definition, in the order the pages give
 * the operations of a Swin block (NVIDIA talk "Swin Transformer training and
 * inference optimization", section 1: window shift / partition / reverse,
 * then attention): shift by a cyclic roll, cut into windows, attention inside
 * each window with the relative position bias and the shift mask added to
 * the scores, reverse the partition, roll back.  Nothing is fused or
 * reordered; the attention is two plain triple loops around a softmax.
 */
#include "swin_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

static long mod_l(long a, long m) {
  long r = a % m;
  return r < 0 ? r + m : r;
}

/* torch.roll semantics: the element at i moves to (i + shift) mod H */
void oracle_roll(const double* x, int B, int H, int W, int C, int sy, int sx, double* y) {
  for (long b = 0; b < B; ++b)
    for (long i = 0; i < H; ++i)
      for (long j = 0; j < W; ++j) {
        long yi = mod_l(i + sy, H), yj = mod_l(j + sx, W);
        const double* src = x + ((b * H + i) * W + j) * (long)C;
        double* dst = y + ((b * H + yi) * W + yj) * (long)C;
        memcpy(dst, src, sizeof(double) * (size_t)C);
      }
}

/* cut [B][H][W][C] into non-overlapping M x M windows, windows in row-major
 * order over the image, tokens in row-major order inside a window */
void oracle_window_partition(const double* x, int B, int H, int W, int C, int M, double* win) {
  long nWy = H / M, nWx = W / M, N = (long)M * M;
  for (long b = 0; b < B; ++b)
    for (long wy = 0; wy < nWy; ++wy)
      for (long wx = 0; wx < nWx; ++wx)
        for (long ty = 0; ty < M; ++ty)
          for (long tx = 0; tx < M; ++tx) {
            long n = (b * nWy + wy) * nWx + wx, t = ty * M + tx;
            const double* src = x + ((b * H + wy * M + ty) * W + wx * M + tx) * (long)C;
            memcpy(win + (n * N + t) * (long)C, src, sizeof(double) * (size_t)C);
          }
}

/* put window tokens back at their image positions (inverse of the above) */
void oracle_window_reverse(const double* win, int B, int H, int W, int C, int M, double* x) {
  long nWy = H / M, nWx = W / M, N = (long)M * M;
  for (long b = 0; b < B; ++b)
    for (long wy = 0; wy < nWy; ++wy)
      for (long wx = 0; wx < nWx; ++wx)
        for (long ty = 0; ty < M; ++ty)
          for (long tx = 0; tx < M; ++tx) {
            long n = (b * nWy + wy) * nWx + wx, t = ty * M + tx;
            double* dst = x + ((b * H + wy * M + ty) * W + wx * M + tx) * (long)C;
            memcpy(dst, win + (n * N + t) * (long)C, sizeof(double) * (size_t)C);
          }
}

/* relative position of query i to key j, (dy, dx) = (y_i - y_j, x_i - x_j),
 * each in [-(M-1), M-1], shifted to be non-negative and flattened row-major
 * over a (2M-1) x (2M-1) table */
void oracle_rel_index(int M, int32_t* idx) {
  int N = M * M;
  for (int i = 0; i < N; ++i)
    for (int j = 0; j < N; ++j) {
      int dy = i / M - j / M, dx = i % M - j % M;
      idx[i * N + j] = (dy + M - 1) * (2 * M - 1) + (dx + M - 1);
    }
}

static int band(int p, int L, int M, int s) {
  if (p < L - M) return 0;
  if (p < L - s) return 1;
  return 2;
}

/* label every position of the shifted frame by the region it came from:
 * after the roll, the last M rows hold two strips that were not adjacent in
 * the image (the wrapped-around strip of s rows and the M-s rows before it);
 * likewise for columns */
void oracle_region_labels(int H, int W, int M, int s, int32_t* lab) {
  for (int y = 0; y < H; ++y)
    for (int x = 0; x < W; ++x)
      lab[y * W + x] = s > 0 ? 3 * band(y, H, M, s) + band(x, W, M, s) : 0;
}

void oracle_shift_mask(int H, int W, int M, int s, double* mask) {
  int N = M * M;
  long nW = (long)(H / M) * (W / M);
  int32_t* lab = (int32_t*)malloc(sizeof(int32_t) * (size_t)H * W);
  double* labd = (double*)malloc(sizeof(double) * (size_t)H * W);
  double* labw = (double*)malloc(sizeof(double) * (size_t)H * W);
  oracle_region_labels(H, W, M, s, lab);
  for (long k = 0; k < (long)H * W; ++k) labd[k] = lab[k];
  /* partition the label image exactly like the features */
  oracle_window_partition(labd, 1, H, W, 1, M, labw);
  for (long w = 0; w < nW; ++w)
    for (int i = 0; i < N; ++i)
      for (int j = 0; j < N; ++j)
        mask[(w * N + i) * N + j] = labw[w * N + i] == labw[w * N + j] ? 0.0 : -100.0;
  free(lab);
  free(labd);
  free(labw);
}

/* ---------------------------------------------------------------------- */
/* attention inside one window                                              */

typedef struct {
  const double* win_qkv;
  const float* table;
  const double* mask;
  const int32_t* rel;
  long nWin, begin, end;
  int nW, M, nh, d, npad;
  double* win_out;
} attn_job;

/* one window, every head: S = Q K^T * (1/sqrt d) + bias + mask, row softmax,
 * O = P V.  Padded tokens (index >= N) are zero; padded keys score -inf. */
static void attend_window(const attn_job* J, long n, double* q, double* k, double* v, double* S,
                          double* P) {
  const int M = J->M, N = M * M, nh = J->nh, d = J->d, Np = J->npad;
  const long C = (long)nh * d;
  const double scale = 1.0 / sqrt((double)d);
  const double* base = J->win_qkv + n * N * 3 * C;
  const double* mk = J->mask ? J->mask + (n % J->nW) * (long)N * N : NULL;
  for (int h = 0; h < nh; ++h) {
    for (int t = 0; t < Np; ++t)
      for (int e = 0; e < d; ++e) {
        int in = t < N;
        q[t * d + e] = in ? base[(t * 3 + 0) * C + h * d + e] : 0.0;
        k[t * d + e] = in ? base[(t * 3 + 1) * C + h * d + e] : 0.0;
        v[t * d + e] = in ? base[(t * 3 + 2) * C + h * d + e] : 0.0;
      }
    for (int i = 0; i < Np; ++i)
      for (int j = 0; j < Np; ++j) {
        if (j >= N) {
          S[i * Np + j] = -INFINITY;
          continue;
        }
        double dot = 0.0;
        for (int e = 0; e < d; ++e) dot += q[i * d + e] * k[j * d + e];
        double sc = dot * scale;
        if (i < N) {
          sc += (double)J->table[(long)J->rel[i * N + j] * nh + h];
          if (mk) sc += mk[i * N + j];
        }
        S[i * Np + j] = sc;
      }
    for (int i = 0; i < Np; ++i) {
      double m = -INFINITY;
      for (int j = 0; j < Np; ++j) m = S[i * Np + j] > m ? S[i * Np + j] : m;
      double sum = 0.0;
      for (int j = 0; j < Np; ++j) {
        P[i * Np + j] = exp(S[i * Np + j] - m);
        sum += P[i * Np + j];
      }
      for (int j = 0; j < Np; ++j) P[i * Np + j] /= sum;
    }
    for (int i = 0; i < N; ++i)
      for (int e = 0; e < d; ++e) {
        double acc = 0.0;
        for (int j = 0; j < Np; ++j) acc += P[i * Np + j] * v[j * d + e];
        J->win_out[(n * N + i) * C + h * d + e] = acc;
      }
  }
}

static void* attn_worker(void* arg) {
  const attn_job* J = (const attn_job*)arg;
  const int Np = J->npad, d = J->d;
  double* q = (double*)malloc(sizeof(double) * (size_t)Np * d);
  double* k = (double*)malloc(sizeof(double) * (size_t)Np * d);
  double* v = (double*)malloc(sizeof(double) * (size_t)Np * d);
  double* S = (double*)malloc(sizeof(double) * (size_t)Np * Np);
  double* P = (double*)malloc(sizeof(double) * (size_t)Np * Np);
  for (long n = J->begin; n < J->end; ++n) attend_window(J, n, q, k, v, S, P);
  free(q);
  free(k);
  free(v);
  free(S);
  free(P);
  return NULL;
}

static int resolve_threads(int nthreads, long work) {
  if (nthreads <= 0) {
    long c = sysconf(_SC_NPROCESSORS_ONLN);
    nthreads = c > 0 ? (int)c : 1;
  }
  if (nthreads > work) nthreads = work > 0 ? (int)work : 1;
  return nthreads;
}

int oracle_window_attention(const double* win_qkv, const float* table, const double* mask,
                            long nWin, int nW, int M, int nh, int d, int npad, int nthreads,
                            double* win_out) {
  const int N = M * M;
  if (npad < N) npad = N;
  int32_t* rel = (int32_t*)malloc(sizeof(int32_t) * (size_t)N * N);
  oracle_rel_index(M, rel);
  nthreads = resolve_threads(nthreads, nWin);
  attn_job* jobs = (attn_job*)calloc((size_t)nthreads, sizeof(attn_job));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  for (int t = 0; t < nthreads; ++t) {
    attn_job* J = &jobs[t];
    J->win_qkv = win_qkv;
    J->table = table;
    J->mask = mask;
    J->rel = rel;
    J->nWin = nWin;
    J->begin = nWin * t / nthreads;
    J->end = nWin * (t + 1) / nthreads;
    J->nW = nW;
    J->M = M;
    J->nh = nh;
    J->d = d;
    J->npad = npad;
    J->win_out = win_out;
    if (t > 0) pthread_create(&th[t], NULL, attn_worker, J);
  }
  attn_worker(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
  free(th);
  free(jobs);
  free(rel);
  return nthreads;
}

/* ---------------------------------------------------------------------- */

static double load_elem(const void* p, int dtype, long i) {
  if (dtype == ORACLE_F32) return (double)((const float*)p)[i];
  if (dtype == ORACLE_BF16) {
    /* a bf16 pattern is the upper half of the fp32 with the same value */
    uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return ((const double*)p)[i];
}

static int bad_args(int B, int H, int W, int nh, int d, int M, int s, int dtype) {
  return B < 0 || H <= 0 || W <= 0 || nh <= 0 || d <= 0 || M <= 0 || H % M || W % M || s < 0 ||
         s >= M || dtype < ORACLE_F64 || dtype > ORACLE_BF16;
}

int oracle_swin_wattn_fwd(const void* qkv, int dtype, const float* table, int B, int H, int W,
                          int nh, int d, int M, int s, int npad, int nthreads, double* out) {
  if (bad_args(B, H, W, nh, d, M, s, dtype)) return -1;
  const long C = (long)nh * d, C3 = 3 * C, HW = (long)H * W;
  const long N = (long)M * M, nW = (long)(H / M) * (W / M), nWin = (long)B * nW;
  double* x = (double*)malloc(sizeof(double) * (size_t)(B * HW * C3));
  double* xr = (double*)malloc(sizeof(double) * (size_t)(B * HW * C3));
  for (long i = 0; i < B * HW * C3; ++i) x[i] = load_elem(qkv, dtype, i);
  /* 1. cyclic shift towards the top-left */
  oracle_roll(x, B, H, W, (int)C3, -s, -s, xr);
  /* 2. window partition */
  oracle_window_partition(xr, B, H, W, (int)C3, M, x);
  free(xr);
  /* 3. attention inside every window, mask only for shifted windows */
  double* mask = NULL;
  if (s > 0) {
    mask = (double*)malloc(sizeof(double) * (size_t)(nW * N * N));
    oracle_shift_mask(H, W, M, s, mask);
  }
  double* wo = (double*)malloc(sizeof(double) * (size_t)(B * HW * C));
  int used = oracle_window_attention(x, table, mask, nWin, (int)nW, M, nh, d, npad, nthreads, wo);
  free(x);
  free(mask);
  /* 4. window reverse, 5. roll back */
  double* o = (double*)malloc(sizeof(double) * (size_t)(B * HW * C));
  oracle_window_reverse(wo, B, H, W, (int)C, M, o);
  oracle_roll(o, B, H, W, (int)C, s, s, out);
  free(wo);
  free(o);
  return used;
}

int oracle_swin_wattn_windows(const void* qkv, int dtype, const float* table, int B, int H,
                              int W, int nh, int d, int M, int s, long nsel, const int64_t* sel,
                              int nthreads, double* out, int64_t* pos) {
  if (bad_args(B, H, W, nh, d, M, s, dtype)) return -1;
  const long C = (long)nh * d, C3 = 3 * C, N = (long)M * M;
  const long nWx = W / M, nW = (long)(H / M) * nWx;
  for (long k = 0; k < nsel; ++k)
    if (sel[k] < 0 || sel[k] >= (long)B * nW) return -1;
  /* gather the selected windows: token t of window w sits at (wy*M+ty,
   * wx*M+tx) of the frame rolled by (-s,-s), whose position p holds the
   * image position (p + s) mod H -- the two index maps of steps 1 and 2 */
  double* win = (double*)malloc(sizeof(double) * (size_t)(nsel * N * C3));
  for (long k = 0; k < nsel; ++k) {
    long b = sel[k] / nW, w = sel[k] % nW, wy = w / nWx, wx = w % nWx;
    for (long t = 0; t < N; ++t) {
      long yr = wy * M + t / M, xr = wx * M + t % M;
      long y = mod_l(yr + s, H), x = mod_l(xr + s, W);
      long p = (b * H + y) * W + x;
      pos[k * N + t] = p;
      for (long c = 0; c < C3; ++c) win[(k * N + t) * C3 + c] = load_elem(qkv, dtype, p * C3 + c);
    }
  }
  double* mask = NULL;
  if (s > 0) {
    mask = (double*)malloc(sizeof(double) * (size_t)(nW * N * N));
    oracle_shift_mask(H, W, M, s, mask);
  }
  /* attention with each selected window's own mask slice */
  double* msel = NULL;
  if (mask) {
    msel = (double*)malloc(sizeof(double) * (size_t)(nsel * N * N));
    for (long k = 0; k < nsel; ++k)
      memcpy(msel + k * N * N, mask + (sel[k] % nW) * N * N, sizeof(double) * (size_t)(N * N));
  }
  int used = oracle_window_attention(win, table, msel, nsel, (int)(nsel > 0 ? nsel : 1), M, nh, d,
                                     (int)N, nthreads, out);
  free(win);
  free(mask);
  free(msel);
  return used;
}

/* ---------------------------------------------------------------------- */
/* linear layer: every output element is its own dot product in fp64 */

typedef struct {
  const void* x;
  const void* w;
  const void* r;
  const float* bias;
  int xdtype, wdtype, rdtype, K, N;
  long t0, t1;
  double* y;
} linear_job;

static void* linear_worker(void* arg) {
  const linear_job* J = (const linear_job*)arg;
  for (long t = J->t0; t < J->t1; ++t)
    for (int j = 0; j < J->N; ++j) {
      double acc = 0.0;
      for (int c = 0; c < J->K; ++c)
        acc += load_elem(J->x, J->xdtype, t * J->K + c) * load_elem(J->w, J->wdtype, (long)j * J->K + c);
      if (J->bias) acc += (double)J->bias[j];
      if (J->r) acc += load_elem(J->r, J->rdtype, t * J->N + j);
      J->y[t * J->N + j] = acc;
    }
  return NULL;
}

int oracle_linear(const void* x, int xdtype, long T, int K, const void* w, int wdtype, int N,
                  const float* bias, const void* residual, int rdtype, int nthreads, double* y) {
  if (T < 0 || K <= 0 || N <= 0 || xdtype < ORACLE_F64 || xdtype > ORACLE_BF16 ||
      wdtype < ORACLE_F64 || wdtype > ORACLE_BF16 || rdtype < ORACLE_F64 || rdtype > ORACLE_BF16)
    return -1;
  nthreads = resolve_threads(nthreads, T > 0 ? T : 1);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  linear_job* jobs = (linear_job*)malloc(sizeof(linear_job) * (size_t)nthreads);
  for (int i = 0; i < nthreads; ++i) {
    linear_job J = {x, w, residual, bias, xdtype, wdtype, rdtype, K, N,
                    T * i / nthreads, T * (i + 1) / nthreads, y};
    jobs[i] = J;
    pthread_create(&th[i], NULL, linear_worker, &jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  free(jobs);
  return nthreads;
}

/* ---------------------------------------------------------------------- */
/* INT8 quantized tensors                                                   */

void oracle_dequant_qkv_i8(const int8_t* codes, long tokens, int C, const float* scales,
                           double* out) {
  for (long t = 0; t < tokens; ++t)
    for (int part = 0; part < 3; ++part)
      for (int c = 0; c < C; ++c) {
        const long i = (t * 3 + part) * C + c;
        out[i] = (double)codes[i] * (double)scales[part];
      }
}

typedef struct {
  const int8_t* x;
  const int8_t* w;
  const void* r;
  const float *sw, *bias, *so;
  float sx;
  int rdtype, K, N;
  long t0, t1;
  int64_t* acc;
  double* y;
  int8_t* yq;
} linear_i8_job;

static void* linear_i8_worker(void* arg) {
  const linear_i8_job* J = (const linear_i8_job*)arg;
  for (long t = J->t0; t < J->t1; ++t)
    for (int j = 0; j < J->N; ++j) {
      /* the integer sum, exact */
      int64_t a = 0;
      for (int c = 0; c < J->K; ++c)
        a += (int64_t)J->x[t * J->K + c] * (int64_t)J->w[(long)j * J->K + c];
      const double b = J->bias ? (double)J->bias[j] : 0.0;
      const long o = t * J->N + j;
      if (J->acc) J->acc[o] = a;
      /* dequantized value, fp64 */
      if (J->y) {
        double v = (double)a * (double)J->sx * (double)J->sw[j] + b;
        if (J->r) v += load_elem(J->r, J->rdtype, o);
        J->y[o] = v;
      }
      /* the output code, decided in fp32 as one fused multiply-add */
      if (J->yq) {
        const float scale = (J->sx * J->sw[j]) / J->so[j];
        const float shift = (J->bias ? J->bias[j] : 0.0f) / J->so[j];
        float q = nearbyintf(fmaf((float)a, scale, shift));
        q = q > 127.0f ? 127.0f : q < -127.0f ? -127.0f : q;
        J->yq[o] = (int8_t)q;
      }
    }
  return NULL;
}

int oracle_linear_i8(const int8_t* xq, long T, int K, float sx, const int8_t* wq, int N,
                     const float* sw, const float* bias, const void* residual, int rdtype,
                     const float* so, int nthreads, int64_t* acc, double* y, int8_t* yq) {
  if (T < 0 || K <= 0 || N <= 0 || !xq || !wq || !sw || rdtype < ORACLE_F64 ||
      rdtype > ORACLE_BF16 || (yq && !so) || (so && residual))
    return -1;
  nthreads = resolve_threads(nthreads, T > 0 ? T : 1);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  linear_i8_job* jobs = (linear_i8_job*)malloc(sizeof(linear_i8_job) * (size_t)nthreads);
  for (int i = 0; i < nthreads; ++i) {
    linear_i8_job J = {xq, wq, residual, sw, bias, so, sx, rdtype, K, N,
                       T * i / nthreads, T * (i + 1) / nthreads, acc, y, yq};
    jobs[i] = J;
    pthread_create(&th[i], NULL, linear_i8_worker, &jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  free(jobs);
  return nthreads;
}

/* ---------------------------------------------------------------------- */
/* layer normalisation: two passes over each row, mean then variance */

int oracle_layernorm(const void* x, int xdtype, long T, int C, const float* gamma,
                     const float* beta, double eps, double* y) {
  if (T < 0 || C <= 0 || !gamma || !beta || eps < 0.0 || xdtype < ORACLE_F64 ||
      xdtype > ORACLE_BF16)
    return -1;
  for (long t = 0; t < T; ++t) {
    double mu = 0.0;
    for (int c = 0; c < C; ++c) mu += load_elem(x, xdtype, t * C + c);
    mu /= C;
    double var = 0.0;
    for (int c = 0; c < C; ++c) {
      const double dv = load_elem(x, xdtype, t * C + c) - mu;
      var += dv * dv;
    }
    var /= C;
    const double r = 1.0 / sqrt(var + eps);
    for (int c = 0; c < C; ++c)
      y[t * C + c] = (load_elem(x, xdtype, t * C + c) - mu) * r * (double)gamma[c] + (double)beta[c];
  }
  return 0;
}

/* ---------------------------------------------------------------------- */
/* backward of the window attention                                         */

typedef struct {
  const double* win_qkv;  /* [nWin][N][3C] */
  const double* win_g;    /* [nWin][N][C]  gradient of the window outputs */
  const float* table;
  const double* mask;     /* [nW][N][N] or NULL */
  const int32_t* rel;
  long begin, end;
  int nW, M, nh, d;
  double* win_dqkv;       /* [nWin][N][3C] */
  double* dtable;         /* [(2M-1)^2][nh], this job's partial sums */
} bwd_job;

static void* bwd_worker(void* arg) {
  const bwd_job* J = (const bwd_job*)arg;
  const int M = J->M, N = M * M, nh = J->nh, d = J->d;
  const long C = (long)nh * d;
  const double scale = 1.0 / sqrt((double)d);
  double* S = (double*)malloc(sizeof(double) * (size_t)N * N);
  double* dP = (double*)malloc(sizeof(double) * (size_t)N * N);
  double* Dr = (double*)malloc(sizeof(double) * (size_t)N);
  for (long n = J->begin; n < J->end; ++n) {
    const double* x = J->win_qkv + n * N * 3 * C;
    const double* g = J->win_g + n * N * C;
    const double* mk = J->mask ? J->mask + (n % J->nW) * (long)N * N : NULL;
    double* dx = J->win_dqkv + n * N * 3 * C;
    for (int h = 0; h < nh; ++h) {
#define Q_(t, e) x[(long)(t) * 3 * C + h * d + (e)]
#define K_(t, e) x[(long)(t) * 3 * C + C + h * d + (e)]
#define V_(t, e) x[(long)(t) * 3 * C + 2 * C + h * d + (e)]
#define G_(t, e) g[(long)(t) * C + h * d + (e)]
      /* recompute the attention weights P (stored in S) */
      for (int i = 0; i < N; ++i) {
        double m = -INFINITY;
        for (int j = 0; j < N; ++j) {
          double dot = 0.0;
          for (int e = 0; e < d; ++e) dot += Q_(i, e) * K_(j, e);
          double sc = dot * scale + (double)J->table[(long)J->rel[i * N + j] * nh + h];
          if (mk) sc += mk[i * N + j];
          S[i * N + j] = sc;
          m = sc > m ? sc : m;
        }
        double sum = 0.0;
        for (int j = 0; j < N; ++j) {
          S[i * N + j] = exp(S[i * N + j] - m);
          sum += S[i * N + j];
        }
        for (int j = 0; j < N; ++j) S[i * N + j] /= sum;
      }
      /* dP = dO V^T and D_i = sum_j P_ij dP_ij */
      for (int i = 0; i < N; ++i) {
        double Di = 0.0;
        for (int j = 0; j < N; ++j) {
          double acc = 0.0;
          for (int e = 0; e < d; ++e) acc += G_(i, e) * V_(j, e);
          dP[i * N + j] = acc;
          Di += S[i * N + j] * acc;
        }
        Dr[i] = Di;
      }
      /* dS = P o (dP - D), kept in dP; the bias gradient */
      for (int i = 0; i < N; ++i)
        for (int j = 0; j < N; ++j) {
          dP[i * N + j] = S[i * N + j] * (dP[i * N + j] - Dr[i]);
          J->dtable[(long)J->rel[i * N + j] * nh + h] += dP[i * N + j];
        }
      /* dQ = dS K * scale, dK = dS^T Q * scale, dV = P^T dO */
      for (int t = 0; t < N; ++t)
        for (int e = 0; e < d; ++e) {
          double aq = 0.0, ak = 0.0, av = 0.0;
          for (int u = 0; u < N; ++u) {
            aq += dP[t * N + u] * K_(u, e);
            ak += dP[u * N + t] * Q_(u, e);
            av += S[u * N + t] * G_(u, e);
          }
          dx[(long)t * 3 * C + h * d + e] = aq * scale;
          dx[(long)t * 3 * C + C + h * d + e] = ak * scale;
          dx[(long)t * 3 * C + 2 * C + h * d + e] = av;
        }
#undef Q_
#undef K_
#undef V_
#undef G_
    }
  }
  free(S);
  free(dP);
  free(Dr);
  return NULL;
}

int oracle_swin_wattn_bwd(const void* qkv, int dtype, const float* table, const void* dout,
                          int dout_dtype, int B, int H, int W, int nh, int d, int M, int s,
                          int nthreads, double* dqkv, double* dtable) {
  if (bad_args(B, H, W, nh, d, M, s, dtype) || dout_dtype < ORACLE_F64 || dout_dtype > ORACLE_BF16)
    return -1;
  const long C = (long)nh * d, C3 = 3 * C, HW = (long)H * W;
  const long N = (long)M * M, nW = (long)(H / M) * (W / M), nWin = (long)B * nW;
  const long T = (long)(2 * M - 1) * (2 * M - 1);
  /* 1. qkv and dout through the roll by (-s, -s) and the partition */
  double* a = (double*)malloc(sizeof(double) * (size_t)(B * HW * C3));
  double* b = (double*)malloc(sizeof(double) * (size_t)(B * HW * C3));
  for (long i = 0; i < B * HW * C3; ++i) a[i] = load_elem(qkv, dtype, i);
  oracle_roll(a, B, H, W, (int)C3, -s, -s, b);
  double* win_qkv = (double*)malloc(sizeof(double) * (size_t)(B * HW * C3));
  oracle_window_partition(b, B, H, W, (int)C3, M, win_qkv);
  for (long i = 0; i < B * HW * C; ++i) a[i] = load_elem(dout, dout_dtype, i);
  oracle_roll(a, B, H, W, (int)C, -s, -s, b);
  double* win_g = (double*)malloc(sizeof(double) * (size_t)(B * HW * C));
  oracle_window_partition(b, B, H, W, (int)C, M, win_g);
  double* mask = NULL;
  if (s > 0) {
    mask = (double*)malloc(sizeof(double) * (size_t)(nW * N * N));
    oracle_shift_mask(H, W, M, s, mask);
  }
  int32_t* rel = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N * N));
  oracle_rel_index(M, rel);
  /* 2. gradients window by window; each thread keeps its own bias partial */
  nthreads = resolve_threads(nthreads, nWin > 0 ? nWin : 1);
  double* win_dqkv = (double*)malloc(sizeof(double) * (size_t)(B * HW * C3));
  double* part = (double*)calloc((size_t)(nthreads * T * nh), sizeof(double));
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  bwd_job* jobs = (bwd_job*)malloc(sizeof(bwd_job) * (size_t)nthreads);
  for (int i = 0; i < nthreads; ++i) {
    bwd_job J = {win_qkv, win_g, table, mask, rel, nWin * i / nthreads, nWin * (i + 1) / nthreads,
                 (int)nW, M, nh, d, win_dqkv, part + (long)i * T * nh};
    jobs[i] = J;
    pthread_create(&th[i], NULL, bwd_worker, &jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  for (long e = 0; e < T * nh; ++e) {
    double acc = 0.0;
    for (int i = 0; i < nthreads; ++i) acc += part[(long)i * T * nh + e];
    dtable[e] = acc;
  }
  /* 3. window reverse and the roll back by (+s, +s) */
  oracle_window_reverse(win_dqkv, B, H, W, (int)C3, M, a);
  oracle_roll(a, B, H, W, (int)C3, s, s, dqkv);
  free(a);
  free(b);
  free(win_qkv);
  free(win_g);
  free(win_dqkv);
  free(mask);
  free(rel);
  free(part);
  free(th);
  free(jobs);
  return nthreads;
}
