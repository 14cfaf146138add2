/*
 * na3d_oracle.c -- plain, slow, obviously-correct CPU oracle for the forward
 * pass of 3-D neighborhood attention (NA3D).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker the GPU path is compared
 * against.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline leg may build, load or call it; the product library never does,
 * and it shares no code, header, table or helper with the HIP sources.
 *
 * What it computes (ROCm/aiter PR "Add 3D neighborhood flash attention
 * (na3d_flash)", sections "Motivation" and "Technical Details"):
 *   - each query token at grid position (t,h,w) attends only to a
 *     KT x KH x KW box of keys around it (Motivation);
 *   - near a border the box is shifted inward so that it always holds exactly
 *     KT*KH*KW keys (Technical Details, "inward border-shift").  Per axis the
 *     box starts at clamp(i - K/2, 0, L - K) (integer K/2, floor);
 *   - tensors are (B,T,H,W,NH,HD) bfloat16 and Q already carries the
 *     head_dim^-0.5 factor, so the score is the plain dot product q.k
 *     (Technical Details, public launcher paragraph);
 *   - the output is the softmax-weighted sum of the window's V rows.
 *
 * Precision: bf16 inputs are widened exactly to double; every sum is taken in
 * double in a fixed order (ascending head-dim index, keys in (dt,dh,dw)
 * lexicographic order); softmax is the two-pass form (max, then exp/sum).
 * The result is written as double.  No blocking, fusion, online softmax or
 * reordering is applied.
 *
 * Parity pins: every function here is pinned in the CPU test suite against
 * results that do not come from this file (hand-worked window starts, dense
 * attention with an explicitly searched mask, closed forms, invariants).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARGS (-1)
#define ORACLE_NO_MEMORY (-2)

/* Exact bf16 -> double: a bf16 value is the top 16 bits of an IEEE float. */
static double bf16_to_double(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Inward-shifted window start on one axis: clamp(i - K/2, 0, L - K).
 * Returns -1 when the arguments are outside the defined range
 * (K < 1, K > L, or i outside [0, L)). */
int na3d_oracle_window_start(int i, int K, int L) {
  if (K < 1 || L < 1 || K > L || i < 0 || i >= L) return -1;
  int s = i - K / 2;
  if (s < 0) s = 0;
  if (s > L - K) s = L - K;
  return s;
}

static int check_dims(int B, int T, int H, int W, int NH, int HD, int KT,
                      int KH, int KW) {
  if (B < 1 || T < 1 || H < 1 || W < 1 || NH < 1 || HD < 1) return 0;
  if (KT < 1 || KH < 1 || KW < 1) return 0;
  if (KT > T || KH > H || KW > W) return 0;
  return 1;
}

/* One query (b,t,h,w,n): fills o[0..HD) and, if wts != NULL, the KT*KH*KW
 * softmax weights in window order.  s and e are caller scratch of K doubles. */
static void one_query(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      int T, int H, int W, int NH, int HD, int KT, int KH,
                      int KW, int b, int t, int h, int w, int n, double* s,
                      double* e, double* o, double* wts) {
  const int64_t head_stride = HD;
  const int64_t tok_stride = (int64_t)NH * HD;
  const int64_t qoff =
      ((((int64_t)b * T + t) * H + h) * W + w) * tok_stride + n * head_stride;
  const int st = na3d_oracle_window_start(t, KT, T);
  const int sh = na3d_oracle_window_start(h, KH, H);
  const int sw = na3d_oracle_window_start(w, KW, W);
  const int K = KT * KH * KW;

  /* scores, keys in (dt,dh,dw) lexicographic order */
  int j = 0;
  for (int dt = 0; dt < KT; ++dt)
    for (int dh = 0; dh < KH; ++dh)
      for (int dw = 0; dw < KW; ++dw, ++j) {
        const int64_t koff =
            ((((int64_t)b * T + (st + dt)) * H + (sh + dh)) * W + (sw + dw)) *
                tok_stride +
            n * head_stride;
        double acc = 0.0;
        for (int d = 0; d < HD; ++d)
          acc += bf16_to_double(q[qoff + d]) * bf16_to_double(k[koff + d]);
        s[j] = acc;
      }

  /* two-pass softmax */
  double m = s[0];
  for (j = 1; j < K; ++j)
    if (s[j] > m) m = s[j];
  double l = 0.0;
  for (j = 0; j < K; ++j) {
    e[j] = exp(s[j] - m);
    l += e[j];
  }
  if (wts)
    for (j = 0; j < K; ++j) wts[j] = e[j] / l;

  /* weighted sum of V rows, same key order */
  for (int d = 0; d < HD; ++d) o[d] = 0.0;
  j = 0;
  for (int dt = 0; dt < KT; ++dt)
    for (int dh = 0; dh < KH; ++dh)
      for (int dw = 0; dw < KW; ++dw, ++j) {
        const int64_t voff =
            ((((int64_t)b * T + (st + dt)) * H + (sh + dh)) * W + (sw + dw)) *
                tok_stride +
            n * head_stride;
        for (int d = 0; d < HD; ++d) o[d] += e[j] * bf16_to_double(v[voff + d]);
      }
  for (int d = 0; d < HD; ++d) o[d] /= l;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

/* Number of threads OpenMP will use for the next parallel region. */
int na3d_oracle_max_threads(int nthreads) {
#ifdef _OPENMP
  set_threads(nthreads);
  return omp_get_max_threads();
#else
  (void)nthreads;
  return 1;
#endif
}

/* Full forward pass.  q,k,v: bf16 bit patterns, (B,T,H,W,NH,HD) contiguous.
 * out: double, same shape.  nthreads <= 0 means the OpenMP default. */
int na3d_oracle_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    double* out, int B, int T, int H, int W, int NH, int HD,
                    int KT, int KH, int KW, int nthreads) {
  if (!q || !k || !v || !out) return ORACLE_BAD_ARGS;
  if (!check_dims(B, T, H, W, NH, HD, KT, KH, KW)) return ORACLE_BAD_ARGS;
  const int K = KT * KH * KW;
  const int64_t rows = (int64_t)B * T * H;
  int failed = 0;
  set_threads(nthreads);
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)K);
    double* e = (double*)malloc(sizeof(double) * (size_t)K);
    if (!s || !e) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < rows; ++r) {
        const int b = (int)(r / ((int64_t)T * H));
        const int t = (int)((r / H) % T);
        const int h = (int)(r % H);
        for (int w = 0; w < W; ++w)
          for (int n = 0; n < NH; ++n) {
            const int64_t ooff =
                ((((int64_t)b * T + t) * H + h) * W + w) * NH * HD +
                (int64_t)n * HD;
            one_query(q, k, v, T, H, W, NH, HD, KT, KH, KW, b, t, h, w, n, s, e,
                      out + ooff, NULL);
          }
      }
    }
    free(s);
    free(e);
  }
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* Selected queries only.  idx holds npts (b,t,h,w,n) quintuples (int64);
 * out receives npts*HD doubles, one HD-row per point, in idx order. */
int na3d_oracle_fwd_points(const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const int64_t* idx, int64_t npts,
                           double* out, int B, int T, int H, int W, int NH,
                           int HD, int KT, int KH, int KW, int nthreads) {
  if (!q || !k || !v || !idx || !out || npts < 0) return ORACLE_BAD_ARGS;
  if (!check_dims(B, T, H, W, NH, HD, KT, KH, KW)) return ORACLE_BAD_ARGS;
  for (int64_t p = 0; p < npts; ++p) {
    const int64_t* c = idx + 5 * p;
    if (c[0] < 0 || c[0] >= B || c[1] < 0 || c[1] >= T || c[2] < 0 ||
        c[2] >= H || c[3] < 0 || c[3] >= W || c[4] < 0 || c[4] >= NH)
      return ORACLE_BAD_ARGS;
  }
  const int K = KT * KH * KW;
  int failed = 0;
  set_threads(nthreads);
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)K);
    double* e = (double*)malloc(sizeof(double) * (size_t)K);
    if (!s || !e) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t p = 0; p < npts; ++p) {
        const int64_t* c = idx + 5 * p;
        one_query(q, k, v, T, H, W, NH, HD, KT, KH, KW, (int)c[0], (int)c[1],
                  (int)c[2], (int)c[3], (int)c[4], s, e, out + p * HD, NULL);
      }
    }
    free(s);
    free(e);
  }
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* Softmax weights of every query: wts is (B,T,H,W,NH,KT*KH*KW) doubles in
 * window order; starts is (B,T,H,W,NH,3) ints holding (st,sh,sw).  Meant for
 * tiny grids (debugging and invariant tests). */
int na3d_oracle_weights(const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, double* wts, int32_t* starts, int B,
                        int T, int H, int W, int NH, int HD, int KT, int KH,
                        int KW) {
  if (!q || !k || !v || !wts || !starts) return ORACLE_BAD_ARGS;
  if (!check_dims(B, T, H, W, NH, HD, KT, KH, KW)) return ORACLE_BAD_ARGS;
  const int K = KT * KH * KW;
  double* s = (double*)malloc(sizeof(double) * (size_t)K);
  double* e = (double*)malloc(sizeof(double) * (size_t)K);
  double* o = (double*)malloc(sizeof(double) * (size_t)HD);
  if (!s || !e || !o) {
    free(s);
    free(e);
    free(o);
    return ORACLE_NO_MEMORY;
  }
  int64_t qi = 0;
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < T; ++t)
      for (int h = 0; h < H; ++h)
        for (int w = 0; w < W; ++w)
          for (int n = 0; n < NH; ++n, ++qi) {
            one_query(q, k, v, T, H, W, NH, HD, KT, KH, KW, b, t, h, w, n, s, e,
                      o, wts + qi * K);
            starts[3 * qi + 0] = na3d_oracle_window_start(t, KT, T);
            starts[3 * qi + 1] = na3d_oracle_window_start(h, KH, H);
            starts[3 * qi + 2] = na3d_oracle_window_start(w, KW, W);
          }
  free(s);
  free(e);
  free(o);
  return ORACLE_OK;
}
