/*
 * conv_oracle.c -- plain, slow, CPU reference for the fused NHWC conv2d layer
 * and the four-tile mosaic packer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do. It shares no code, header, table or constant with the
 * HIP library.
 *
 * What it computes (sources: the nanoinfer README page, section on the naive
 * nested-loop convolution kept as the reference kernel, and its statement
 * that a 1x1 stride-1 unpadded convolution is a GEMM on the untouched input;
 * the zerolat.eu YOLOv4 report, section 7 "Accuracy recovery" table for the
 * Mish definition and section 4 for the 2x2 mosaic placement):
 *
 *   pre[n,ho,wo,co] = B[co] + sum_{kh,kw,ci} X[n, ho*sh-ph+kh, wo*sw-pw+kw,
 *                                               g*Cg + ci] * W[co,kh,kw,ci]
 *   with g = co / (Cout/groups), Cg = Cin/groups, X = 0 outside the image.
 *   (cross-correlation, no kernel flip; zero padding, pad_h on top and
 *   bottom, pad_w on left and right; output Ho = (H+2ph-KH)/sh + 1.)
 *
 * Float inputs (fp32, or bf16 values widened exactly to fp32) accumulate in
 * double; the activation is applied in double and the result is NOT rounded
 * to the output type. The absolute-value convolution
 *   A = |B| + sum |X*W|
 * is returned beside it so the caller can form a relative error that stays
 * defined under cancellation.
 *
 * int8 inputs accumulate exactly in int64; R32 = acc + bias (checked to fit
 * int32). The int32 checkpoint output is R32. The int8 output is
 *   v = fl32( fl32(R32) * s[co] )    (IEEE float32: one RNE convert, one RNE
 *                                      multiply, no fused multiply-add)
 *   m = act(v)                        (ReLU/ReLU6 exact in float32, Mish in
 *                                      double from v)
 *   Q = clamp(round_half_even(m), -127, 127)
 *
 * The loops are written in the order of the definition; OpenMP only splits
 * independent output rows across threads, which changes no arithmetic.
 *
 * The file also holds the SPP max-pool block (oracle_spp) and the
 * upsample-and-concat of two maps (oracle_upcat), each defined where it
 * stands.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no -ffast-math).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ACT_NONE = 0, ACT_RELU = 1, ACT_RELU6 = 2, ACT_MISH = 3 };

enum {
  ORC_OK = 0,
  ORC_E_SHAPE = -2,
  ORC_E_RANGE = -8 /* int8 accumulator + bias does not fit int32 */
};

typedef struct {
  int64_t n, h, w, cin, cout;
  int64_t kh, kw, sh, sw, ph, pw, groups;
  int64_t ho, wo;
} geom_t;

static int make_geom(geom_t *g, int64_t n, int64_t h, int64_t w, int64_t cin,
                     int64_t cout, int64_t kh, int64_t kw, int64_t sh,
                     int64_t sw, int64_t ph, int64_t pw, int64_t groups) {
  if (n <= 0 || h <= 0 || w <= 0 || cin <= 0 || cout <= 0 || kh <= 0 ||
      kw <= 0 || sh <= 0 || sw <= 0 || ph < 0 || pw < 0 || groups <= 0)
    return ORC_E_SHAPE;
  if (cin % groups || cout % groups) return ORC_E_SHAPE;
  int64_t hp = h + 2 * ph - kh, wp = w + 2 * pw - kw;
  if (hp < 0 || wp < 0) return ORC_E_SHAPE;
  g->n = n; g->h = h; g->w = w; g->cin = cin; g->cout = cout;
  g->kh = kh; g->kw = kw; g->sh = sh; g->sw = sw; g->ph = ph; g->pw = pw;
  g->groups = groups;
  g->ho = hp / sh + 1;
  g->wo = wp / sw + 1;
  return ORC_OK;
}

/* Mish(x) = x * tanh(softplus(x)), softplus(x) = ln(1 + e^x), written as
 * max(x,0) + log1p(exp(-|x|)) so that exp never overflows. */
double oracle_mish(double x) {
  double sp = (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
  return x * tanh(sp);
}

double oracle_act(double x, int act) {
  switch (act) {
    case ACT_RELU: return x > 0.0 ? x : 0.0;
    case ACT_RELU6: return x > 0.0 ? (x < 6.0 ? x : 6.0) : 0.0;
    case ACT_MISH: return oracle_mish(x);
    default: return x;
  }
}

/* One output element of the float convolution: returns pre-activation in
 * double and, when abs_out is not NULL, the absolute-value sum through it
 * (the pre-activation's sum is the same either way). */
static double conv_point_float(const geom_t *g, const float *x, const float *wt,
                               const float *b, int64_t n, int64_t ho,
                               int64_t wo, int64_t co, double *abs_out) {
  const int64_t cg = g->cin / g->groups;
  const int64_t og = g->cout / g->groups;
  const int64_t grp = co / og;
  double acc = 0.0, aacc = 0.0;
  if (b) {
    acc = (double)b[co];
    aacc = fabs((double)b[co]);
  }
  for (int64_t kh = 0; kh < g->kh; ++kh) {
    int64_t hi = ho * g->sh - g->ph + kh;
    if (hi < 0 || hi >= g->h) continue;
    for (int64_t kw = 0; kw < g->kw; ++kw) {
      int64_t wi = wo * g->sw - g->pw + kw;
      if (wi < 0 || wi >= g->w) continue;
      const float *xp = x + ((n * g->h + hi) * g->w + wi) * g->cin + grp * cg;
      const float *wp = wt + ((co * g->kh + kh) * g->kw + kw) * cg;
      if (abs_out) {
        for (int64_t ci = 0; ci < cg; ++ci) {
          double p = (double)xp[ci] * (double)wp[ci];
          acc += p;
          aacc += fabs(p);
        }
      } else {
        for (int64_t ci = 0; ci < cg; ++ci) acc += (double)xp[ci] * (double)wp[ci];
      }
    }
  }
  if (abs_out) *abs_out = aacc;
  return acc;
}

static int set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
  return omp_get_max_threads();
#else
  (void)nthreads;
  return 1;
#endif
}

/* Full float convolution. r (required) gets act(pre); a (optional) gets the
 * absolute-value convolution. Both are [n][ho][wo][cout] doubles. */
int oracle_conv_float(const float *x, const float *wt, const float *b,
                      int64_t n, int64_t h, int64_t w, int64_t cin,
                      int64_t cout, int64_t kh, int64_t kw, int64_t sh,
                      int64_t sw, int64_t ph, int64_t pw, int64_t groups,
                      int act, double *r, double *a, int nthreads) {
  geom_t g;
  int st = make_geom(&g, n, h, w, cin, cout, kh, kw, sh, sw, ph, pw, groups);
  if (st) return st;
  set_threads(nthreads);
  int64_t rows = g.n * g.ho;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t row = 0; row < rows; ++row) {
    int64_t nn = row / g.ho, ho = row % g.ho;
    for (int64_t wo = 0; wo < g.wo; ++wo)
      for (int64_t co = 0; co < g.cout; ++co) {
        double ab = 0.0;
        double pre = conv_point_float(&g, x, wt, b, nn, ho, wo, co, a ? &ab : NULL);
        int64_t o = ((nn * g.ho + ho) * g.wo + wo) * g.cout + co;
        r[o] = oracle_act(pre, act);
        if (a) a[o] = ab;
      }
  }
  return ORC_OK;
}

/* Same definition evaluated only at the flat output indices idx[0..cnt). */
int oracle_conv_float_at(const float *x, const float *wt, const float *b,
                         int64_t n, int64_t h, int64_t w, int64_t cin,
                         int64_t cout, int64_t kh, int64_t kw, int64_t sh,
                         int64_t sw, int64_t ph, int64_t pw, int64_t groups,
                         int act, const int64_t *idx, int64_t cnt, double *r,
                         double *a, int nthreads) {
  geom_t g;
  int st = make_geom(&g, n, h, w, cin, cout, kh, kw, sh, sw, ph, pw, groups);
  if (st) return st;
  int64_t total = g.n * g.ho * g.wo * g.cout;
  for (int64_t i = 0; i < cnt; ++i)
    if (idx[i] < 0 || idx[i] >= total) return ORC_E_SHAPE;
  set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t i = 0; i < cnt; ++i) {
    int64_t o = idx[i];
    int64_t co = o % g.cout, t = o / g.cout;
    int64_t wo = t % g.wo;
    t /= g.wo;
    int64_t ho = t % g.ho, nn = t / g.ho;
    double ab = 0.0;
    double pre = conv_point_float(&g, x, wt, b, nn, ho, wo, co, a ? &ab : NULL);
    r[i] = oracle_act(pre, act);
    if (a) a[i] = ab;
  }
  return ORC_OK;
}

/* ---------------------------------------------------------------- int8 -- */

static int64_t conv_point_i8(const geom_t *g, const int8_t *x, const int8_t *wt,
                             int64_t n, int64_t ho, int64_t wo, int64_t co) {
  const int64_t cg = g->cin / g->groups;
  const int64_t og = g->cout / g->groups;
  const int64_t grp = co / og;
  int64_t acc = 0;
  for (int64_t kh = 0; kh < g->kh; ++kh) {
    int64_t hi = ho * g->sh - g->ph + kh;
    if (hi < 0 || hi >= g->h) continue;
    for (int64_t kw = 0; kw < g->kw; ++kw) {
      int64_t wi = wo * g->sw - g->pw + kw;
      if (wi < 0 || wi >= g->w) continue;
      const int8_t *xp = x + ((n * g->h + hi) * g->w + wi) * g->cin + grp * cg;
      const int8_t *wp = wt + ((co * g->kh + kh) * g->kw + kw) * cg;
      for (int64_t ci = 0; ci < cg; ++ci) acc += (int64_t)xp[ci] * (int64_t)wp[ci];
    }
  }
  return acc;
}

/* Requantise one int32 value. Returns the int8 code; *m_out gets the value
 * the rounding was applied to (as double), so the caller can find elements
 * that sit on a rounding tie. */
int oracle_requant(int32_t r32, float s, int act, double *m_out) {
  volatile float f = (float)r32; /* RNE int -> float */
  volatile float v = f * s;      /* one RNE float multiply */
  double m;
  switch (act) {
    case ACT_RELU: {
      float t = v > 0.0f ? v : 0.0f;
      m = (double)t;
      break;
    }
    case ACT_RELU6: {
      float t = v > 0.0f ? (v < 6.0f ? v : 6.0f) : 0.0f;
      m = (double)t;
      break;
    }
    case ACT_MISH: m = oracle_mish((double)v); break;
    default: m = (double)v; break;
  }
  if (m_out) *m_out = m;
  double q = rint(m); /* default rounding mode: nearest, ties to even */
  if (q > 127.0) q = 127.0;
  if (q < -127.0) q = -127.0;
  return (int)q;
}

static int i8_point(const geom_t *g, const int8_t *x, const int8_t *wt,
                    const int32_t *b, const float *s, int act, int out_i32,
                    int64_t nn, int64_t ho, int64_t wo, int64_t co,
                    int32_t *y32, int8_t *y8, double *m, int64_t o) {
  int64_t acc = conv_point_i8(g, x, wt, nn, ho, wo, co);
  if (b) acc += b[co];
  if (acc > 2147483647LL || acc < -2147483648LL) return ORC_E_RANGE;
  int32_t r32 = (int32_t)acc;
  if (out_i32) {
    if (act == ACT_RELU && r32 < 0) r32 = 0;
    y32[o] = r32;
  } else {
    double mm;
    y8[o] = (int8_t)oracle_requant(r32, s[co], act, &mm);
    if (m) m[o] = mm;
  }
  return ORC_OK;
}

/* Full int8 convolution. out_i32 != 0: y32 gets R32 (act NONE or RELU).
 * Otherwise y8 gets the requantised code and m (optional) the pre-rounding
 * value. b may be NULL (zero bias); s is required for int8 output. */
int oracle_conv_i8(const int8_t *x, const int8_t *wt, const int32_t *b,
                   const float *s, int64_t n, int64_t h, int64_t w,
                   int64_t cin, int64_t cout, int64_t kh, int64_t kw,
                   int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                   int64_t groups, int act, int out_i32, int32_t *y32,
                   int8_t *y8, double *m, int nthreads) {
  geom_t g;
  int st = make_geom(&g, n, h, w, cin, cout, kh, kw, sh, sw, ph, pw, groups);
  if (st) return st;
  if (out_i32 && act != ACT_NONE && act != ACT_RELU) return ORC_E_SHAPE;
  if (!out_i32 && !s) return ORC_E_SHAPE;
  set_threads(nthreads);
  int64_t rows = g.n * g.ho;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t row = 0; row < rows; ++row) {
    int64_t nn = row / g.ho, ho = row % g.ho;
    for (int64_t wo = 0; wo < g.wo; ++wo)
      for (int64_t co = 0; co < g.cout; ++co) {
        int64_t o = ((nn * g.ho + ho) * g.wo + wo) * g.cout + co;
        if (i8_point(&g, x, wt, b, s, act, out_i32, nn, ho, wo, co, y32, y8, m, o))
          bad |= 1;
      }
  }
  return bad ? ORC_E_RANGE : ORC_OK;
}

/* Sampled int8 convolution at flat output indices; outputs are indexed by
 * sample position i, not by the flat index. */
int oracle_conv_i8_at(const int8_t *x, const int8_t *wt, const int32_t *b,
                      const float *s, int64_t n, int64_t h, int64_t w,
                      int64_t cin, int64_t cout, int64_t kh, int64_t kw,
                      int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                      int64_t groups, int act, int out_i32,
                      const int64_t *idx, int64_t cnt, int32_t *y32,
                      int8_t *y8, double *m, int nthreads) {
  geom_t g;
  int st = make_geom(&g, n, h, w, cin, cout, kh, kw, sh, sw, ph, pw, groups);
  if (st) return st;
  if (out_i32 && act != ACT_NONE && act != ACT_RELU) return ORC_E_SHAPE;
  if (!out_i32 && !s) return ORC_E_SHAPE;
  int64_t total = g.n * g.ho * g.wo * g.cout;
  for (int64_t i = 0; i < cnt; ++i)
    if (idx[i] < 0 || idx[i] >= total) return ORC_E_SHAPE;
  set_threads(nthreads);
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(| : bad)
  for (int64_t i = 0; i < cnt; ++i) {
    int64_t o = idx[i];
    int64_t co = o % g.cout, t = o / g.cout;
    int64_t wo = t % g.wo;
    t /= g.wo;
    int64_t ho = t % g.ho, nn = t / g.ho;
    if (i8_point(&g, x, wt, b, s, act, out_i32, nn, ho, wo, co, y32, y8, m, i))
      bad |= 1;
  }
  return bad ? ORC_E_RANGE : ORC_OK;
}

/* ------------------------------------------------------------- mosaic -- */

/* IEEE binary32 -> bfloat16 bits, round to nearest, ties to even; NaN stays
 * a quiet NaN. This is the textbook definition of RNE truncation of the low
 * 16 mantissa bits. */
uint16_t oracle_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu))
    return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/* tiles: [4*m][th][tw][c] float; canvas: [m][2th][2tw][c_pad].
 * Tile 4i+0 goes top-left, 4i+1 top-right, 4i+2 bottom-left, 4i+3
 * bottom-right of canvas i; channels c..c_pad-1 are zero.
 * out_bf16 != 0: canvas holds bf16 bits (uint16); else float. */
int oracle_mosaic(const float *tiles, int64_t m, int64_t th, int64_t tw,
                  int64_t c, int64_t c_pad, int out_bf16, void *canvas) {
  if (m <= 0 || th <= 0 || tw <= 0 || c <= 0 || c_pad < c) return ORC_E_SHAPE;
  for (int64_t i = 0; i < m; ++i)
    for (int64_t y = 0; y < 2 * th; ++y)
      for (int64_t x = 0; x < 2 * tw; ++x) {
        int64_t quad = 2 * (y >= th) + (x >= tw);
        const float *src =
            tiles + (((4 * i + quad) * th + (y % th)) * tw + (x % tw)) * c;
        int64_t o = ((i * 2 * th + y) * 2 * tw + x) * c_pad;
        for (int64_t ch = 0; ch < c_pad; ++ch) {
          float v = ch < c ? src[ch] : 0.0f;
          if (out_bf16)
            ((uint16_t *)canvas)[o + ch] = oracle_f32_to_bf16(v);
          else
            ((float *)canvas)[o + ch] = v;
        }
      }
  return ORC_OK;
}

/*
 * SPP max-pool block (zerolat.eu YOLOv4 report, section 9 "Four custom Tensix
 * kernels", K3: the 5, 9 and 13 spatial max-pool windows of the SPP block; section 3
 * names SPP as the block that combines local and wider context with those
 * three windows). Written from the definition of a stride-1 max pool whose
 * output has the input's size, NOT from the cascade identity the report's
 * kernel uses:
 *
 *   P_k[n,h,w,c] = max { X[n,h',w',c] : |h'-h| <= k/2, |w'-w| <= k/2,
 *                        0 <= h' < H, 0 <= w' < W }          k = 5, 9, 13
 *
 * (positions outside the image never win: padding with -infinity).
 * Output y[n,h,w, j*C + c], channel blocks j = 0, 1, 2, 3 = P13, P9, P5, X.
 * dtype 0: float32; 1: bf16 bit patterns, compared as the values they
 * encode; 2: int8. Values are compared with '>', so of equal values the first
 * in (h', w') scan order is kept (this matters only for -0 against +0).
 */
static double spp_val(const void *x, int dtype, int64_t i) {
  if (dtype == 0) return ((const float *)x)[i];
  if (dtype == 1) {
    uint32_t b = (uint32_t)((const uint16_t *)x)[i] << 16;
    float f;
    memcpy(&f, &b, 4);
    return f;
  }
  return ((const int8_t *)x)[i];
}

static void spp_put(const void *x, int dtype, int64_t src, void *y, int64_t dst) {
  if (dtype == 0)
    ((float *)y)[dst] = ((const float *)x)[src];
  else if (dtype == 1)
    ((uint16_t *)y)[dst] = ((const uint16_t *)x)[src];
  else
    ((int8_t *)y)[dst] = ((const int8_t *)x)[src];
}

int oracle_spp(const void *x, int dtype, int64_t n, int64_t h, int64_t w, int64_t c, void *y) {
  if (n <= 0 || h <= 0 || w <= 0 || c <= 0 || dtype < 0 || dtype > 2) return ORC_E_SHAPE;
  static const int kWin[3] = {13, 9, 5};
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t in = 0; in < n; ++in)
    for (int64_t ih = 0; ih < h; ++ih)
      for (int64_t iw = 0; iw < w; ++iw)
        for (int64_t ic = 0; ic < c; ++ic) {
          const int64_t out_px = ((in * h + ih) * w + iw) * 4 * c;
          for (int j = 0; j < 3; ++j) {
            const int64_t r = kWin[j] / 2;
            int64_t best = -1;
            double bv = 0.0;
            for (int64_t hh = ih - r; hh <= ih + r; ++hh)
              for (int64_t ww = iw - r; ww <= iw + r; ++ww) {
                if (hh < 0 || hh >= h || ww < 0 || ww >= w) continue;
                const int64_t src = ((in * h + hh) * w + ww) * c + ic;
                const double v = spp_val(x, dtype, src);
                if (best < 0 || v > bv) {
                  best = src;
                  bv = v;
                }
              }
            spp_put(x, dtype, best, y, out_px + j * c + ic);
          }
          spp_put(x, dtype, ((in * h + ih) * w + iw) * c + ic, y, out_px + 3 * c + ic);
        }
  return ORC_OK;
}

/*
 * Upsample x2 + concat (zerolat.eu YOLOv4 report, section 9 "Four custom Tensix
 * kernels", K4: two neck feature maps, one repeated 2x in rows and columns, joined
 * along channels into the next convolution's input). Two sources s = 0, 1,
 * each [n][ho >> up_s][wo >> up_s][c_s] (up_s = 1: nearest-neighbour 2x
 * upsampling, every source pixel feeds a 2x2 block; up_s = 0: same size),
 * written one after the other along channels:
 *   y[n,i,j, k]        = S0[n, i >> up0, j >> up0, k]          k < c0
 *   y[n,i,j, c0 + k]   = S1[n, i >> up1, j >> up1, k]          k < c1
 * A byte copy: esz is the element size (any dtype).
 */
int oracle_upcat(const void *s0, int64_t c0, int up0, const void *s1, int64_t c1, int up1, int64_t esz,
                 int64_t n, int64_t ho, int64_t wo, void *y) {
  if (n <= 0 || ho <= 0 || wo <= 0 || c0 <= 0 || c1 <= 0 || esz <= 0) return ORC_E_SHAPE;
  if (((up0 || up1) && (ho % 2 || wo % 2)) || up0 < 0 || up0 > 1 || up1 < 0 || up1 > 1) return ORC_E_SHAPE;
  const int64_t ct = c0 + c1;
  for (int64_t in = 0; in < n; ++in)
    for (int64_t i = 0; i < ho; ++i)
      for (int64_t j = 0; j < wo; ++j)
        for (int64_t k = 0; k < ct; ++k) {
          const int s = k >= c0;
          const int up = s ? up1 : up0;
          const int64_t c = s ? c1 : c0, kk = s ? k - c0 : k;
          const int64_t hs = ho >> up, ws = wo >> up;
          const int64_t src = ((in * hs + (i >> up)) * ws + (j >> up)) * c + kk;
          const int64_t dst = ((in * ho + i) * wo + j) * ct + k;
          memcpy((char *)y + dst * esz, (const char *)(s ? s1 : s0) + src * esz, (size_t)esz);
        }
  return ORC_OK;
}

int oracle_num_threads(int nthreads) { return set_threads(nthreads); }
