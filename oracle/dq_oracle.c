/*
 * dq_oracle.c -- plain, slow CPU oracle for the D-Quant hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; it shares no code, header, table or constant generator
 * with kv_cache_entropy_amd/csrc.  Only tests/, __graft_entry__.smoke() and
 * the cpu_baseline leg of bench.py use it (through oracle/__init__.py).
 *
 * Source of the method: the pages
 *   [P1] "D-Quant: Entropy Coding Meets KV Cache at 2.26 Bits" (aimodeling.com
 *        news item, English translation), sections "Why Fixed Width Is a
 *        Ceiling", "Drift: Bending Variable Back to Fixed", "The Numbers".
 *   [P2] "D-Quant: Driftable Entropy Coding for KV Cache Quantization"
 *        (arxivdaily.com listing, abstract), same abstract on fugumt.com.
 * The pages give the pipeline only in words (rotate, normalise, quantise with
 * an analytic N(0,1) model, rANS into a fixed byte container, drift symbols to
 * a cheaper neighbour until the stream fits, dequantise inside attention).
 * Every step they leave open is fixed here by a stated reading; each function
 * names the reading it implements.
 *
 * Precision: the pages fix none.  Steps whose result decides an integer (the
 * rotation and norm that decide symbols) are evaluated in fp32 in the order
 * written here, which is the order the GPU encoder uses; everything else
 * (table build, attention) is fp64.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define DQO_D 128              /* head dimension                        */
#define DQO_MBITS 12           /* rANS table precision: M = 4096        */
#define DQO_M (1u << DQO_MBITS)
#define DQO_RANS_LOW (1u << 23) /* state interval [2^23, 2^31)          */
#define DQO_FMIN 16            /* smallest table frequency              */
#define DQO_MAX_LEVELS 16
#define DQO_MAX_C 132          /* 4 state bytes + at most 128 renorm bytes */

/* error codes (same meaning as the library's, chosen independently) */
#define DQO_OK 0
#define DQO_EINVAL -1
#define DQO_EBUDGET -3

/* ------------------------------------------------------------------------ */
/* SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014): output n (0-based) of the stream seeded with
 * `seed` is mix(seed + (n+1)*gamma).  Used only to draw the rotation signs,
 * which the pages call a "rotation" without saying which one [P1, Why Fixed
 * Width Is a Ceiling]; reading: randomized Walsh-Hadamard with SplitMix64
 * signs. */
uint64_t dqo_splitmix64(uint64_t seed, uint64_t n) {
  uint64_t z = seed + (n + 1u) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* sign of coordinate i for kv head g: -1 iff bit (i mod 64) of word
 * splitmix64(seed, 2g + i/64) is set. */
static int sign_neg(uint64_t seed, int g, int i) {
  uint64_t w = dqo_splitmix64(seed, (uint64_t)(2 * g + i / 64));
  return (int)((w >> (i % 64)) & 1u);
}

/* ------------------------------------------------------------------------ */
/* IEEE binary16 from binary64, round to nearest, ties to even (IEEE 754
 * section 4.3.1).  NaN maps to the quiet NaN 0x7E00. */
uint16_t dqo_f16_from_f64(double v) {
  if (isnan(v)) return 0x7E00;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a >= 65520.0) return (uint16_t)(sign | 0x7C00); /* rounds to +-inf */
  double quantum;
  if (a >= 0x1p-14) {
    int e;
    frexp(a, &e);                     /* a = m * 2^e, m in [0.5, 1) */
    quantum = ldexp(1.0, e - 1 - 10); /* 10 fraction bits */
  } else {
    quantum = 0x1p-24; /* subnormal spacing */
  }
  double r = nearbyint(a / quantum) * quantum; /* ties to even */
  if (r == 0.0) return sign;
  if (r < 0x1p-14) return (uint16_t)(sign | (uint16_t)(r / 0x1p-24));
  int e;
  double m = frexp(r, &e); /* r = m * 2^e */
  int E = e - 1;           /* r = (2m) * 2^E, 2m in [1, 2) */
  uint16_t frac = (uint16_t)((2.0 * m - 1.0) * 1024.0);
  return (uint16_t)(sign | ((uint16_t)(E + 15) << 10) | frac);
}

double dqo_f64_from_f16(uint16_t h) {
  int sign = (h >> 15) & 1, E = (h >> 10) & 31, frac = h & 1023;
  double v;
  if (E == 0) v = ldexp((double)frac, -24);
  else if (E == 31) v = frac ? NAN : INFINITY;
  else v = ldexp(1.0 + frac / 1024.0, E - 15);
  return sign ? -v : v;
}

static float f32_from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* ------------------------------------------------------------------------ */
/* Probability model and reconstruction levels.
 *
 * [P1, Drift: Bending Variable Back to Fixed]: after the preprocessing the
 * values are close enough to a standard normal that the probability model
 * is derived analytically, with no calibration data; keys use 8 levels and
 * values 6.
 * Readings: symmetric mid-rise uniform cells of width step64/64 (in units of
 * the per-coordinate standard deviation); magnitude cell m in [0, h) covers
 * [m*step, (m+1)*step), the last cell is open; cell mass from the normal CDF;
 * 12-bit frequencies f_m = max(16, round_half_even(4096*P_m)) per half, the
 * innermost cell absorbing the rounding remainder; reconstruction level is
 * the cell's conditional mean (centroid) rounded to fp16.
 * Symbol order: s = 0 .. L-1 runs from the outermost negative cell to the
 * outermost positive cell; s = h + m for positive values, h - 1 - m for
 * negative ones. */
typedef struct {
  int levels, half, step64, C, hkv;
  uint64_t seed;
  uint32_t freq[DQO_MAX_LEVELS];
  uint32_t cum[DQO_MAX_LEVELS + 1];
  uint16_t recon[DQO_MAX_LEVELS]; /* fp16 bits */
  double mass[DQO_MAX_LEVELS];    /* true cell probability of each symbol */
  int order;                      /* drift order: 0 magnitude, 1 rate-distortion */
  float rd_w[DQO_MAX_LEVELS / 2]; /* rate-distortion weights, magnitude m >= 1 */
} dqo_codec;

static double normal_upper_tail(double t) { /* P(Z >= t), t >= 0 or inf */
  if (isinf(t)) return 0.0;
  return 0.5 * erfc(t / sqrt(2.0));
}
static double normal_pdf(double t) {
  if (isinf(t)) return 0.0;
  return exp(-0.5 * t * t) / sqrt(2.0 * M_PI);
}

/* Fills the table; returns DQO_EINVAL for bad parameters and DQO_EBUDGET when
 * the table cannot meet the two structural conditions the drift search relies
 * on (every frequency >= 16 after the remainder is absorbed; each step inward
 * at least 1.15x more probable, see dqo_codec_check). */
int dqo_table(int levels, int step64, uint32_t *freq, uint32_t *cum,
              uint16_t *recon, double *mass) {
  if (levels < 2 || levels > DQO_MAX_LEVELS || (levels & 1)) return DQO_EINVAL;
  if (step64 < 1 || step64 > 1023) return DQO_EINVAL;
  int h = levels / 2;
  double step = step64 / 64.0;
  double P[DQO_MAX_LEVELS / 2], lam[DQO_MAX_LEVELS / 2];
  int32_t f[DQO_MAX_LEVELS / 2];
  int32_t total = 0;
  for (int m = 0; m < h; m++) {
    double lo = m * step;
    double hi = (m == h - 1) ? INFINITY : (m + 1) * step;
    P[m] = normal_upper_tail(lo) - normal_upper_tail(hi);
    lam[m] = (normal_pdf(lo) - normal_pdf(hi)) / P[m];
    double q = nearbyint(4096.0 * P[m]);
    f[m] = q < DQO_FMIN ? DQO_FMIN : (int32_t)q;
    total += f[m];
  }
  f[0] += 2048 - total;
  if (f[0] < DQO_FMIN) return DQO_EBUDGET;
  for (int m = 1; m < h; m++)
    if (100 * f[m - 1] < 115 * f[m]) return DQO_EBUDGET;
  for (int s = 0; s < levels; s++) {
    int pos = s >= h;
    int m = pos ? s - h : h - 1 - s;
    freq[s] = (uint32_t)f[m];
    recon[s] = dqo_f16_from_f64(pos ? lam[m] : -lam[m]);
    if (mass) mass[s] = P[m];
  }
  cum[0] = 0;
  for (int s = 0; s < levels; s++) cum[s + 1] = cum[s] + freq[s];
  return DQO_OK;
}

/* Worst-case check for the all-innermost vector (every symbol at f_0), which
 * is what the multi-pass drift falls back to and what a zero/degenerate
 * vector encodes to: the rANS length bound 8*B <= sum(log2(M/f)) + 0.0903
 * (see dqo_rans_encode) must leave 4 + B <= C. */
int dqo_codec_init(dqo_codec *c, int levels, int step64, int C, int hkv,
                   uint64_t seed) {
  memset(c, 0, sizeof(*c));
  if (C < 5 || C > DQO_MAX_C || hkv < 1 || hkv > 1024) return DQO_EINVAL;
  int st = dqo_table(levels, step64, c->freq, c->cum, c->recon, c->mass);
  if (st) return st;
  c->levels = levels;
  c->half = levels / 2;
  c->step64 = step64;
  c->C = C;
  c->hkv = hkv;
  c->seed = seed;
  double bits = DQO_D * log2((double)DQO_M / c->freq[c->half]) + 0.0903;
  int bmax = (int)floor(bits / 8.0);
  if (4 + bmax > C) return DQO_EBUDGET;
  /* rate-distortion weight of a move from magnitude m to m - 1: the level
   * gap over the bits it saves, (l_m - l_{m-1}) / log2(f_{m-1} / f_m),
   * evaluated in double and rounded once to fp32 */
  for (int m = 1; m < c->half; m++) {
    double lm = dqo_f64_from_f16(c->recon[c->half + m]);
    double lm1 = dqo_f64_from_f16(c->recon[c->half + m - 1]);
    double bits_saved = log2((double)c->freq[c->half + m - 1] / (double)c->freq[c->half + m]);
    c->rd_w[m] = (float)((lm - lm1) / bits_saved);
  }
  return DQO_OK;
}

int dqo_codec_check(int levels, int step64, int C) {
  dqo_codec c;
  return dqo_codec_init(&c, levels, step64, C, 1, 0);
}

/* ------------------------------------------------------------------------ */
/* rANS, single 32-bit state, byte-wise renormalisation (Duda, "Asymmetric
 * numeral systems", arXiv:1311.2540; streaming form with L = 2^23, b = 2^8).
 * The pages name rANS as the coder that writes each token's K or V symbols
 * into a fixed-size byte container [P1, Drift: Bending Variable Back to
 * Fixed].
 *
 * Encoder: x starts at 2^23; symbols are pushed from i = 127 down to 0; before
 * pushing s, bytes x & 255 are emitted while x >= f_s * 2^19; then
 * x <- floor(x / f_s) * 4096 + (x mod f_s) + cum_s.  Output layout: the final
 * x as 4 little-endian bytes, then the emitted bytes in reverse emission order
 * (the decoder's reading order).
 * Returns the stream length 4 + B and writes min(len, cap) bytes to out. */
int dqo_rans_encode(const uint8_t *sym, const uint32_t *freq,
                    const uint32_t *cum, uint8_t *out, int cap) {
  uint8_t emitted[4 * DQO_D + 8];
  int B = 0;
  uint32_t x = DQO_RANS_LOW;
  for (int i = DQO_D - 1; i >= 0; i--) {
    uint32_t f = freq[sym[i]], c = cum[sym[i]];
    while (x >= (f << 19)) {
      emitted[B++] = (uint8_t)(x & 255u);
      x >>= 8;
    }
    x = (x / f) * DQO_M + (x % f) + c;
  }
  int len = 4 + B;
  uint8_t tmp[4 * DQO_D + 12];
  tmp[0] = (uint8_t)x;
  tmp[1] = (uint8_t)(x >> 8);
  tmp[2] = (uint8_t)(x >> 16);
  tmp[3] = (uint8_t)(x >> 24);
  for (int j = 0; j < B; j++) tmp[4 + j] = emitted[B - 1 - j];
  if (out)
    for (int j = 0; j < len && j < cap; j++) out[j] = tmp[j];
  return len;
}

/* Decoder: x = the 4 leading bytes (little endian); for i = 0 .. 127:
 * slot = x mod 4096, s = the symbol with cum_s <= slot < cum_{s+1},
 * x <- f_s * (x >> 12) + slot - cum_s, and if x < 2^23 one byte is shifted in
 * (bytes past the end of the C-byte container read as 0).  With every
 * frequency >= 16 a valid stream never needs more than one byte per step.
 * Reports the final state (2^23 for a valid container) and the number of
 * container bytes consumed. */
void dqo_rans_decode(const uint8_t *cont, int C, int levels,
                     const uint32_t *freq, const uint32_t *cum, uint8_t *sym,
                     uint32_t *final_state, int *consumed) {
  uint32_t x = (uint32_t)cont[0] | ((uint32_t)cont[1] << 8) |
               ((uint32_t)cont[2] << 16) | ((uint32_t)cont[3] << 24);
  int p = 4;
  for (int i = 0; i < DQO_D; i++) {
    uint32_t slot = x & (DQO_M - 1);
    int s = 0;
    while (!(cum[s] <= slot && slot < cum[s + 1])) s++;
    sym[i] = (uint8_t)s;
    x = freq[s] * (x >> DQO_MBITS) + slot - cum[s];
    if (x < DQO_RANS_LOW) {
      uint32_t b = p < C ? cont[p] : 0u;
      x = (x << 8) | b;
      p++;
    }
  }
  (void)levels;
  if (final_state) *final_state = x;
  if (consumed) *consumed = p;
}

/* ------------------------------------------------------------------------ */
/* Rotation and normalisation [P1, Why Fixed Width Is a Ceiling; P2, abstract]:
 * the pages rotate and normalise each vector so its coordinates look
 * N(0,1).  Reading: y = H * D * x with D = diag(+-1) from the seeded signs and
 * H the unnormalised 128x128 Sylvester-Hadamard matrix, evaluated in fp32 as
 * the fast transform with butterfly widths 1, 2, ..., 64; the norm is
 * ||x||_2, whose square is summed in fp32 by halving (i + 64, i + 32, ...),
 * stored as the fp16 nearest to its exact square root; each coordinate of
 * y / n_h then has unit variance (||y|| = sqrt(128) * ||x||). */
static void rotate_f32(const float *x, uint64_t seed, int g, float *y) {
  for (int i = 0; i < DQO_D; i++) y[i] = sign_neg(seed, g, i) ? -x[i] : x[i];
  for (int w = 1; w < DQO_D; w <<= 1)
    for (int i = 0; i < DQO_D; i++)
      if ((i & w) == 0) {
        float a = y[i], b = y[i + w];
        y[i] = a + b;
        y[i + w] = a - b;
      }
}

static uint16_t norm_f16(const float *x) {
  float a[DQO_D];
  for (int i = 0; i < DQO_D; i++) a[i] = x[i] * x[i];
  for (int w = DQO_D / 2; w >= 1; w >>= 1)
    for (int i = 0; i < w; i++) a[i] = a[i] + a[i + w];
  return dqo_f16_from_f64(sqrt((double)a[0]));
}

/* ------------------------------------------------------------------------ */
/* Per-vector result detail, for tests. */
typedef struct {
  uint16_t norm;         /* stored fp16 norm */
  int32_t len0;          /* stream length before drift */
  int32_t len;           /* final stream length (<= C) */
  int32_t moves;         /* symbol moves made by drift (one level each) */
  int32_t passes;        /* extra drift passes beyond the first (multilevel) */
  int32_t degenerate;    /* 1: zero norm, 2: inf/nan norm */
  uint8_t sym0[DQO_D];   /* symbols before drift */
  uint8_t sym[DQO_D];    /* symbols stored */
  float y[DQO_D];        /* rotated fp32 coordinates */
} dqo_vec_detail;

/* Quantisation [P1, Drift: Bending Variable Back to Fixed: 8 / 6 levels]:
 * the cell count m_i = #{k in 1..h-1 : |y_i| >= k*step*n_h} with the product
 * k*step*n_h exact in fp32; s = h + m for y >= 0 (so -0.0 is positive), else
 * h - 1 - m.  A vector whose stored norm is 0, inf or NaN is coded as all h
 * (innermost positive level) with no drift.
 *
 * Drift [P1, Drift: Bending Variable Back to Fixed; P2, abstract]: when the
 * stream does not fit the C-byte container, some symbols move from a costly
 * level to the adjacent cheaper one until it fits; the pages report that no
 * moved symbol goes more than one level.  Readings: the cheaper neighbour is
 * one level toward zero (innermost pair never moves); candidates are symbols
 * with m >= 1 ordered by m descending, then |y| ascending (fp32 compare), then
 * index ascending; the result is the smallest k >= 1 such that moving the
 * first k candidates one level inward fits.  If even all of them do not fit,
 * all are moved and the search repeats on the new symbols (a multilevel
 * event; the codec check guarantees the all-innermost vector fits). */
/* Rate-distortion drift order (an option beside the pages' order; the pages
 * point to the rate-distortion toolbox of video coding [P1, So What]).  Moving |y| = a
 * from magnitude m to m - 1 adds n (l_m - l_{m-1}) (2a - n (l_m + l_{m-1}))
 * to the squared error (l = fp16 levels, n = stored norm); dropping the
 * common factor n and dividing by the bits saved gives the key
 *   key = (2a - n (l_m + l_{m-1})) * w_m,
 * computed in fp32: n (l_m + l_{m-1}) is exact (11 x 12 significant bits),
 * then one rounding for the difference and one for the product.
 * Candidates are taken in ascending key, then ascending index. */
static float rd_key(const dqo_codec *c, int m, float a, float nf) {
  float lm = (float)dqo_f64_from_f16(c->recon[c->half + m]);
  float lm1 = (float)dqo_f64_from_f16(c->recon[c->half + m - 1]);
  float t = nf * (lm + lm1);
  float u = 2.0f * a - t;
  return u * c->rd_w[m];
}

/* Does candidate i come before candidate j in the codec's drift order? */
static int drift_before(const dqo_codec *c, const uint8_t *mlev, const float *y,
                        float nf, int i, int j) {
  float ai = fabsf(y[i]), aj = fabsf(y[j]);
  if (c->order == 1) {
    float ki = rd_key(c, mlev[i], ai, nf), kj = rd_key(c, mlev[j], aj, nf);
    return ki < kj || (ki == kj && i < j);
  }
  return mlev[i] > mlev[j] || (mlev[i] == mlev[j] && (ai < aj || (ai == aj && i < j)));
}

static void encode_vector(const dqo_codec *c, const uint16_t *xb, int g,
                          uint8_t *cont, dqo_vec_detail *d) {
  float x[DQO_D], y[DQO_D];
  for (int i = 0; i < DQO_D; i++) x[i] = f32_from_bf16(xb[i]);
  rotate_f32(x, c->seed, g, y);
  uint16_t nh = norm_f16(x);
  double nf = dqo_f64_from_f16(nh);
  const int h = c->half;
  uint8_t s[DQO_D], mlev[DQO_D];
  int degenerate = 0;
  if (nf == 0.0) degenerate = 1;
  else if (isinf(nf) || isnan(nf)) degenerate = 2;
  if (degenerate) {
    for (int i = 0; i < DQO_D; i++) { s[i] = (uint8_t)h; mlev[i] = 0; }
  } else {
    float thr[DQO_MAX_LEVELS / 2];
    for (int k = 1; k < h; k++) thr[k] = (float)((double)(k * c->step64) * nf / 64.0);
    for (int i = 0; i < DQO_D; i++) {
      float ay = fabsf(y[i]);
      int m = 0;
      for (int k = 1; k < h; k++)
        if (ay >= thr[k]) m++;
      mlev[i] = (uint8_t)m;
      s[i] = (uint8_t)(y[i] >= 0.0f ? h + m : h - 1 - m);
    }
  }
  if (d) {
    memcpy(d->sym0, s, DQO_D);
    memcpy(d->y, y, sizeof(y));
  }
  int len = dqo_rans_encode(s, c->freq, c->cum, NULL, 0);
  int len0 = len, moves = 0, passes = 0;
  while (len > c->C) {
    /* candidate list in drift order (selection sort: plain and obviously
     * ordered by the stated key) */
    int cand[DQO_D], n = 0;
    for (int i = 0; i < DQO_D; i++)
      if (mlev[i] >= 1) cand[n++] = i;
    for (int a = 0; a < n; a++) {
      int best = a;
      for (int b = a + 1; b < n; b++)
        if (drift_before(c, mlev, y, (float)nf, cand[b], cand[best])) best = b;
      int t = cand[a]; cand[a] = cand[best]; cand[best] = t;
    }
    uint8_t trial[DQO_D];
    int found = 0;
    for (int k = 1; k <= n; k++) {
      memcpy(trial, s, DQO_D);
      for (int a = 0; a < k; a++) {
        int i = cand[a];
        trial[i] = (uint8_t)(trial[i] >= h ? trial[i] - 1 : trial[i] + 1);
      }
      len = dqo_rans_encode(trial, c->freq, c->cum, NULL, 0);
      if (len <= c->C) {
        for (int a = 0; a < k; a++) mlev[cand[a]]--;
        memcpy(s, trial, DQO_D);
        moves += k;
        found = 1;
        break;
      }
    }
    if (!found) { /* all n moved and still too long: next pass */
      for (int a = 0; a < n; a++) mlev[cand[a]]--;
      memcpy(s, trial, DQO_D);
      moves += n;
      passes++;
    }
  }
  memset(cont, 0, (size_t)c->C);
  dqo_rans_encode(s, c->freq, c->cum, cont, c->C);
  if (d) {
    d->norm = nh;
    d->len0 = len0;
    d->len = len;
    d->moves = moves;
    d->passes = passes;
    d->degenerate = degenerate;
    memcpy(d->sym, s, DQO_D);
  }
}

/* stats layout (uint64): [0] vectors, [1] drifted vectors, [2] moved symbols,
 * [3] multilevel events, [4] inf/nan norms, [5] zero norms,
 * [6 + L] count of final stream length L, L = 0 .. 132 */
#define DQO_NSTATS (6 + DQO_MAX_C + 1)

/* Batch encode of x[T][Hkv][128] (bf16 bits, element strides stride_t and
 * stride_h) into cont[Hkv][num_slots][C] and norm[Hkv][num_slots] at the
 * given slots.  Returns DQO_OK or a negative code. */
int dqo_encode(int levels, int step64, int C, int hkv, uint64_t seed, int order,
               const uint16_t *x, int64_t T, int64_t stride_t, int64_t stride_h,
               const int64_t *slots, int64_t num_slots, uint8_t *cont,
               uint16_t *norm, uint64_t *stats, int nthreads) {
  dqo_codec c;
  int st = dqo_codec_init(&c, levels, step64, C, hkv, seed);
  if (st) return st;
  if (order != 0 && order != 1) return DQO_EINVAL;
  c.order = order;
  for (int64_t t = 0; t < T; t++)
    if (slots[t] < 0 || slots[t] >= num_slots) return DQO_EINVAL;
  uint64_t acc[DQO_NSTATS];
  memset(acc, 0, sizeof(acc));
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
  int64_t nvec = T * hkv;
#pragma omp parallel
  {
    uint64_t loc[DQO_NSTATS];
    memset(loc, 0, sizeof(loc));
#pragma omp for schedule(dynamic, 64)
    for (int64_t v = 0; v < nvec; v++) {
      int64_t t = v / hkv;
      int g = (int)(v % hkv);
      uint16_t xb[DQO_D];
      for (int i = 0; i < DQO_D; i++) xb[i] = x[t * stride_t + g * stride_h + i];
      dqo_vec_detail d;
      int64_t slot = slots[t];
      encode_vector(&c, xb, g, cont + ((int64_t)g * num_slots + slot) * C, &d);
      norm[(int64_t)g * num_slots + slot] = d.norm;
      loc[0] += 1;
      loc[1] += d.moves > 0;
      loc[2] += (uint64_t)d.moves;
      loc[3] += (uint64_t)d.passes;
      loc[4] += d.degenerate == 2;
      loc[5] += d.degenerate == 1;
      loc[6 + d.len] += 1;
    }
#pragma omp critical
    for (int k = 0; k < DQO_NSTATS; k++) acc[k] += loc[k];
  }
  if (stats)
    for (int k = 0; k < DQO_NSTATS; k++) stats[k] += acc[k];
  return DQO_OK;
}

/* Single-vector encode with full detail (tests). */
int dqo_encode_detail(int levels, int step64, int C, int hkv, uint64_t seed,
                      int order, int g, const uint16_t *xb, uint8_t *cont,
                      dqo_vec_detail *d) {
  dqo_codec c;
  int st = dqo_codec_init(&c, levels, step64, C, hkv, seed);
  if (st) return st;
  if (order != 0 && order != 1) return DQO_EINVAL;
  c.order = order;
  if (g < 0 || g >= hkv) return DQO_EINVAL;
  encode_vector(&c, xb, g, cont, d);
  return DQO_OK;
}

int dqo_detail_size(void) { return (int)sizeof(dqo_vec_detail); }

/* Container -> symbols for n containers of kv head `head` at `slots`. */
int dqo_decode_symbols(int levels, int step64, int C, const uint8_t *cont,
                       int64_t num_slots, int head, int hkv,
                       const int64_t *slots, int64_t n, uint8_t *sym,
                       uint32_t *final_state, int32_t *consumed) {
  dqo_codec c;
  int st = dqo_codec_init(&c, levels, step64, C, hkv, 0);
  if (st) return st;
  for (int64_t j = 0; j < n; j++) {
    if (slots[j] < 0 || slots[j] >= num_slots) return DQO_EINVAL;
    const uint8_t *p = cont + ((int64_t)head * num_slots + slots[j]) * C;
    uint32_t fs;
    int cons;
    dqo_rans_decode(p, C, levels, c.freq, c.cum, sym + j * DQO_D, &fs, &cons);
    if (final_state) final_state[j] = fs;
    if (consumed) consumed[j] = cons;
  }
  return DQO_OK;
}

/* ------------------------------------------------------------------------ */
/* Dequantisation and decode attention, fp64, from the plain definitions.
 * [P2, abstract]: the fixed-size streams allow regular memory access and
 * parallel dequantisation inside the attention kernel; [P1, intro and So
 * What]: entropy decoding sits inside attention.
 * Dequantised vector: xhat = D * H * (n_h * r(s)) / 128, the exact inverse of
 * the rotation (H * H = 128 I) applied to the fp16 reconstruction levels
 * r(s) scaled by the fp16 norm; H is applied as the dense matrix
 * H_ij = (-1)^popcount(i & j).
 * Attention (readings: GQA with consecutive query heads sharing a kv head,
 * one query token per sequence): out[b,h] = sum_t softmax_t(sm_scale *
 * q[b,h] . khat_t) vhat_t over t < seq_len[b], kv head g = h / (Hq / Hkv). */
static void dequant_vector(const dqo_codec *c, const uint8_t *cont,
                           uint16_t nh, int g, double *out) {
  uint8_t s[DQO_D];
  dqo_rans_decode(cont, c->C, c->levels, c->freq, c->cum, s, NULL, NULL);
  double n = dqo_f64_from_f16(nh), r[DQO_D];
  for (int j = 0; j < DQO_D; j++) r[j] = n * dqo_f64_from_f16(c->recon[s[j]]);
  for (int i = 0; i < DQO_D; i++) {
    double acc = 0.0;
    for (int j = 0; j < DQO_D; j++)
      acc += (__builtin_popcount((unsigned)(i & j)) & 1) ? -r[j] : r[j];
    out[i] = (sign_neg(c->seed, g, i) ? -acc : acc) / 128.0;
  }
}

int dqo_dequant(int levels, int step64, int C, int hkv, uint64_t seed,
                const uint8_t *cont, const uint16_t *norm, int64_t num_slots,
                int head, const int64_t *slots, int64_t n, double *out) {
  dqo_codec c;
  int st = dqo_codec_init(&c, levels, step64, C, hkv, seed);
  if (st) return st;
  for (int64_t j = 0; j < n; j++) {
    int64_t idx = (int64_t)head * num_slots + slots[j];
    dequant_vector(&c, cont + idx * C, norm[idx], head, out + j * DQO_D);
  }
  return DQO_OK;
}

typedef struct {
  int levels, step64, C;
  uint64_t seed;
} dqo_codec_args;

/* Slot of token t of sequence b: contiguous (seq_start) or paged (page
 * table of 64-token pages, a block table; every container stays at
 * cont + (g * S + slot) * C, the fixed stride the pages rely on). */
typedef struct {
  const int64_t *seq_start; /* contiguous layout, or NULL */
  const int32_t *pages;     /* [B][max_pages] page ids, or NULL */
  int max_pages;
} slot_map;

#define DQO_PAGE 64

static int64_t slot_of(const slot_map *m, int b, int64_t t) {
  if (m->pages)
    return (int64_t)m->pages[(int64_t)b * m->max_pages + t / DQO_PAGE] * DQO_PAGE + t % DQO_PAGE;
  return m->seq_start[b] + t;
}

static int attention_impl(dqo_codec_args ka, dqo_codec_args va, int hkv,
                          const uint16_t *q, int B, int Hq, const uint8_t *kc,
                          const uint16_t *kn, const uint8_t *vc,
                          const uint16_t *vn, int64_t num_slots,
                          const slot_map *map, const int32_t *seq_len,
                          double sm_scale, double *out, int nthreads) {
  dqo_codec ck, cv;
  int st = dqo_codec_init(&ck, ka.levels, ka.step64, ka.C, hkv, ka.seed);
  if (st) return st;
  st = dqo_codec_init(&cv, va.levels, va.step64, va.C, hkv, va.seed);
  if (st) return st;
  if (B < 0 || Hq < 1 || Hq % hkv) return DQO_EINVAL;
  for (int b = 0; b < B; b++) {
    if (seq_len[b] < 1) return DQO_EINVAL;
    if (map->pages) {
      if ((int64_t)seq_len[b] > (int64_t)map->max_pages * DQO_PAGE) return DQO_EINVAL;
      for (int64_t p = 0; p < ((int64_t)seq_len[b] + DQO_PAGE - 1) / DQO_PAGE; p++) {
        int32_t id = map->pages[(int64_t)b * map->max_pages + p];
        if (id < 0 || ((int64_t)id + 1) * DQO_PAGE > num_slots) return DQO_EINVAL;
      }
    } else if (map->seq_start[b] < 0 || map->seq_start[b] + seq_len[b] > num_slots) {
      return DQO_EINVAL;
    }
  }
  int group = Hq / hkv;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bg = 0; bg < (int64_t)B * hkv; bg++) {
    int b = (int)(bg / hkv), g = (int)(bg % hkv);
    int64_t L = seq_len[b];
    double *kh = malloc(sizeof(double) * (size_t)L * DQO_D);
    double *vh = malloc(sizeof(double) * (size_t)L * DQO_D);
    double *sc = malloc(sizeof(double) * (size_t)L);
    for (int64_t t = 0; t < L; t++) {
      int64_t idx = (int64_t)g * num_slots + slot_of(map, b, t);
      dequant_vector(&ck, kc + idx * ck.C, kn[idx], g, kh + t * DQO_D);
      dequant_vector(&cv, vc + idx * cv.C, vn[idx], g, vh + t * DQO_D);
    }
    for (int hh = 0; hh < group; hh++) {
      int h = g * group + hh;
      double qv[DQO_D];
      for (int i = 0; i < DQO_D; i++)
        qv[i] = (double)f32_from_bf16(q[((int64_t)b * Hq + h) * DQO_D + i]);
      double mx = -INFINITY;
      for (int64_t t = 0; t < L; t++) {
        double a = 0.0;
        for (int i = 0; i < DQO_D; i++) a += qv[i] * kh[t * DQO_D + i];
        sc[t] = sm_scale * a;
        if (sc[t] > mx) mx = sc[t];
      }
      double den = 0.0, o[DQO_D];
      for (int i = 0; i < DQO_D; i++) o[i] = 0.0;
      for (int64_t t = 0; t < L; t++) {
        double p = exp(sc[t] - mx);
        den += p;
        for (int i = 0; i < DQO_D; i++) o[i] += p * vh[t * DQO_D + i];
      }
      for (int i = 0; i < DQO_D; i++)
        out[((int64_t)b * Hq + h) * DQO_D + i] = o[i] / den;
    }
    free(kh);
    free(vh);
    free(sc);
  }
  return DQO_OK;
}

int dqo_attention(dqo_codec_args ka, dqo_codec_args va, int hkv,
                  const uint16_t *q /* bf16 [B][Hq][128] */, int B, int Hq,
                  const uint8_t *kc, const uint16_t *kn, const uint8_t *vc,
                  const uint16_t *vn, int64_t num_slots,
                  const int64_t *seq_start, const int32_t *seq_len,
                  double sm_scale, double *out /* [B][Hq][128] */,
                  int nthreads) {
  slot_map m = {seq_start, NULL, 0};
  return attention_impl(ka, va, hkv, q, B, Hq, kc, kn, vc, vn, num_slots, &m,
                        seq_len, sm_scale, out, nthreads);
}

/* Chunked-prefill attention over the compressed cache (the pages' serving
 * figures include an 8K prompt [P1, The Numbers]).
 * Reading: a chunk of Tq new tokens has already been encoded at the end of
 * each sequence, so the sequence holds seq_len[b] tokens of which the last
 * Tq are the chunk; query j of sequence b sits at position
 * p = seq_len[b] - Tq + j and attends causally to tokens 0..p, all of
 * them read from their containers.
 * q: bf16 [B][Tq][Hq][128]; out: [B][Tq][Hq][128]. */
int dqo_attention_prefill(dqo_codec_args ka, dqo_codec_args va, int hkv,
                          const uint16_t *q, int B, int Tq, int Hq,
                          const uint8_t *kc, const uint16_t *kn,
                          const uint8_t *vc, const uint16_t *vn,
                          int64_t num_slots, const int64_t *seq_start,
                          const int32_t *seq_len, double sm_scale, double *out,
                          int nthreads) {
  dqo_codec ck, cv;
  int st = dqo_codec_init(&ck, ka.levels, ka.step64, ka.C, hkv, ka.seed);
  if (st) return st;
  st = dqo_codec_init(&cv, va.levels, va.step64, va.C, hkv, va.seed);
  if (st) return st;
  if (B < 0 || Tq < 1 || Hq < 1 || Hq % hkv) return DQO_EINVAL;
  for (int b = 0; b < B; b++)
    if (seq_len[b] < Tq || seq_start[b] < 0 || seq_start[b] + seq_len[b] > num_slots)
      return DQO_EINVAL;
  int group = Hq / hkv;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bg = 0; bg < (int64_t)B * hkv; bg++) {
    int b = (int)(bg / hkv), g = (int)(bg % hkv);
    int64_t L = seq_len[b];
    double *kh = malloc(sizeof(double) * (size_t)L * DQO_D);
    double *vh = malloc(sizeof(double) * (size_t)L * DQO_D);
    double *sc = malloc(sizeof(double) * (size_t)L);
    for (int64_t t = 0; t < L; t++) {
      int64_t idx = (int64_t)g * num_slots + seq_start[b] + t;
      dequant_vector(&ck, kc + idx * ck.C, kn[idx], g, kh + t * DQO_D);
      dequant_vector(&cv, vc + idx * cv.C, vn[idx], g, vh + t * DQO_D);
    }
    for (int j = 0; j < Tq; j++) {
      int64_t pos = L - Tq + j; /* keys 0..pos */
      for (int hh = 0; hh < group; hh++) {
        int h = g * group + hh;
        const uint16_t *qp = q + (((int64_t)b * Tq + j) * Hq + h) * DQO_D;
        double qv[DQO_D];
        for (int i = 0; i < DQO_D; i++) qv[i] = (double)f32_from_bf16(qp[i]);
        double mx = -INFINITY;
        for (int64_t t = 0; t <= pos; t++) {
          double a = 0.0;
          for (int i = 0; i < DQO_D; i++) a += qv[i] * kh[t * DQO_D + i];
          sc[t] = sm_scale * a;
          if (sc[t] > mx) mx = sc[t];
        }
        double den = 0.0, o[DQO_D];
        for (int i = 0; i < DQO_D; i++) o[i] = 0.0;
        for (int64_t t = 0; t <= pos; t++) {
          double p = exp(sc[t] - mx);
          den += p;
          for (int i = 0; i < DQO_D; i++) o[i] += p * vh[t * DQO_D + i];
        }
        double *op = out + (((int64_t)b * Tq + j) * Hq + h) * DQO_D;
        for (int i = 0; i < DQO_D; i++) op[i] = o[i] / den;
      }
    }
    free(kh);
    free(vh);
    free(sc);
  }
  return DQO_OK;
}

/* The same attention over a paged pool: token t of sequence b is in slot
 * pages[b * max_pages + t / 64] * 64 + t % 64. */
int dqo_attention_paged(dqo_codec_args ka, dqo_codec_args va, int hkv,
                        const uint16_t *q, int B, int Hq, const uint8_t *kc,
                        const uint16_t *kn, const uint8_t *vc,
                        const uint16_t *vn, int64_t num_slots,
                        const int32_t *pages, int max_pages,
                        const int32_t *seq_len, double sm_scale, double *out,
                        int nthreads) {
  slot_map m = {NULL, pages, max_pages};
  return attention_impl(ka, va, hkv, q, B, Hq, kc, kn, vc, vn, num_slots, &m,
                        seq_len, sm_scale, out, nthreads);
}

/* table export for tests */
int dqo_codec_tables(int levels, int step64, int C, uint32_t *freq,
                     uint32_t *cum, uint16_t *recon, double *mass) {
  dqo_codec c;
  int st = dqo_codec_init(&c, levels, step64, C, 1, 0);
  if (st) return st;
  for (int s = 0; s < levels; s++) {
    freq[s] = c.freq[s];
    recon[s] = c.recon[s];
    mass[s] = c.mass[s];
  }
  for (int s = 0; s <= levels; s++) cum[s] = c.cum[s];
  return DQO_OK;
}

int dqo_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
