/*
 * oracle.c -- plain, slow, obviously-correct CPU oracle for per-head KV-cache
 * retention scoring, HubKV score refinement, protected Top-K selection, K/V
 * compaction and the H2O streaming eviction step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source,
 * header, helper or constant with the GPU library, and the GPU library never
 * calls it.
 *
 * Rules kept here:
 *   - every floating-point reduction is done in double, in plain loops;
 *   - no SIMD intrinsics, no BLAS, no blocking or reordering beyond the
 *     definitions; OpenMP only across independent (layer, sequence, KV head)
 *     units;
 *   - built with -ffp-contract=off so the fp32 gate arithmetic below is the
 *     exact op sequence written.
 *
 * Readings of points the pages leave open (each is also listed in the design
 * notes of the repository):
 *   R1  scoring queries are the last W positions of each sequence;
 *   R2  causal: window row w of a sequence of length N sees keys i <= N-W+w;
 *   R3  softmax scale is an explicit argument (1/sqrt(d) in every workload);
 *   R4  scores are summed over the W window rows and over the G query heads
 *       that share a KV head (contiguous grouping h -> h / G);
 *   R5  a hub is any token equal to the maximum of its width-`pool` window,
 *       the window truncated at the sequence ends (ties are all hubs);
 *   R6  every non-hub is discounted by gamma;
 *   R7  the gated score is z = s + r^2 (beta * q - s), q the discounted score,
 *       evaluated in fp32 as fmaf(fl(r*r), fl(beta*q) - s, s);
 *   R8  head selectivity = 1 - H(s/sum s)/ln N (normalised negentropy of the
 *       head's base scores); beta = clip(sel / mean_heads(sel), lo, hi), and
 *       beta = 1 when the mean selectivity is not positive;
 *   R9  the kept count k includes sink and recent tokens; Top-K order is
 *       (z descending, position ascending), NaN lowest, -0 == +0; the output
 *       index list is ascending;
 *   R10 H2O step: the query's softmax runs over the cached tokens before the
 *       new token is added (optionally including it), the new token enters
 *       with accumulated score 0 (or its own probability), and when the cache
 *       is over capacity the lowest accumulated score among tokens outside
 *       the sink and recent windows is evicted, ties to the oldest position;
 *   R11 the H2O step's attention output uses those same probabilities on the
 *       values of the same tokens (before the new token is inserted);
 *   R13 NestedKV score: keys are normalised to unit length; the stable
 *       memory is their sequence mean, the episodic memory the mean of
 *       ceil(N / nblocks)-position blocks, the current memory the mean of the
 *       trailing `window` keys (the token itself included); a scale's
 *       discriminative power is the max minus the min of its anomaly over the
 *       head; log_prior and the surprise threshold theta are arguments;
 *   R12 layer-wide budget: the caller gives the kept total of a (layer,
 *       sequence) over all its KV heads; each head first keeps its protected
 *       positions and a floor of its own best candidates, and the rest of
 *       the total goes to the best remaining (head, position) pairs, ties to
 *       the lower head, then the lower position.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_EINVAL -1

static int g_threads = 0;

void orc_set_threads(int n) {
  g_threads = n;
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#endif
}

int orc_get_threads(void) {
#ifdef _OPENMP
  int n = 0;
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
  return n;
#else
  return 1;
#endif
}

static int64_t total_len(int B, const int64_t* seqlens) {
  int64_t T = 0;
  for (int b = 0; b < B; ++b) T += seqlens[b];
  return T;
}

static int64_t seq_start(int b, const int64_t* seqlens) {
  int64_t c = 0;
  for (int i = 0; i < b; ++i) c += seqlens[i];
  return c;
}

/* --------------------------------------------------------------------------
 * Base score: H2O accumulated attention mass over an observation window.
 *
 * H2O breakdown page, "Observation 2": a token's score is the attention
 * probability it receives, summed over query positions.  KV-cache survey page,
 * section 1.1: decode attention is softmax(q K^T / sqrt(d_head)).  KV-cache
 * survey page, section 4.3: the SnapKV variant reads these patterns from the
 * prefill queries.  GQA grouping: KV-cache survey page, section 3.3.
 *
 * q [L][Hq][B*W][d], k [L][Hkv][T][d], s [L][Hkv][T] (fp32, rounded from the
 * double sum), stats [L][B][Hkv][2] = {sum_i s_i, sum_i s_i ln s_i} over the
 * fp32 s of the sequence (0 ln 0 := 0).
 * ------------------------------------------------------------------------ */
int orc_score(const float* q, const float* k, int B, const int64_t* seqlens, int L, int Hq,
              int Hkv, int W, int d, double scale, int causal, float* s, double* stats) {
  if (B <= 0 || L <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || W <= 0 || d <= 0) return ORC_EINVAL;
  for (int b = 0; b < B; ++b)
    if (seqlens[b] < W) return ORC_EINVAL;
  const int G = Hq / Hkv;
  const int64_t T = total_len(B, seqlens);
  const int units = L * B * Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int u = 0; u < units; ++u) {
    const int l = u / (B * Hkv);
    const int b = (u / Hkv) % B;
    const int g = u % Hkv;
    const int64_t N = seqlens[b];
    const int64_t cu = seq_start(b, seqlens);
    double* acc = (double*)calloc((size_t)N, sizeof(double));
    double* x = (double*)malloc((size_t)N * sizeof(double));
    const float* kb = k + ((int64_t)(l * Hkv + g) * T + cu) * d;
    for (int hl = 0; hl < G; ++hl) {
      const int h = g * G + hl;
      for (int w = 0; w < W; ++w) {
        const float* qr = q + ((int64_t)(l * Hq + h) * B * W + (int64_t)b * W + w) * d;
        const int64_t p = N - W + w;              /* absolute position of the query */
        const int64_t nvis = causal ? p + 1 : N;  /* keys 0..nvis-1 are visible */
        double m = -INFINITY;
        for (int64_t i = 0; i < nvis; ++i) {
          const float* kr = kb + i * d;
          double dot = 0.0;
          for (int j = 0; j < d; ++j) dot += (double)qr[j] * (double)kr[j];
          x[i] = scale * dot;
          if (x[i] > m) m = x[i];
        }
        double lsum = 0.0;
        for (int64_t i = 0; i < nvis; ++i) lsum += exp(x[i] - m);
        for (int64_t i = 0; i < nvis; ++i) acc[i] += exp(x[i] - m) / lsum;
      }
    }
    float* so = s + (int64_t)(l * Hkv + g) * T + cu;
    double S = 0.0, A = 0.0;
    for (int64_t i = 0; i < N; ++i) {
      so[i] = (float)acc[i];
      const double v = (double)so[i];
      S += v;
      if (v > 0.0) A += v * log(v);
    }
    if (stats) {
      double* st = stats + (((int64_t)l * B + b) * Hkv + g) * 2;
      st[0] = S;
      st[1] = A;
    }
    free(acc);
    free(x);
  }
  return ORC_OK;
}

/* Head statistics from a given score array (used when scores are supplied
 * directly rather than computed by orc_score). */
int orc_head_stats(const float* s, int B, const int64_t* seqlens, int L, int Hkv, double* stats) {
  const int64_t T = total_len(B, seqlens);
  for (int l = 0; l < L; ++l)
    for (int b = 0; b < B; ++b)
      for (int g = 0; g < Hkv; ++g) {
        const float* so = s + (int64_t)(l * Hkv + g) * T + seq_start(b, seqlens);
        double S = 0.0, A = 0.0;
        for (int64_t i = 0; i < seqlens[b]; ++i) {
          const double v = (double)so[i];
          S += v;
          if (v > 0.0) A += v * log(v);
        }
        double* st = stats + (((int64_t)l * B + b) * Hkv + g) * 2;
        st[0] = S;
        st[1] = A;
      }
  return ORC_OK;
}

/* --------------------------------------------------------------------------
 * Head calibration (HubKV walkthrough, "Method", step 3: a mild head weight
 * from selectivity, clipped to [0.8, 1.2]; the sharp-locator vs flat-background
 * head observation motivates it).  Selectivity formula: reading R8.
 * stats [L][B][Hkv][2] -> beta [L][B][Hkv].
 * ------------------------------------------------------------------------ */
int orc_beta(const double* stats, int B, const int64_t* seqlens, int L, int Hkv, float beta_lo,
             float beta_hi, float* beta) {
  if (!(beta_lo <= beta_hi)) return ORC_EINVAL;
  double* sel = (double*)malloc((size_t)Hkv * sizeof(double));
  for (int l = 0; l < L; ++l)
    for (int b = 0; b < B; ++b) {
      const double lnN = log((double)seqlens[b]);
      double mean = 0.0;
      for (int g = 0; g < Hkv; ++g) {
        const double* st = stats + (((int64_t)l * B + b) * Hkv + g) * 2;
        const double S = st[0], A = st[1];
        double v = 0.0;
        if (seqlens[b] > 1 && S > 0.0) {
          const double H = log(S) - A / S; /* entropy of s / S */
          v = 1.0 - H / lnN;
        }
        sel[g] = v;
        mean += v;
      }
      mean /= (double)Hkv;
      for (int g = 0; g < Hkv; ++g) {
        double bt = 1.0;
        if (mean > 0.0 && isfinite(mean)) {
          bt = sel[g] / mean;
          if (bt < (double)beta_lo) bt = (double)beta_lo;
          if (bt > (double)beta_hi) bt = (double)beta_hi;
        }
        beta[((int64_t)l * B + b) * Hkv + g] = (float)bt;
      }
    }
  free(sel);
  return ORC_OK;
}

/* --------------------------------------------------------------------------
 * Refinement (HubKV walkthrough, "Method", steps 1, 2 and 4):
 *   1. local hubs: a token is a hub when it equals the max over a width-`pool`
 *      window centred on it (max-pooling, width 5 on the page);
 *   2. SMD discount: hubs keep their score, other tokens are scaled by gamma
 *      (0.5 on the page);
 *   4. ratio gate: z = s + r^2 (beta_h q - s), r the compression ratio.
 * s, z [L][Hkv][T]; beta [L][B][Hkv].
 * ------------------------------------------------------------------------ */
int orc_refine(const float* s, float* z, int B, const int64_t* seqlens, int L, int Hkv,
               const float* beta, int pool, float gamma, float r) {
  if (pool < 1 || (pool % 2) == 0) return ORC_EINVAL;
  const int half = pool / 2;
  const int64_t T = total_len(B, seqlens);
  const float r2 = r * r;
  const int units = L * B * Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int u = 0; u < units; ++u) {
    const int l = u / (B * Hkv);
    const int b = (u / Hkv) % B;
    const int g = u % Hkv;
    const int64_t N = seqlens[b];
    const int64_t off = (int64_t)(l * Hkv + g) * T + seq_start(b, seqlens);
    const float bt = beta[((int64_t)l * B + b) * Hkv + g];
    for (int64_t i = 0; i < N; ++i) {
      const int64_t lo = i - half < 0 ? 0 : i - half;
      const int64_t hi = i + half > N - 1 ? N - 1 : i + half;
      float mx = s[off + lo];
      for (int64_t j = lo + 1; j <= hi; ++j)
        if (s[off + j] > mx) mx = s[off + j];
      const float si = s[off + i];
      const int hub = (si == mx);
      const float qi = hub ? si : gamma * si;
      const float t = bt * qi;
      const float dlt = t - si;
      z[off + i] = fmaf(r2, dlt, si);
    }
  }
  return ORC_OK;
}

/* --------------------------------------------------------------------------
 * Protected Top-K (HubKV walkthrough: modular Top-K, F(S) = sum of scores, is
 * what the refined scores are handed to; H2O breakdown page, heavy + recent
 * section and per-head section; KV-cache survey page, sections 4.1-4.2: keep
 * the first sink tokens and the recent window).  Reading R9.
 * z [L][Hkv][T]; kept [B]; idx [L][Hkv][sum kept].
 * ------------------------------------------------------------------------ */
typedef struct {
  float z;
  int64_t pos;
} zpos_t;

static int zpos_cmp(const void* a, const void* b) {
  const zpos_t* x = (const zpos_t*)a;
  const zpos_t* y = (const zpos_t*)b;
  const int xn = isnan(x->z), yn = isnan(y->z);
  if (xn != yn) return xn ? 1 : -1; /* NaN ranks last */
  if (!xn) {
    if (x->z > y->z) return -1; /* descending; -0 == +0 under == */
    if (x->z < y->z) return 1;
  }
  return (x->pos < y->pos) ? -1 : (x->pos > y->pos ? 1 : 0);
}

int64_t orc_protected_count(int64_t N, int n_sink, int n_recent) {
  const int64_t a = n_sink < N ? n_sink : N;         /* [0, a) */
  const int64_t c = N - n_recent > 0 ? N - n_recent : 0; /* [c, N) */
  if (c <= a) return N;
  return a + (N - c);
}

int orc_select(const float* z, int B, const int64_t* seqlens, int L, int Hkv, const int64_t* kept,
               int n_sink, int n_recent, int32_t* idx) {
  if (n_sink < 0 || n_recent < 0) return ORC_EINVAL;
  int64_t K = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t P = orc_protected_count(seqlens[b], n_sink, n_recent);
    if (kept[b] < P || kept[b] > seqlens[b]) return ORC_EINVAL;
    K += kept[b];
  }
  const int64_t T = total_len(B, seqlens);
  const int units = L * B * Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int u = 0; u < units; ++u) {
    const int l = u / (B * Hkv);
    const int b = (u / Hkv) % B;
    const int g = u % Hkv;
    const int64_t N = seqlens[b];
    const float* zb = z + (int64_t)(l * Hkv + g) * T + seq_start(b, seqlens);
    int64_t koff = 0;
    for (int i = 0; i < b; ++i) koff += kept[i];
    int32_t* out = idx + (int64_t)(l * Hkv + g) * K + koff;
    unsigned char* keep = (unsigned char*)calloc((size_t)N, 1);
    zpos_t* cand = (zpos_t*)malloc((size_t)N * sizeof(zpos_t));
    int64_t nc = 0, np = 0;
    for (int64_t i = 0; i < N; ++i) {
      const int prot = (i < n_sink) || (i >= N - n_recent);
      if (prot) {
        keep[i] = 1;
        ++np;
      } else {
        cand[nc].z = zb[i];
        cand[nc].pos = i;
        ++nc;
      }
    }
    qsort(cand, (size_t)nc, sizeof(zpos_t), zpos_cmp);
    const int64_t want = kept[b] - np;
    for (int64_t j = 0; j < want; ++j) keep[cand[j].pos] = 1;
    int64_t o = 0;
    for (int64_t i = 0; i < N; ++i)
      if (keep[i]) out[o++] = (int32_t)i;
    free(keep);
    free(cand);
  }
  return ORC_OK;
}

/* --------------------------------------------------------------------------
 * NestedKV key-only score (NestedKV summary page: the continuum memory state
 * of three key means, the outer teacher's head-adaptive blending and its
 * surprise-gated routing).  Reading R13.  Per (layer l, KV head g, sequence
 * b), with k^_i = k_i / |k_i| (0 for a zero key):
 *   mu_s     the mean of k^ over the sequence;
 *   mu_e(i)  the mean of k^ over i's block, blocks of ceil(N / nblocks)
 *            positions from the start;
 *   mu_c(i)  the mean of k^ over the trailing window [i - window + 1, i];
 *   a_x(i) = -cos(k^_i, mu_x) (0 when either vector is zero);
 *   D_x = max_i a_x - min_i a_x, w = softmax(D + log_prior);
 *   sigma(i) = population standard deviation of (a_s, a_e, a_c);
 *   s_i = max(a_s, a_e, a_c) when sigma(i) > theta, else sum_x w_x a_x.
 * k [L][Hkv][T][d]; s [L][Hkv][T]; anomalies (nullable) [L][Hkv][T][3];
 * weights (nullable) [L][B][Hkv][3].
 * ------------------------------------------------------------------------ */
static double cos_d(const double* x, const double* y, int d) {
  double xy = 0.0, xx = 0.0, yy = 0.0;
  for (int e = 0; e < d; ++e) {
    xy += x[e] * y[e];
    xx += x[e] * x[e];
    yy += y[e] * y[e];
  }
  if (xx == 0.0 || yy == 0.0) return 0.0;
  return xy / (sqrt(xx) * sqrt(yy));
}

int orc_nestedkv(const float* k, int B, const int64_t* seqlens, int L, int Hkv, int d, int nblocks,
                 int window, const double* log_prior, double theta, float* s, float* anomalies,
                 float* weights) {
  if (nblocks < 1 || window < 1 || d < 1) return ORC_EINVAL;
  const int64_t T = total_len(B, seqlens);
  const int units = L * Hkv * B;
#pragma omp parallel for schedule(dynamic, 1)
  for (int u = 0; u < units; ++u) {
    const int l = u / (Hkv * B), g = (u / B) % Hkv, b = u % B;
    const int64_t N = seqlens[b];
    const int64_t row0 = (int64_t)(l * Hkv + g) * T + seq_start(b, seqlens);
    const float* kb = k + row0 * d;
    double* kh = (double*)malloc((size_t)(N * d) * sizeof(double));
    double* a = (double*)malloc((size_t)(N * 3) * sizeof(double));
    double* mu = (double*)calloc((size_t)d, sizeof(double));
    double* me = (double*)malloc((size_t)d * sizeof(double));
    double* mc = (double*)malloc((size_t)d * sizeof(double));
    for (int64_t i = 0; i < N; ++i) {
      double nn = 0.0;
      for (int e = 0; e < d; ++e) nn += (double)kb[i * d + e] * (double)kb[i * d + e];
      const double inv = nn > 0.0 ? 1.0 / sqrt(nn) : 0.0;
      for (int e = 0; e < d; ++e) kh[i * d + e] = (double)kb[i * d + e] * inv;
    }
    /* stable memory */
    for (int64_t i = 0; i < N; ++i)
      for (int e = 0; e < d; ++e) mu[e] += kh[i * d + e];
    for (int e = 0; e < d; ++e) mu[e] /= (double)N;
    const int64_t bs = (N + nblocks - 1) / nblocks;
    for (int64_t i = 0; i < N; ++i) {
      const double* x = kh + i * d;
      /* episodic memory: i's block (its mean is formed once per block) */
      const int64_t m0 = (i / bs) * bs, m1 = m0 + bs < N ? m0 + bs : N;
      if (i == m0) {
        for (int e = 0; e < d; ++e) me[e] = 0.0;
        for (int64_t j = m0; j < m1; ++j)
          for (int e = 0; e < d; ++e) me[e] += kh[j * d + e];
        for (int e = 0; e < d; ++e) me[e] /= (double)(m1 - m0);
      }
      /* current memory: the trailing window */
      const int64_t c0 = i - window + 1 > 0 ? i - window + 1 : 0;
      for (int e = 0; e < d; ++e) mc[e] = 0.0;
      for (int64_t j = c0; j <= i; ++j)
        for (int e = 0; e < d; ++e) mc[e] += kh[j * d + e];
      for (int e = 0; e < d; ++e) mc[e] /= (double)(i - c0 + 1);
      a[i * 3 + 0] = -cos_d(x, mu, d);
      a[i * 3 + 1] = -cos_d(x, me, d);
      a[i * 3 + 2] = -cos_d(x, mc, d);
    }
    /* head-adaptive blend */
    double w[3], D[3];
    for (int x = 0; x < 3; ++x) {
      double lo = a[x], hi = a[x];
      for (int64_t i = 1; i < N; ++i) {
        if (a[i * 3 + x] < lo) lo = a[i * 3 + x];
        if (a[i * 3 + x] > hi) hi = a[i * 3 + x];
      }
      D[x] = hi - lo + (log_prior ? log_prior[x] : 0.0);
    }
    const double dm = D[0] > D[1] ? (D[0] > D[2] ? D[0] : D[2]) : (D[1] > D[2] ? D[1] : D[2]);
    double den = 0.0;
    for (int x = 0; x < 3; ++x) den += exp(D[x] - dm);
    for (int x = 0; x < 3; ++x) w[x] = exp(D[x] - dm) / den;
    if (weights)
      for (int x = 0; x < 3; ++x) weights[(((int64_t)l * B + b) * Hkv + g) * 3 + x] = (float)w[x];
    /* surprise-gated routing */
    for (int64_t i = 0; i < N; ++i) {
      const double* ai = a + i * 3;
      const double mean = (ai[0] + ai[1] + ai[2]) / 3.0;
      const double var = ((ai[0] - mean) * (ai[0] - mean) + (ai[1] - mean) * (ai[1] - mean) +
                          (ai[2] - mean) * (ai[2] - mean)) / 3.0;
      const double sg = sqrt(var);
      double v;
      if (sg > theta) {
        v = ai[0];
        if (ai[1] > v) v = ai[1];
        if (ai[2] > v) v = ai[2];
      } else {
        v = w[0] * ai[0] + w[1] * ai[1] + w[2] * ai[2];
      }
      s[row0 + i] = (float)v;
      if (anomalies)
        for (int x = 0; x < 3; ++x) anomalies[(row0 + i) * 3 + x] = (float)ai[x];
    }
    free(kh);
    free(a);
    free(mu);
    free(me);
    free(mc);
  }
  return ORC_OK;
}

/* --------------------------------------------------------------------------
 * Layer-wide budget (NestedKV summary page, head-wise memory allocation: the
 * layer's budget goes to the globally highest (token, head) pairs, each head
 * keeping a minimum of its own; KV-cache survey page, section 4.4: budgets
 * set per layer).  Reading R12.  Per (layer l, sequence b):
 *   every head keeps the protected positions and its floor: the first
 *   f = min(floor_min, number of candidates) of its candidates in the order
 *   of reading R9 (z descending, position ascending, NaN lowest);
 *   the other candidates of all heads compete for the rest of the budget,
 *   R = layer_kept[l][b] - Hkv * (|P| + f), in (z descending, head
 *   ascending, position ascending) order.
 * z [L][Hkv][T]; layer_kept [L][B] host.  idx: for each (l, b) in row-major
 * order, the heads' kept positions head after head, each ascending;
 * head_kept [L][B][Hkv].
 * ------------------------------------------------------------------------ */
typedef struct {
  float z;
  int64_t pos;
  int head;
} zhp_t;

static int zhp_cmp(const void* a, const void* b) {
  const zhp_t* x = (const zhp_t*)a;
  const zhp_t* y = (const zhp_t*)b;
  const int xn = isnan(x->z), yn = isnan(y->z);
  if (xn != yn) return xn ? 1 : -1;
  if (!xn) {
    if (x->z > y->z) return -1;
    if (x->z < y->z) return 1;
  }
  if (x->head != y->head) return x->head < y->head ? -1 : 1;
  return (x->pos < y->pos) ? -1 : (x->pos > y->pos ? 1 : 0);
}

int orc_select_layer(const float* z, int B, const int64_t* seqlens, int L, int Hkv,
                     const int64_t* layer_kept, int n_sink, int n_recent, int floor_min,
                     int32_t* idx, int32_t* head_kept) {
  if (n_sink < 0 || n_recent < 0 || floor_min < 0 || Hkv < 1) return ORC_EINVAL;
  for (int l = 0; l < L; ++l)
    for (int b = 0; b < B; ++b) {
      const int64_t N = seqlens[b];
      const int64_t P = orc_protected_count(N, n_sink, n_recent);
      const int64_t f = floor_min < N - P ? floor_min : N - P;
      const int64_t k = layer_kept[(int64_t)l * B + b];
      if (k < (int64_t)Hkv * (P + f) || k > (int64_t)Hkv * N) return ORC_EINVAL;
    }
  const int64_t T = total_len(B, seqlens);
  const int units = L * B;
#pragma omp parallel for schedule(dynamic, 1)
  for (int u = 0; u < units; ++u) {
    const int l = u / B, b = u % B;
    const int64_t N = seqlens[b];
    const int64_t P = orc_protected_count(N, n_sink, n_recent);
    const int64_t f = floor_min < N - P ? floor_min : N - P;
    int64_t off = 0;
    for (int v = 0; v < u; ++v) off += layer_kept[v];
    unsigned char* keep = (unsigned char*)calloc((size_t)(Hkv * N), 1);
    zpos_t* cand = (zpos_t*)malloc((size_t)N * sizeof(zpos_t));
    zhp_t* pool = (zhp_t*)malloc((size_t)(Hkv * N) * sizeof(zhp_t));
    int64_t np = 0;
    for (int g = 0; g < Hkv; ++g) {
      const float* zb = z + (int64_t)(l * Hkv + g) * T + seq_start(b, seqlens);
      unsigned char* kg = keep + (int64_t)g * N;
      int64_t nc = 0;
      for (int64_t i = 0; i < N; ++i) {
        if ((i < n_sink) || (i >= N - n_recent)) {
          kg[i] = 1;
        } else {
          cand[nc].z = zb[i];
          cand[nc].pos = i;
          ++nc;
        }
      }
      qsort(cand, (size_t)nc, sizeof(zpos_t), zpos_cmp);
      for (int64_t j = 0; j < nc; ++j) {
        if (j < f) {
          kg[cand[j].pos] = 1; /* the head's floor */
        } else {
          pool[np].z = cand[j].z;
          pool[np].pos = cand[j].pos;
          pool[np].head = g;
          ++np;
        }
      }
    }
    qsort(pool, (size_t)np, sizeof(zhp_t), zhp_cmp);
    const int64_t R = layer_kept[u] - (int64_t)Hkv * (P + f);
    for (int64_t j = 0; j < R; ++j) keep[(int64_t)pool[j].head * N + pool[j].pos] = 1;
    int64_t o = off;
    for (int g = 0; g < Hkv; ++g) {
      int32_t n = 0;
      for (int64_t i = 0; i < N; ++i)
        if (keep[(int64_t)g * N + i]) {
          idx[o++] = (int32_t)i;
          ++n;
        }
      head_kept[(int64_t)u * Hkv + g] = n;
    }
    free(keep);
    free(cand);
    free(pool);
  }
  return ORC_OK;
}

/* --------------------------------------------------------------------------
 * Compaction: physically drop evicted K/V rows (H2O breakdown page, "two code
 * bases": the real-drop variant removes evicted tokens' K/V from the cache).
 * k_in/v_in [L][Hkv][T][d], idx [L][Hkv][sum kept], out [L][Hkv][sum kept][d].
 * ------------------------------------------------------------------------ */
int orc_compact(const void* k_in, const void* v_in, const int32_t* idx, int elem_bytes, int B,
                const int64_t* seqlens, const int64_t* kept, int L, int Hkv, int d, void* k_out,
                void* v_out) {
  const int64_t T = total_len(B, seqlens);
  int64_t K = 0;
  for (int b = 0; b < B; ++b) K += kept[b];
  const size_t row = (size_t)d * (size_t)elem_bytes;
  for (int l = 0; l < L; ++l)
    for (int g = 0; g < Hkv; ++g) {
      int64_t koff = 0;
      for (int b = 0; b < B; ++b) {
        const int64_t cu = seq_start(b, seqlens);
        for (int64_t j = 0; j < kept[b]; ++j) {
          const int64_t src = (int64_t)(l * Hkv + g) * T + cu + idx[(int64_t)(l * Hkv + g) * K + koff + j];
          const int64_t dst = (int64_t)(l * Hkv + g) * K + koff + j;
          memcpy((char*)k_out + dst * row, (const char*)k_in + src * row, row);
          memcpy((char*)v_out + dst * row, (const char*)v_in + src * row, row);
        }
        koff += kept[b];
      }
    }
  return ORC_OK;
}

/* Compaction of a layer-wide selection: the rows of idx (orc_select_layer's
 * layout) in order, each from the head that head_kept assigns it to.
 * k_out/v_out [sum of layer_kept][d]. */
int orc_compact_layer(const void* k_in, const void* v_in, const int32_t* idx,
                      const int32_t* head_kept, int elem_bytes, int B, const int64_t* seqlens,
                      int L, int Hkv, int d, void* k_out, void* v_out) {
  const int64_t T = total_len(B, seqlens);
  const size_t row = (size_t)d * (size_t)elem_bytes;
  int64_t o = 0;
  for (int l = 0; l < L; ++l)
    for (int b = 0; b < B; ++b) {
      const int64_t cu = seq_start(b, seqlens);
      for (int g = 0; g < Hkv; ++g) {
        const int32_t n = head_kept[((int64_t)l * B + b) * Hkv + g];
        for (int32_t j = 0; j < n; ++j, ++o) {
          const int64_t src = (int64_t)(l * Hkv + g) * T + cu + idx[o];
          memcpy((char*)k_out + o * row, (const char*)k_in + src * row, row);
          memcpy((char*)v_out + o * row, (const char*)v_in + src * row, row);
        }
      }
    }
  return ORC_OK;
}

/* --------------------------------------------------------------------------
 * H2O streaming step (H2O breakdown page, "greedy eviction" with its Algorithm
 * 1 description, the heavy + recent dual-buffer section, and the FlexGen
 * section: fixed slots, the evicted slot is overwritten by the new token).
 * Reading R10.  Per (sequence b, KV head g), independently (per-head section):
 *   p_h = softmax over cached tokens (and the new one when include_self) of
 *         scale * q_h . k_slot, for each query head h of the group;
 *   acc_slot += sum_h p_h(slot);
 *   the new token t enters with acc = include_self ? sum_h p_h(new) : 0;
 *   an empty slot (pos < 0; lowest index first) takes it with no eviction;
 *   otherwise the candidate with the smallest acc among positions in
 *   [n_sink, t - n_recent] (the new token included when it qualifies) is
 *   evicted, ties to the oldest position; its slot takes the new token.
 * q [B][Hq][d], knew/vnew [B][Hkv][d], kc/vc [B][Hkv][C][d], acc/pos
 * [B][Hkv][C], t [B]; evicted [B][Hkv] (position or -1); probs (nullable)
 * [B][Hq][C+1] (last entry: the new token's own probability, 0 unless
 * include_self); margin (nullable) [B][Hkv]: relative gap between the two
 * smallest candidate accumulated scores (+inf with fewer than two).
 * out (nullable) [B][Hq][d]: the step's attention output, reading R11 --
 *   the KV-cache page's decode attention (section 1.1) restricted to the
 *   retained tokens as in the H2O page's problem statement (evicted tokens
 *   leave the normaliser): out_h = sum over occupied slots of p_h(slot) *
 *   v_slot, plus p_h(new) * v_new when include_self, with the same p_h that
 *   are added to the accumulated scores, on the cache as it was before the
 *   new token is inserted.
 * ------------------------------------------------------------------------ */
int orc_h2o_step(const float* q, const float* knew, const float* vnew, float* kc, float* vc,
                 float* acc, int32_t* pos, const int64_t* t, int B, int Hq, int Hkv, int d, int C,
                 int n_sink, int n_recent, double scale, int include_self, int32_t* evicted,
                 float* probs, float* margin, float* out) {
  if (Hq % Hkv || C < 1 || n_sink < 0 || n_recent < 0 || C < n_sink + n_recent) return ORC_EINVAL;
  const int G = Hq / Hkv;
  const int units = B * Hkv;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int u = 0; u < units; ++u) {
    const int b = u / Hkv, g = u % Hkv;
    const int64_t tt = t[b];
    float* K = kc + (int64_t)u * C * d;
    float* V = vc + (int64_t)u * C * d;
    float* A = acc + (int64_t)u * C;
    int32_t* P = pos + (int64_t)u * C;
    const float* kn = knew + (int64_t)u * d;
    const float* vn = vnew + (int64_t)u * d;
    double* add = (double*)calloc((size_t)C, sizeof(double));
    double* x = (double*)malloc((size_t)(C + 1) * sizeof(double));
    double self_add = 0.0;
    for (int hl = 0; hl < G; ++hl) {
      const int h = g * G + hl;
      const float* qh = q + ((int64_t)b * Hq + h) * d;
      double m = -INFINITY;
      for (int j = 0; j < C; ++j) {
        if (P[j] < 0) continue;
        double dot = 0.0;
        for (int e = 0; e < d; ++e) dot += (double)qh[e] * (double)K[(int64_t)j * d + e];
        x[j] = scale * dot;
        if (x[j] > m) m = x[j];
      }
      if (include_self) {
        double dot = 0.0;
        for (int e = 0; e < d; ++e) dot += (double)qh[e] * (double)kn[e];
        x[C] = scale * dot;
        if (x[C] > m) m = x[C];
      }
      double lsum = 0.0;
      for (int j = 0; j < C; ++j)
        if (P[j] >= 0) lsum += exp(x[j] - m);
      if (include_self) lsum += exp(x[C] - m);
      float* pr = probs ? probs + ((int64_t)b * Hq + h) * (C + 1) : NULL;
      for (int j = 0; j < C; ++j) {
        const double p = (P[j] >= 0) ? exp(x[j] - m) / lsum : 0.0;
        add[j] += p;
        if (pr) pr[j] = (float)p;
      }
      const double ps = include_self ? exp(x[C] - m) / lsum : 0.0;
      self_add += ps;
      if (pr) pr[C] = (float)ps;
      if (out) {
        float* oh = out + ((int64_t)b * Hq + h) * d;
        for (int e = 0; e < d; ++e) {
          double o = 0.0;
          for (int j = 0; j < C; ++j)
            if (P[j] >= 0) o += exp(x[j] - m) / lsum * (double)V[(int64_t)j * d + e];
          if (include_self) o += ps * (double)vn[e];
          oh[e] = (float)o;
        }
      }
    }
    for (int j = 0; j < C; ++j)
      if (P[j] >= 0) A[j] = (float)((double)A[j] + add[j]);
    const float acc_new = (float)self_add;
    /* insertion */
    int empty = -1;
    for (int j = 0; j < C; ++j)
      if (P[j] < 0) {
        empty = j;
        break;
      }
    int32_t ev = -1;
    float best = 0.f, second = 0.f;
    int nbest = 0;
    if (empty >= 0) {
      memcpy(K + (int64_t)empty * d, kn, (size_t)d * sizeof(float));
      memcpy(V + (int64_t)empty * d, vn, (size_t)d * sizeof(float));
      A[empty] = acc_new;
      P[empty] = (int32_t)tt;
    } else {
      /* candidates: cached tokens and the new token itself, outside both windows */
      int bj = -2; /* -1 = the new token */
      int64_t bpos = 0;
      for (int j = -1; j < C; ++j) {
        const int64_t pj = (j < 0) ? tt : P[j];
        const float aj = (j < 0) ? acc_new : A[j];
        if (pj < n_sink || pj > tt - n_recent) continue;
        if (nbest == 0 || aj < best || (aj == best && pj < bpos)) {
          if (nbest > 0) second = best;
          best = aj;
          bj = j;
          bpos = pj;
        } else if (nbest == 1 || aj < second) {
          second = aj;
        }
        ++nbest;
      }
      if (bj == -2) {
        bad |= 1;
      } else if (bj == -1) {
        ev = (int32_t)tt; /* the new token itself is dropped */
      } else {
        ev = P[bj];
        memcpy(K + (int64_t)bj * d, kn, (size_t)d * sizeof(float));
        memcpy(V + (int64_t)bj * d, vn, (size_t)d * sizeof(float));
        A[bj] = acc_new;
        P[bj] = (int32_t)tt;
      }
    }
    if (evicted) evicted[u] = ev;
    if (margin) {
      if (nbest >= 2) {
        const double den = fabs((double)second) > 1e-30 ? fabs((double)second) : 1e-30;
        margin[u] = (float)(((double)second - (double)best) / den);
      } else {
        margin[u] = INFINITY;
      }
    }
    free(add);
    free(x);
  }
  return bad ? ORC_EINVAL : ORC_OK;
}
