/*
 * dspark_oracle.c -- plain, slow, fp64 CPU oracle for the DSpark per-round
 * draft-and-verify hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The HIP library shares
 * no code, header, table or constant generator with this file.
 *
 * Pages cited (titles as published):
 *   [P1] "DSpark: Confidence-Scheduled Speculative Decoding with
 *        Semi-Autoregressive Generation 요약 설명" (summary page)
 *   [P2] "DSpark: Confidence-Scheduled Speculative Decoding with
 *        Semi-Autoregressive Generation" (notes page, section "DSpark 핵심 기술")
 *
 * Everything here is the plain definition written out in double precision,
 * one loop per definition, no blocking or fusion.  Readings where the pages are
 * silent are marked READING and are listed with their reasons in the design
 * notes of the repository.
 *
 * Random numbers (READING, pages silent): Philox4x32-10 as defined by Salmon,
 * Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11),
 * keyed by the 64-bit seed, with counter (v>>2, k, r, stream) and word v&3.
 * Streams: 0/4 draft Gumbel (block/member), 1 accept uniform, 2/6 residual
 * Gumbel (block/member), 3/7 bonus Gumbel (block/member).
 *
 * Categorical draws (READING, the pages only say that tokens are sampled from
 * the distributions): two-level Gumbel-max.  The vocabulary is cut into
 * consecutive blocks of 32 entries (the last may be shorter); a block is
 * chosen by Gumbel-max over the blocks' log-masses, then a member of that
 * block by Gumbel-max over its log-weights.  The law of the draw is exactly
 * P(block) P(v | block) = softmax(w)_v.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

/* Thread count of the row loops below (OpenMP; timing of the CPU baseline). */
ORACLE_API void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
ORACLE_API int oracle_max_threads(void) { return omp_get_max_threads(); }

/* Entries per sampling block of the two-level Gumbel-max draw (READING). */
#define ORACLE_SAMPLE_BLOCK 32

/* ------------------------------------------------------------------------ */
/* Counter-based random numbers (Philox4x32-10, SC'11).                      */
/* ------------------------------------------------------------------------ */

/* One Philox4x32 round: two 32x32->64 multiplies (S-box), a fixed
 * permutation and an xor with the round key. */
static void philox_round(uint32_t x[4], const uint32_t key[2]) {
  const uint64_t prod0 = (uint64_t)0xD2511F53u * (uint64_t)x[0];
  const uint64_t prod1 = (uint64_t)0xCD9E8D57u * (uint64_t)x[2];
  uint32_t y[4];
  y[0] = (uint32_t)(prod1 >> 32) ^ x[1] ^ key[0];
  y[1] = (uint32_t)prod1;
  y[2] = (uint32_t)(prod0 >> 32) ^ x[3] ^ key[1];
  y[3] = (uint32_t)prod0;
  memcpy(x, y, sizeof y);
}

/* Ten rounds; the key is bumped by the Weyl constants between rounds. */
ORACLE_API void oracle_philox4x32_10(uint32_t key0, uint32_t key1,
                                     const uint32_t counter[4], uint32_t out[4]) {
  uint32_t x[4] = {counter[0], counter[1], counter[2], counter[3]};
  uint32_t key[2] = {key0, key1};
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      key[0] += 0x9E3779B9u;
      key[1] += 0xBB67AE85u;
    }
    philox_round(x, key);
  }
  memcpy(out, x, sizeof x);
}

/* The 32-bit word that element (stream, r, k, v) draws.  READING: counter
 * (v>>2, k, r, stream), key = seed, word index v&3. */
ORACLE_API uint32_t oracle_word(uint64_t seed, uint32_t stream, uint32_t r,
                                uint32_t k, uint32_t v) {
  const uint32_t ctr[4] = {v >> 2, k, r, stream};
  uint32_t out[4];
  oracle_philox4x32_10((uint32_t)seed, (uint32_t)(seed >> 32), ctr, out);
  return out[v & 3u];
}

/* Words for elements v0 .. v0+n-1 of one (stream, r, k) row. */
ORACLE_API void oracle_words(uint64_t seed, uint32_t stream, uint32_t r, uint32_t k,
                             uint32_t v0, int64_t n, uint32_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_word(seed, stream, r, k, v0 + (uint32_t)i);
}

/* Uniform in (0,1): the top 23 bits plus one half, times 2^-23.  Every value
 * lies in [2^-24, 1-2^-24] and is exactly representable in binary32. */
ORACLE_API double oracle_uniform(uint32_t word) {
  return ((double)(word >> 9) + 0.5) * 0x1p-23;
}

/* Standard Gumbel variate by inversion of its CDF exp(-exp(-g)). */
ORACLE_API double oracle_gumbel(uint32_t word) {
  return -log(-log(oracle_uniform(word)));
}

/* ------------------------------------------------------------------------ */
/* Row primitives.                                                           */
/* ------------------------------------------------------------------------ */

/* log sum_v exp(z_v), with the maximum taken out first. */
ORACLE_API double oracle_logsumexp(int64_t n, const double* z) {
  double m = -INFINITY;
  for (int64_t v = 0; v < n; ++v)
    if (z[v] > m) m = z[v];
  if (m == -INFINITY) return -INFINITY;
  double s = 0.0;
  for (int64_t v = 0; v < n; ++v) s += exp(z[v] - m);
  return m + log(s);
}

/* argmax_v (w_v + g_v) with the lowest index winning exact ties; returns the
 * index and writes the gap between the best and the runner-up score (the
 * "margin" used to flag near-ties). */
ORACLE_API int64_t oracle_gumbel_argmax(int64_t n, const double* w, const double* g,
                                        double* margin) {
  int64_t best = -1;
  double s1 = -INFINITY, s2 = -INFINITY;
  for (int64_t v = 0; v < n; ++v) {
    const double s = w[v] + g[v];
    if (s > s1 || best < 0) {
      s2 = s1;
      s1 = s;
      best = v;
    } else if (s > s2) {
      s2 = s;
    }
  }
  if (margin) *margin = s1 - s2;
  return best;
}

/* Two-level Gumbel-max draw from softmax(w) over n entries (w may hold -inf,
 * at least one entry finite).  Level 1: block b (entries [b*block,
 * min((b+1)*block, n))) scores logsumexp(w over the block) plus the Gumbel
 * variate of element b of stream `stream_block`; the best block wins (lowest
 * b on exact ties).  Level 2: inside the winning block, entry v scores
 * w_v plus the Gumbel variate of element v of stream `stream_member`.
 * margin = the smaller of the two levels' top-2 gaps. */
ORACLE_API int64_t oracle_two_level_draw(int64_t n, const double* w, int64_t block,
                                         uint64_t seed, uint32_t stream_block,
                                         uint32_t stream_member, uint32_t r, uint32_t k,
                                         double* margin) {
  const int64_t nb = (n + block - 1) / block;
  double* lb = (double*)malloc((size_t)nb * sizeof(double));
  double* gb = (double*)malloc((size_t)nb * sizeof(double));
  for (int64_t b = 0; b < nb; ++b) {
    const int64_t v0 = b * block;
    const int64_t len = (v0 + block <= n) ? block : n - v0;
    lb[b] = oracle_logsumexp(len, w + v0);
    gb[b] = oracle_gumbel(oracle_word(seed, stream_block, r, k, (uint32_t)b));
  }
  double m1, m2;
  const int64_t bstar = oracle_gumbel_argmax(nb, lb, gb, &m1);
  const int64_t v0 = bstar * block;
  const int64_t len = (v0 + block <= n) ? block : n - v0;
  double g[64];
  double* gm = len <= 64 ? g : (double*)malloc((size_t)len * sizeof(double));
  for (int64_t i = 0; i < len; ++i)
    gm[i] = oracle_gumbel(oracle_word(seed, stream_member, r, k, (uint32_t)(v0 + i)));
  const int64_t x = v0 + oracle_gumbel_argmax(len, w + v0, gm, &m2);
  if (gm != g) free(gm);
  free(lb);
  free(gb);
  if (margin) *margin = m1 < m2 ? m1 : m2;
  return x;
}

/* Standard speculative acceptance: accept draft token x with probability
 * min(1, p^t(x)/p^d(x)); with u uniform, accept iff u < p^t(x)/p^d(x), taken
 * in log space as ln u < ln p^t(x) - ln p^d(x).  [P1 요약; P2 배경, step 3]
 * READING: strict inequality. */
ORACLE_API int oracle_accept(double ln_u, double lpt_x, double lpd_x) {
  return ln_u < (lpt_x - lpd_x);
}

/* Log-weights of the residual distribution max(0, p^t - p^d) (unnormalised;
 * -inf where p^t <= p^d).  ln(p^t - p^d) is evaluated as
 * ln p^t + ln(1 - exp(ln p^d - ln p^t)) to avoid cancellation.
 * Returns the number of entries with positive residual. */
ORACLE_API int64_t oracle_residual_logw(int64_t n, const double* lpd, const double* lpt,
                                        double* logw) {
  int64_t positive = 0;
  for (int64_t v = 0; v < n; ++v) {
    if (lpt[v] > lpd[v]) {
      logw[v] = lpt[v] + log1p(-exp(lpd[v] - lpt[v]));
      if (logw[v] > -INFINITY) ++positive;
    } else {
      logw[v] = -INFINITY;
    }
  }
  return positive;
}

/* Analytic stepwise acceptance c* = 1 - 0.5*||p^d - p^t||_1, evaluated as the
 * equal quantity sum_v min(p^d_v, p^t_v).  [P1 §3.2.1 Confidence Head] */
ORACLE_API double oracle_cstar(int64_t n, const double* lpd, const double* lpt) {
  double s = 0.0;
  for (int64_t v = 0; v < n; ++v) s += exp(lpd[v] < lpt[v] ? lpd[v] : lpt[v]);
  return s;
}

/* ------------------------------------------------------------------------ */
/* Stage 1: Markov-head draft sampling, one position for a batch of rows.    */
/* [P1 §3.1; P2 "최종 분포"]: p_k = softmax(U_k + B_k), sampled left to right.*/
/* The caller supplies z = U_k + W1[x_{k-1}] W2 in fp64 (the contraction is a */
/* plain matrix product done by the caller with a library matmul).           */
/* ------------------------------------------------------------------------ */
ORACLE_API void oracle_draft_rows(int64_t nrows, int64_t V, const double* z,
                                  uint64_t seed, const int32_t* r_idx, const int32_t* k_idx,
                                  int32_t* token, double* lse, double* logq, double* margin) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < nrows; ++i) {
    const double* zi = z + i * V;
    const double l = oracle_logsumexp(V, zi);
    double mg;
    const int64_t x = oracle_two_level_draw(V, zi, ORACLE_SAMPLE_BLOCK, seed, 0u, 4u,
                                            (uint32_t)r_idx[i], (uint32_t)k_idx[i], &mg);
    token[i] = (int32_t)x;
    lse[i] = l;
    logq[i] = zi[x] - l;
    if (margin) margin[i] = mg;
  }
}

/* ------------------------------------------------------------------------ */
/* Stage 2: verification of a batch of requests.                             */
/* zd: [nreq, gamma, V] draft logits, zt: [nreq, gamma+1, V] target logits,  */
/* both fp64.  tokens: [nreq, gamma] drafted tokens; lengths: [nreq] verify  */
/* lengths in [0, gamma].  r_idx: request ids used for the random streams.   */
/* Outputs: cstar [nreq, gamma] (NaN for k > length), n_accept [nreq],       */
/* out_token [nreq], accept_mask [nreq, gamma] (1 accepted, 0 rejected,      */
/* 255 not verified), acc_margin [nreq, gamma] |ln u - ln ratio|,            */
/* out_margin [nreq] top-2 gap of the final draw, lse_t [nreq, gamma+1]      */
/* (NaN where not computed).                                                 */
/* [P1 요약 / P2 배경]: rejection sampling keeps the longest accepted prefix, */
/* resamples from the normalised max(0, p^t - p^d) at the first rejection    */
/* and draws a bonus token from p^t when all verified tokens are accepted.    */
/* ------------------------------------------------------------------------ */
ORACLE_API void oracle_verify_requests(int64_t nreq, int64_t gamma, int64_t V,
                                       const double* zd, const double* zt,
                                       const int32_t* tokens, const int32_t* lengths,
                                       uint64_t seed, const int32_t* r_idx,
                                       float* cstar, int32_t* n_accept, int32_t* out_token,
                                       uint8_t* accept_mask, double* acc_margin,
                                       double* out_margin, double* lse_t_out,
                                       double* lse_d_out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t q = 0; q < nreq; ++q) {
    const uint32_t r = (uint32_t)r_idx[q];
    const int64_t len = lengths[q];
    double* lpd = (double*)malloc((size_t)V * sizeof(double));
    double* lpt = (double*)malloc((size_t)V * sizeof(double));
    double* w = (double*)malloc((size_t)V * sizeof(double));
    for (int64_t k = 0; k < gamma; ++k) {
      cstar[q * gamma + k] = NAN;
      accept_mask[q * gamma + k] = 255;
      acc_margin[q * gamma + k] = NAN;
      if (lse_d_out) lse_d_out[q * gamma + k] = NAN;
    }
    for (int64_t k = 0; k <= gamma; ++k)
      if (lse_t_out) lse_t_out[q * (gamma + 1) + k] = NAN;

    int64_t n = len;  /* accepted count; stays len if nothing is rejected */
    int64_t kstar = -1;
    for (int64_t k = 1; k <= len; ++k) {
      const double* zdk = zd + (q * gamma + (k - 1)) * V;
      const double* ztk = zt + (q * (gamma + 1) + (k - 1)) * V;
      const double ld = oracle_logsumexp(V, zdk);
      const double lt = oracle_logsumexp(V, ztk);
      for (int64_t v = 0; v < V; ++v) {
        lpd[v] = zdk[v] - ld;
        lpt[v] = ztk[v] - lt;
      }
      if (lse_t_out) lse_t_out[q * (gamma + 1) + (k - 1)] = lt;
      if (lse_d_out) lse_d_out[q * gamma + (k - 1)] = ld;
      cstar[q * gamma + (k - 1)] = (float)oracle_cstar(V, lpd, lpt);
      const int32_t x = tokens[q * gamma + (k - 1)];
      const double ln_u = log(oracle_uniform(oracle_word(seed, 1u, r, (uint32_t)k, 0u)));
      acc_margin[q * gamma + (k - 1)] = fabs(ln_u - (lpt[x] - lpd[x]));
      if (kstar < 0) {
        const int ok = oracle_accept(ln_u, lpt[x], lpd[x]);
        accept_mask[q * gamma + (k - 1)] = (uint8_t)ok;
        if (!ok) {
          kstar = k;
          n = k - 1;
        }
      }
    }

    double mg = NAN;
    int64_t y;
    if (kstar > 0) {
      /* recompute the rejected row's log-probabilities */
      const double* zdk = zd + (q * gamma + (kstar - 1)) * V;
      const double* ztk = zt + (q * (gamma + 1) + (kstar - 1)) * V;
      const double ld = oracle_logsumexp(V, zdk);
      const double lt = oracle_logsumexp(V, ztk);
      for (int64_t v = 0; v < V; ++v) {
        lpd[v] = zdk[v] - ld;
        lpt[v] = ztk[v] - lt;
      }
      const int64_t positive = oracle_residual_logw(V, lpd, lpt, w);
      if (positive == 0)  /* READING: empty residual after rounding -> p^t */
        for (int64_t v = 0; v < V; ++v) w[v] = lpt[v];
      y = oracle_two_level_draw(V, w, ORACLE_SAMPLE_BLOCK, seed, 2u, 6u, r, (uint32_t)kstar, &mg);
    } else {
      /* bonus token from p^t at position len+1 (row index len) */
      const int64_t b = len + 1;
      const double* ztb = zt + (q * (gamma + 1) + (b - 1)) * V;
      y = oracle_two_level_draw(V, ztb, ORACLE_SAMPLE_BLOCK, seed, 3u, 7u, r, (uint32_t)b, &mg);
    }
    n_accept[q] = (int32_t)n;
    out_token[q] = (int32_t)y;
    if (out_margin) out_margin[q] = mg;
    free(lpd);
    free(lpt);
    free(w);
  }
}

/* ------------------------------------------------------------------------ */
/* Confidence head with Sequential Temperature Scaling.                     */
/* [P1 §3.2.1]: c_k from the backbone state h_k and the Markov embedding of   */
/* x_{k-1}; STS rescales each position's logit by a per-position temperature.*/
/* READING: c = sigmoid((w . [h; W1[x_{k-1}]]) / T_k), no bias term.          */
/* h: [nrows, H] fp64, e: [nrows, rank] fp64 (W1 rows), w: [H + rank].       */
/* ------------------------------------------------------------------------ */
ORACLE_API void oracle_confidence_rows(int64_t nrows, int64_t H, int64_t rank,
                                       const double* h, const double* e, const double* w,
                                       const double* temp, float* c) {
  for (int64_t i = 0; i < nrows; ++i) {
    double s = 0.0;
    for (int64_t j = 0; j < H; ++j) s += w[j] * h[i * H + j];
    for (int64_t j = 0; j < rank; ++j) s += w[H + j] * e[i * rank + j];
    c[i] = (float)(1.0 / (1.0 + exp(-s / temp[i])));
  }
}

/* ------------------------------------------------------------------------ */
/* Stage 3: prefix-survival products a_{r,j} = prod_{i<=j} c_{r,i}.          */
/* [P1 §3.2.2].  READING: sequential binary32 multiplies, a_{r,1} = c_{r,1}. */
/* ------------------------------------------------------------------------ */
ORACLE_API void oracle_prefix_products(int64_t R, int64_t gamma, const float* c, float* a) {
  for (int64_t r = 0; r < R; ++r) {
    float acc = 1.0f;
    for (int64_t j = 0; j < gamma; ++j) {
      volatile float prod = acc * c[r * gamma + j];  /* one binary32 rounding */
      acc = prod;
      a[r * gamma + j] = acc;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Stage 4: hardware-aware prefix scheduler (Algorithm 1).                   */
/* [P1 §3.2.2]: B = sum_r (1 + l_r), tau = sum_r (1 + sum_{j<=l_r} a_{r,j}),  */
/* Theta = tau * SPS(B); candidates are taken in order of survival          */
/* probability and the search stops as soon as Theta does not improve.       */
/* READINGS: start at l = 0 (B = R, tau = R); candidate order by the key     */
/* (-a, r, j); continue only on strict improvement; SPS(B) = sps[B-1];       */
/* tau accumulated exactly in units of 2^-38 (each a rounded to the nearest  */
/* multiple, ties to even), Theta = double(tau) * SPS(B).                    */
/* ------------------------------------------------------------------------ */
typedef struct {
  float a;
  int32_t r, j;
} cand_t;

static int cand_cmp(const void* pa, const void* pb) {
  const cand_t* x = (const cand_t*)pa;
  const cand_t* y = (const cand_t*)pb;
  if (x->a != y->a) return x->a > y->a ? -1 : 1;
  if (x->r != y->r) return x->r < y->r ? -1 : 1;
  return (x->j > y->j) - (x->j < y->j);
}

/* a (fp32 in [0,1]) in units of 2^-38, rounded to nearest even. */
ORACLE_API int64_t oracle_tau_units(float a) {
  return (int64_t)nearbyint(ldexp((double)a, 38));
}

ORACLE_API int64_t oracle_schedule(int64_t R, int64_t gamma, const float* a,
                                   const float* sps, int64_t n_sps,
                                   int32_t* lengths, double* stats, double* theta_path,
                                   double* stop_gap) {
  const int64_t n = R * gamma;
  if (n_sps < R * (gamma + 1)) return -1;
  cand_t* cand = (cand_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(cand_t));
  for (int64_t r = 0; r < R; ++r)
    for (int64_t j = 1; j <= gamma; ++j) {
      cand[r * gamma + (j - 1)].a = a[r * gamma + (j - 1)];
      cand[r * gamma + (j - 1)].r = (int32_t)r;
      cand[r * gamma + (j - 1)].j = (int32_t)j;
    }
  qsort(cand, (size_t)n, sizeof(cand_t), cand_cmp);

  for (int64_t r = 0; r < R; ++r) lengths[r] = 0;
  int64_t B = R;
  int64_t tau_units = R * ((int64_t)1 << 38);
  double theta = ldexp((double)tau_units, -38) * (double)sps[B - 1];
  if (theta_path) theta_path[0] = theta;
  int64_t sel = 0;
  double gap = NAN;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t B2 = B + 1;
    const int64_t tau2 = tau_units + oracle_tau_units(cand[i].a);
    const double theta2 = ldexp((double)tau2, -38) * (double)sps[B2 - 1];
    if (theta_path) theta_path[i + 1] = theta2;
    if (!(theta2 > theta)) {  /* first non-improvement: stop (causal) */
      gap = (theta - theta2) / theta;
      break;
    }
    B = B2;
    tau_units = tau2;
    theta = theta2;
    lengths[cand[i].r] = cand[i].j;  /* order respects prefixes */
    ++sel;
  }
  if (theta_path)
    for (int64_t i = sel + 2; i <= n; ++i) theta_path[i] = NAN;
  stats[0] = (double)B;
  stats[1] = ldexp((double)tau_units, -38);
  stats[2] = theta;
  stats[3] = (double)sel;
  if (stop_gap) *stop_gap = gap;
  free(cand);
  return sel;
}

/* ------------------------------------------------------------------------ */
/* Production variant of the prefix scheduler.  [P1 §5.2]                    */
/* The deployed scheduler fits Algorithm 1 to an irregular, discontinuous    */
/* SPS(B) curve and to zero-overhead scheduling: the capacity K of a round   */
/* is chosen from confidences of two rounds earlier, and the round's own      */
/* candidates are ranked by their current survival probability, of which the */
/* first K are verified.  When the capacity is predicted from past rounds     */
/* the early-stopping break is left out, so that a throughput cliff does not  */
/* trap the search in a local optimum.                                        */
/* READINGS: the capacity is the number of candidates, taken in the order of  */
/* Algorithm 1, at which Theta is largest along the whole path (l = 0 up to   */
/* every candidate); the smallest such count wins ties.  tau and Theta are    */
/* formed exactly as in Algorithm 1.                                          */
/* ------------------------------------------------------------------------ */
static cand_t* sorted_candidates(int64_t R, int64_t gamma, const float* a) {
  const int64_t n = R * gamma;
  cand_t* cand = (cand_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(cand_t));
  for (int64_t r = 0; r < R; ++r)
    for (int64_t j = 1; j <= gamma; ++j) {
      cand[r * gamma + (j - 1)].a = a[r * gamma + (j - 1)];
      cand[r * gamma + (j - 1)].r = (int32_t)r;
      cand[r * gamma + (j - 1)].j = (int32_t)j;
    }
  qsort(cand, (size_t)n, sizeof(cand_t), cand_cmp);
  return cand;
}

/* Capacity: returns K (or -1 if the SPS table is too short); stats = (B, tau,
 * Theta, K) at K; theta_path[i] = Theta after the first i candidates, i = 0..n
 * (every entry: there is no stop). */
ORACLE_API int64_t oracle_schedule_capacity(int64_t R, int64_t gamma, const float* a,
                                            const float* sps, int64_t n_sps, double* stats,
                                            double* theta_path) {
  const int64_t n = R * gamma;
  if (n_sps < R * (gamma + 1)) return -1;
  cand_t* cand = sorted_candidates(R, gamma, a);
  int64_t tau_units = R * ((int64_t)1 << 38);
  double best = ldexp((double)tau_units, -38) * (double)sps[R - 1];
  int64_t best_i = 0, best_tau = tau_units;
  if (theta_path) theta_path[0] = best;
  for (int64_t i = 0; i < n; ++i) {
    tau_units += oracle_tau_units(cand[i].a);
    const double theta = ldexp((double)tau_units, -38) * (double)sps[R + i];  /* SPS(R+i+1) */
    if (theta_path) theta_path[i + 1] = theta;
    if (theta > best) {  /* strict: the smallest count wins ties */
      best = theta;
      best_i = i + 1;
      best_tau = tau_units;
    }
  }
  stats[0] = (double)(R + best_i);
  stats[1] = ldexp((double)best_tau, -38);
  stats[2] = best;
  stats[3] = (double)best_i;
  free(cand);
  return best_i;
}

/* Top-K: verify the first min(K, n) candidates in survival order (K >= 0);
 * lengths [R]; stats = (B, tau, Theta, taken) with Theta = tau * SPS(B). */
ORACLE_API int64_t oracle_schedule_topk(int64_t R, int64_t gamma, const float* a,
                                        const float* sps, int64_t n_sps, int64_t K,
                                        int32_t* lengths, double* stats) {
  const int64_t n = R * gamma;
  if (n_sps < R * (gamma + 1) || K < 0) return -1;
  cand_t* cand = sorted_candidates(R, gamma, a);
  const int64_t take = K < n ? K : n;
  for (int64_t r = 0; r < R; ++r) lengths[r] = 0;
  int64_t tau_units = R * ((int64_t)1 << 38);
  for (int64_t i = 0; i < take; ++i) {
    tau_units += oracle_tau_units(cand[i].a);
    lengths[cand[i].r] = cand[i].j;  /* order respects prefixes */
  }
  stats[0] = (double)(R + take);
  stats[1] = ldexp((double)tau_units, -38);
  stats[2] = stats[1] * (double)sps[R + take - 1];
  stats[3] = (double)take;
  free(cand);
  return take;
}

/* ------------------------------------------------------------------------ */
/* Static-threshold verification and per-position conditional acceptance.   */
/* [P1 §4.3.3, §4.3.1]                                                       */
/* The threshold experiment verifies, per request, the prefix whose          */
/* estimated survival stays at or above a fixed threshold; READING: l_r is   */
/* the largest j with a_{r,i} >= theta for every i <= j (the prefix form,    */
/* equal to max{j : a_{r,j} >= theta} when a is non-increasing).             */
/* ------------------------------------------------------------------------ */
ORACLE_API void oracle_threshold_lengths(int64_t R, int64_t gamma, const float* a,
                                         double theta, int32_t* lengths) {
  for (int64_t r = 0; r < R; ++r) {
    int32_t l = 0;
    while (l < gamma && (double)a[r * gamma + l] >= theta) ++l;
    lengths[r] = l;
  }
}

/* Conditional acceptance at position k counts only rollouts whose earlier
 * draft tokens were all accepted [P1 §4.3.1].  mask [R, gamma]: 1 accepted,
 * 0 rejected, 255 not verified.  reached[k-1] = requests whose positions
 * 1..k-1 are accepted and whose position k was verified; accepted[k-1] = those
 * of them that accepted position k. */
ORACLE_API void oracle_conditional_acceptance(int64_t R, int64_t gamma, const uint8_t* mask,
                                              int64_t* reached, int64_t* accepted) {
  for (int64_t k = 0; k < gamma; ++k) reached[k] = accepted[k] = 0;
  for (int64_t r = 0; r < R; ++r) {
    for (int64_t k = 0; k < gamma; ++k) {
      int prefix_ok = 1;
      for (int64_t i = 0; i < k; ++i)
        if (mask[r * gamma + i] != 1) prefix_ok = 0;
      if (!prefix_ok || mask[r * gamma + k] == 255) continue;
      reached[k] += 1;
      if (mask[r * gamma + k] == 1) accepted[k] += 1;
    }
  }
}

/* Threshold sweep over one fully verified round: for each threshold, the
 * tokens a threshold-limited verify would check, sum_r l_r(theta), and the
 * draft tokens it would accept, sum_r min(n_r, l_r(theta)), where n_r is the
 * accepted length of the full verify (acceptance at a position does not depend
 * on how far the verify reaches). */
ORACLE_API void oracle_threshold_sweep(int64_t R, int64_t gamma, const float* a,
                                       const int32_t* n_accept, int64_t n_thr,
                                       const double* thresholds, int64_t* verified,
                                       int64_t* accepted) {
  int32_t* l = (int32_t*)malloc((size_t)(R > 0 ? R : 1) * sizeof(int32_t));
  for (int64_t g = 0; g < n_thr; ++g) {
    oracle_threshold_lengths(R, gamma, a, thresholds[g], l);
    verified[g] = accepted[g] = 0;
    for (int64_t r = 0; r < R; ++r) {
      verified[g] += l[r];
      accepted[g] += n_accept[r] < l[r] ? n_accept[r] : l[r];
    }
  }
  free(l);
}

/* ------------------------------------------------------------------------ */
/* Sequential Temperature Scaling fit.  [P1 §3.2.1]                          */
/* STS calibrates the cumulative prefix survival on held-out rollouts: a     */
/* one-dimensional grid search runs left to right, each position's           */
/* temperature chosen to minimise that position's Expected Calibration Error */
/* with the earlier positions' temperatures held fixed.                      */
/* READINGS: rollout n has confidence-head scores s[n, j] (the logit before  */
/* the sigmoid) and survival labels y[n, j] = 1 iff its draft positions      */
/* 1..j were all accepted; c = sigmoid(s / T) evaluated in binary64 and      */
/* rounded to binary32; a_j = fl32(a_{j-1} * c_j), a_0 = 1 (the scheduler's   */
/* prefix products); ECE over M equal-width bins of [0, 1], bin =            */
/* min(floor(a M), M - 1): ECE = (1/N) sum_b |sum_{n in b} (y_n - a_n)|,     */
/* with every a rounded to the nearest multiple of 2^-40 so that the sums    */
/* are exact integers; the smallest ECE wins, the lowest grid index on ties. */
/* Outputs: temps[j] = chosen grid value, ece_units[j] = N * ECE at it in    */
/* units of 2^-40, ece1_units[j] = the same at T = 1 with the earlier         */
/* positions calibrated, a [N, gamma] the calibrated survival.               */
/* ------------------------------------------------------------------------ */
static float sts_conf(double s, double T) { return (float)(1.0 / (1.0 + exp(-s / T))); }

static int64_t sts_units(float a) { return (int64_t)nearbyint(ldexp((double)a, 40)); }

/* N * ECE in units of 2^-40 of survival values a [N] against labels y [N]. */
ORACLE_API int64_t oracle_ece_units(int64_t N, const float* a, const uint8_t* y, int64_t M) {
  int64_t* acc = (int64_t*)calloc((size_t)M, sizeof(int64_t));
  for (int64_t n = 0; n < N; ++n) {
    int64_t b = (int64_t)floor((double)a[n] * (double)M);
    if (b > M - 1) b = M - 1;
    if (b < 0) b = 0;
    acc[b] += ((int64_t)(y[n] != 0) << 40) - sts_units(a[n]);
  }
  int64_t e = 0;
  for (int64_t b = 0; b < M; ++b) e += acc[b] < 0 ? -acc[b] : acc[b];
  free(acc);
  return e;
}

ORACLE_API void oracle_sts_fit(int64_t N, int64_t gamma, const double* s, const uint8_t* y,
                               int64_t G, const double* grid, int64_t M, float* temps,
                               int64_t* ece_units, int64_t* ece1_units, float* a) {
  float* prev = (float*)malloc((size_t)(N > 0 ? N : 1) * sizeof(float));
  float* cur = (float*)malloc((size_t)(N > 0 ? N : 1) * sizeof(float));
  uint8_t* yj = (uint8_t*)malloc((size_t)(N > 0 ? N : 1));
  for (int64_t n = 0; n < N; ++n) prev[n] = 1.0f;
  for (int64_t j = 0; j < gamma; ++j) {
    for (int64_t n = 0; n < N; ++n) yj[n] = y[n * gamma + j];
    int64_t best = -1, best_e = 0;
    for (int64_t g = 0; g < G; ++g) {
      for (int64_t n = 0; n < N; ++n) {
        volatile float p = prev[n] * sts_conf(s[n * gamma + j], grid[g]);
        cur[n] = p;
      }
      const int64_t e = oracle_ece_units(N, cur, yj, M);
      if (best < 0 || e < best_e) {
        best = g;
        best_e = e;
      }
    }
    for (int64_t n = 0; n < N; ++n) {
      volatile float p = prev[n] * sts_conf(s[n * gamma + j], 1.0);
      cur[n] = p;
    }
    ece1_units[j] = oracle_ece_units(N, cur, yj, M);
    temps[j] = (float)grid[best];
    ece_units[j] = best_e;
    for (int64_t n = 0; n < N; ++n) {
      volatile float p = prev[n] * sts_conf(s[n * gamma + j], grid[best]);
      prev[n] = p;
      a[n * gamma + j] = p;
    }
  }
  free(prev);
  free(cur);
  free(yj);
}
