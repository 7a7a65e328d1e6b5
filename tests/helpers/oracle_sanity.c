/* oracle_sanity.c -- drives every entry point of the CPU oracle on small
 * inputs (ragged sizes, masked entries, empty verify lengths, exact ties), so
 * that a build with AddressSanitizer and UndefinedBehaviorSanitizer checks its
 * memory accesses and arithmetic.  Test infrastructure: built and run by
 * tests/test_oracle_sanitized.py with gcc on the host.  Prints "ok" and exits 0
 * when every call returns and the few checked facts hold. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../oracle/dspark_oracle.c"

static double lcg(uint64_t* s) {
  *s = *s * 6364136223846793005ull + 1442695040888963407ull;
  return ((double)(*s >> 11) * 0x1p-53) * 2.0 - 1.0;
}

#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      return 1;                                               \
    }                                                         \
  } while (0)

int main(void) {
  uint64_t st = 12345;
  /* random numbers */
  uint32_t ctr[4] = {1, 2, 3, 4}, out[4];
  oracle_philox4x32_10(7u, 9u, ctr, out);
  uint32_t words[37];
  oracle_words(99, 0, 3, 2, 5, 37, words);
  for (int i = 0; i < 37; ++i) {
    const double u = oracle_uniform(words[i]);
    CHECK(u > 0.0 && u < 1.0);
    CHECK(isfinite(oracle_gumbel(words[i])));
  }

  /* row primitives, with masked entries and a ragged last block */
  enum { N = 101 };
  double w[N], g[N], lpd[N], lpt[N], res[N], margin;
  for (int i = 0; i < N; ++i) {
    w[i] = (i % 7 == 3) ? -INFINITY : 4.0 * lcg(&st);
    g[i] = lcg(&st);
  }
  CHECK(isfinite(oracle_logsumexp(N, w)));
  const int64_t am = oracle_gumbel_argmax(N, w, g, &margin);
  CHECK(am >= 0 && am < N && w[am] > -INFINITY);
  for (int64_t blk = 1; blk <= 64; blk *= 4) {
    const int64_t x = oracle_two_level_draw(N, w, blk, 5, 0, 4, 1, 2, &margin);
    CHECK(x >= 0 && x < N && w[x] > -INFINITY);
  }
  const double lw = oracle_logsumexp(N, w);
  for (int i = 0; i < N; ++i) {
    lpd[i] = w[i] - lw;
    lpt[i] = (w[i] > -INFINITY ? w[i] + 0.3 * lcg(&st) : -INFINITY);
  }
  const double lt = oracle_logsumexp(N, lpt);
  for (int i = 0; i < N; ++i) lpt[i] -= lt;
  CHECK(oracle_residual_logw(N, lpd, lpt, res) > 0);
  const double cs = oracle_cstar(N, lpd, lpt);
  CHECK(cs > 0.0 && cs <= 1.0 + 1e-12);
  (void)oracle_accept(-0.5, -1.0, -2.0);

  /* draft and verify of a tiny batch: 3 requests, gamma 3, V 70 */
  enum { R = 3, G = 3, V = 70 };
  static double zd[R * G * V], zt[R * (G + 1) * V];
  for (int i = 0; i < R * G * V; ++i) zd[i] = 3.0 * lcg(&st);
  for (int i = 0; i < R * (G + 1) * V; ++i) zt[i] = 3.0 * lcg(&st);
  int32_t r_idx[R * G], k_idx[R * G], tok[R * G], rq[R] = {0, 1, 2}, lengths[R] = {3, 0, 2};
  double lse[R * G], logq[R * G], mg[R * G];
  for (int i = 0; i < R * G; ++i) {
    r_idx[i] = i / G;
    k_idx[i] = i % G + 1;
  }
  oracle_draft_rows(R * G, V, zd, 11, r_idx, k_idx, tok, lse, logq, mg);
  for (int i = 0; i < R * G; ++i) CHECK(tok[i] >= 0 && tok[i] < V);
  float cstar[R * G];
  int32_t n_acc[R], out_tok[R];
  uint8_t mask[R * G];
  double acc_m[R * G], out_m[R], lse_t[R * (G + 1)], lse_d[R * G];
  oracle_verify_requests(R, G, V, zd, zt, tok, lengths, 11, rq, cstar, n_acc, out_tok, mask, acc_m,
                         out_m, lse_t, lse_d);
  for (int r = 0; r < R; ++r) {
    CHECK(n_acc[r] >= 0 && n_acc[r] <= lengths[r]);
    CHECK(out_tok[r] >= 0 && out_tok[r] < V);
  }
  /* the empty residual: target rows equal to the draft rows */
  static double zeq[R * (G + 1) * V];
  for (int r = 0; r < R; ++r)
    for (int i = 0; i < (G + 1) * V; ++i)
      zeq[r * (G + 1) * V + i] = i < G * V ? zd[r * G * V + i] : zt[r * (G + 1) * V + i];
  oracle_verify_requests(R, G, V, zd, zeq, tok, lengths, 11, rq, cstar, n_acc, out_tok, mask, acc_m,
                         out_m, NULL, NULL);

  /* confidence head */
  enum { H = 9, RK = 4 };
  double h[R * H], e[R * RK], wc[H + RK], temp[R];
  for (int i = 0; i < R * H; ++i) h[i] = lcg(&st);
  for (int i = 0; i < R * RK; ++i) e[i] = lcg(&st);
  for (int i = 0; i < H + RK; ++i) wc[i] = lcg(&st);
  for (int i = 0; i < R; ++i) temp[i] = 1.2;
  float c[R];
  oracle_confidence_rows(R, H, RK, h, e, wc, temp, c);

  /* prefix products, Algorithm 1 and the production variants; exact ties */
  enum { SR = 5, SG = 4 };
  float cc[SR * SG], a[SR * SG], sps[SR * (SG + 1)];
  for (int i = 0; i < SR * SG; ++i) cc[i] = (i % 3 == 0) ? 0.5f : 0.75f;
  for (int b = 0; b < SR * (SG + 1); ++b) sps[b] = 1000.0f / (1.0f + 0.05f * (float)(b + 1));
  oracle_prefix_products(SR, SG, cc, a);
  int32_t len[SR];
  double stats[4], path[SR * SG + 1], gap;
  CHECK(oracle_schedule(SR, SG, a, sps, SR * (SG + 1), len, stats, path, &gap) >= 0);
  CHECK(oracle_schedule(SR, SG, a, sps, SR * SG, len, stats, path, &gap) == -1);
  const int64_t K = oracle_schedule_capacity(SR, SG, a, sps, SR * (SG + 1), stats, path);
  CHECK(K >= 0 && K <= SR * SG);
  CHECK(oracle_schedule_topk(SR, SG, a, sps, SR * (SG + 1), K, len, stats) == K);
  CHECK(oracle_schedule_topk(SR, SG, a, sps, SR * (SG + 1), 1000, len, stats) == SR * SG);
  oracle_threshold_lengths(SR, SG, a, 0.4, len);
  uint8_t m2[SR * SG];
  for (int i = 0; i < SR * SG; ++i) m2[i] = (uint8_t)((i % 5 == 4) ? 255 : (i % 3 != 1));
  int64_t reached[SG], accepted[SG];
  oracle_conditional_acceptance(SR, SG, m2, reached, accepted);
  int32_t na[SR] = {0, 4, 2, 1, 3};
  double thr[3] = {0.0, 0.3, 1.1};
  int64_t ver[3], acc3[3];
  oracle_threshold_sweep(SR, SG, a, na, 3, thr, ver, acc3);
  CHECK(ver[0] == SR * SG && ver[2] == 0);

  /* STS fit */
  enum { SN = 40, SGM = 3, GRID = 6, BINS = 5 };
  double s[SN * SGM], grid[GRID];
  uint8_t y[SN * SGM];
  for (int i = 0; i < SN * SGM; ++i) {
    s[i] = 2.0 * lcg(&st);
    y[i] = (uint8_t)(lcg(&st) > 0.0);
  }
  for (int i = 0; i < GRID; ++i) grid[i] = 0.5 + 0.3 * i;
  float temps[SGM], asts[SN * SGM];
  int64_t eu[SGM], e1[SGM];
  oracle_sts_fit(SN, SGM, s, y, GRID, grid, BINS, temps, eu, e1, asts);
  for (int j = 0; j < SGM; ++j) CHECK(eu[j] <= e1[j]);
  float av[SN];
  for (int i = 0; i < SN; ++i) av[i] = (float)(0.5 + 0.5 * lcg(&st));
  CHECK(oracle_ece_units(SN, av, y, BINS) >= 0);
  CHECK(oracle_tau_units(1.0f) == ((int64_t)1 << 38));
  printf("ok\n");
  return 0;
}
