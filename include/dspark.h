/*
 * dspark.h -- C ABI of the MI355X (gfx950) DSpark draft-and-verify hot path.
 *
 * Pages cited (titles as published):
 *   [P1] "DSpark: Confidence-Scheduled Speculative Decoding with
 *        Semi-Autoregressive Generation 요약 설명" (summary page)
 *   [P2] "DSpark: Confidence-Scheduled Speculative Decoding with
 *        Semi-Autoregressive Generation" (notes page, "DSpark 핵심 기술")
 *
 * Conventions shared by every entry point
 *   - Tensor arguments are DEVICE pointers, row-major, owned by the caller.  The
 *     library keeps no pointer after the work it enqueued has completed and
 *     allocates no memory on the hot path (scratch comes from the caller's
 *     workspace, sized by the *_workspace_bytes queries).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *     call is asynchronous on it; outputs are valid after the stream syncs.
 *     Calls on different streams must use different workspaces.
 *   - Arguments are checked on the host before anything is enqueued.  On error
 *     the call returns a negative dspark_status, enqueues nothing, leaves the
 *     outputs untouched and records a message for dspark_last_error().
 *   - Values the host cannot see (token ids, confidences, logits) are
 *     preconditions: token ids must lie in [0, V), confidences in [0, 1], and
 *     the logits U, T and the weights finite (a logit may be -inf to mask an
 *     entry); out-of-range values or NaN give unspecified results but every
 *     memory access stays in bounds (token ids are clamped before they index
 *     W1).
 *   - dtype: DSPARK_F32 (binary32) or DSPARK_BF16 (bfloat16 bit patterns) for
 *     U, T, W1 and W2.  The Markov-head rank must be 256 (the pages' default).
 *   - Random numbers: Philox4x32-10 (Salmon et al., SC'11) with key words
 *     (seed mod 2^32, seed >> 32) and counter (i>>2, k, r, stream), taking word
 *     i&3 of the output; r is the request index, k the 1-based block position
 *     and i the element index within the stream (a token id or a block index,
 *     below).  Uniform u = ((w>>9) + 1/2) 2^-23; Gumbel variate
 *     G(stream, r, k, i) = -ln(-ln u).
 *   - Categorical draws: every token the library samples is a two-level
 *     Gumbel-max draw from softmax(w) over a row of V log-weights w (entries may
 *     be -inf).  The vocabulary is cut into blocks b of 32 tokens
 *     [32b, 32b+32), the last one shorter when 32 does not divide V, and
 *       block  b* = argmax_b ( log sum_{v in b} exp(w_v) + G(S, r, k, b) ),
 *       token  x  = argmax_{v in b*} ( w_v + G(S + 4, r, k, v) ),
 *     the lowest block, then the lowest token, winning exact ties (a block with
 *     no finite entry never wins).  P(x = v) = softmax(w)_v exactly.  The
 *     streams S (block) / S + 4 (member) are 0 / 4 for the draft, 2 / 6 for the
 *     residual draw and 3 / 7 for the bonus draw; stream 1 holds the acceptance
 *     uniforms (element i = 0).  The library takes each decision in binary64 on
 *     the stored inputs; its binary32 screening only skips blocks that a
 *     proven error bound shows cannot win.
 *   - No C++ exception crosses this interface.
 */
#ifndef DSPARK_H_
#define DSPARK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSPARK_OK = 0,
  DSPARK_ERR_ARG = -1,        /* null pointer or negative / zero size */
  DSPARK_ERR_SHAPE = -2,      /* unsupported dimension */
  DSPARK_ERR_DTYPE = -3,      /* unknown dtype */
  DSPARK_ERR_WORKSPACE = -4,  /* workspace missing, too small or misaligned */
  DSPARK_ERR_RANGE = -5,      /* host-visible value out of range */
  DSPARK_ERR_HIP = -6         /* HIP runtime error while enqueuing */
} dspark_status;

typedef enum { DSPARK_F32 = 0, DSPARK_BF16 = 1 } dspark_dtype;

/* One decoding round's problem: R requests, gamma block positions, vocabulary
 * V, Markov-head rank, storage dtype and the round's random seed.
 * Limits: 1 <= R <= 65536, 1 <= gamma <= 64, 1 <= V < 2^26, R*gamma <= 2^20. */
typedef struct {
  int32_t R;
  int32_t gamma;
  int32_t V;
  int32_t rank;
  int32_t dtype;
  int32_t reserved;  /* must be 0 */
  uint64_t seed;
} dspark_problem;

/* Bytes of the packed W2 operand (see dspark_pack_w2). Returns 0 on bad input. */
size_t dspark_w2_packed_bytes(const dspark_problem* p);

/* Repack the Markov-head factor W2 [rank, V] into the vocabulary-major layout
 * the kernels stream (a once-per-model weight preparation, not part of a round).
 * W2p must hold dspark_w2_packed_bytes(p) bytes, 256-byte aligned.  With
 * n = ceil(V/32) tiles of 32 tokens:
 *   bf16: tile t holds 16 steps x 64 lanes x 8 values, entry
 *         ((t*16 + s)*64 + l)*8 + e = W2[128*(l/32) + 8*s + e][32*t + pi(l%32)],
 *         pi(m) = 16*((m>>2)&1) + 4*(m>>3) + (m&3), zero beyond V (n*16 KB).
 *   f32:  W2 transposed, [n*32, rank], zero rows beyond V.
 * Then n floats: tile t's max |W2[i][v]| over i < rank and its tokens v < V
 * (the factor of the contraction's error bound). */
int dspark_pack_w2(const dspark_problem* p, const void* W2, void* W2p, void* stream);

/* Workspace bytes needed by dspark_draft_step and dspark_verify for problem p
 * (one buffer serves both when they run on one stream). 0 on bad input. */
size_t dspark_workspace_bytes(const dspark_problem* p);

/* Stage 1 -- Markov-head semi-autoregressive draft sampling.  [P1 §3.1; P2]
 * For k = 1..gamma and every request r, with x_0 = anchors[r]:
 *   z_v = U[r,k-1,v] + sum_i W1[x_{k-1}, i] W2[i, v]      (rank-256 bias B_k)
 *   lse[r,k-1]  = log sum_v exp(z_v)                     (p^d_k = softmax(z))
 *   x_k         = the two-level draw from softmax(z) with streams 0 / 4 at (r, k)
 *   logq[r,k-1] = z_{x_k} - lse[r,k-1]                   (log p^d_k(x_k))
 * U: [R, gamma, V] dtype; W1: [V, 256] dtype; W2p: packed W2; anchors: [R] int32.
 * Outputs: tokens [R, gamma] int32, lse and logq [R, gamma] float64.
 * logpd: NULL, or float32 [R, gamma, V] that receives log p^d_k(v) = z_v - lse
 * of every position (a parity / debugging output that costs a full write;
 * z in binary32, the difference in binary64 rounded to binary32).
 * ws: dspark_workspace_bytes(p) bytes, 256-byte aligned. */
int dspark_draft_step(const dspark_problem* p, const void* U, const void* W1, const void* W2p,
                      const int32_t* anchors, int32_t* tokens, double* lse, double* logq,
                      float* logpd, void* ws, size_t ws_bytes, void* stream);

/* dspark_draft_step without a workspace, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, outputs and results as
 * dspark_draft_step; the draft's scratch (split records and the next
 * position's matrix-core operands) is a fixed 8 MiB device array of the
 * library instead, one per GPU, held until the process ends.  The call
 * allocates nothing and records no timing events.  Problems whose draft
 * scratch exceeds 8 MiB are rejected with DSPARK_ERR_WORKSPACE (every R up to
 * 8192 fits at V <= 2^20).  The array of the current device is used: calls
 * that overlap on one GPU (on different streams, or from different threads)
 * race on it and must be ordered by the caller; a call may start once the
 * previous call's work on that GPU has been enqueued before it on the same
 * stream, or has completed.  Nothing in the array needs to start at zero. */
int dspark_draft_step_noalloc(const dspark_problem* p, const void* U, const void* W1,
                              const void* W2p, const int32_t* anchors, int32_t* tokens,
                              double* lse, double* logq, float* logpd, void* stream);

/* Stage 2 -- standard speculative rejection sampling with bonus token, and the
 * analytic acceptance c*.  [P1 요약, §3.2.1; P2 배경]
 * For request r with verify length l_r = lengths[r] (all gamma if lengths is
 * NULL), for k = 1..l_r:
 *   p^d_k = softmax(U[r,k-1] + W1[x_{k-1}] W2) (recomputed; lse_d from stage 1)
 *   p^t_k = softmax(T[r,k-1])
 *   cstar[r,k-1] = sum_v min(p^d_k, p^t_k) = 1 - ||p^d_k - p^t_k||_1 / 2
 *   accept x_k iff ln u < ln p^t_k(x_k) - logq[r,k-1], u = uniform(stream 1, r, k, v=0)
 * n_accept[r] = number of leading accepted positions.  If a position k* <= l_r
 * is rejected, out_token[r] = the two-level draw from the normalised
 * max(0, p^t_{k*} - p^d_{k*}) (log-weights ln max(0, p^t - p^d)) with streams
 * 2 / 6 at (r, k*), or from p^t_{k*} with the same streams if no entry has
 * p^t > p^d in binary64; otherwise out_token[r] = the two-level draw from
 * softmax(T[r,l_r]) = p^t_{l_r+1} with streams 3 / 7 at (r, l_r + 1) (bonus).
 * T: [R, gamma+1, V] dtype (row gamma is the bonus row).  tokens, lse_d, logq:
 * stage-1 outputs.  lengths: [R] int32 in [0, gamma] or NULL.
 * Outputs: cstar [R, gamma] float32 (NaN for k > l_r); n_accept, out_token [R]
 * int32; accept_mask [R, gamma] uint8 or NULL (1 accepted, 0 rejected, 255 not
 * decided); lse_t [R, gamma+1] float64 or NULL (NaN where not computed). */
int dspark_verify(const dspark_problem* p, const void* U, const void* W1, const void* W2p,
                  const int32_t* anchors, const int32_t* tokens, const double* lse_d,
                  const double* logq, const void* T, const int32_t* lengths, float* cstar,
                  int32_t* n_accept, int32_t* out_token, uint8_t* accept_mask, double* lse_t,
                  void* ws, size_t ws_bytes, void* stream);

/* Confidence head with Sequential Temperature Scaling.  [P1 §3.2.1]
 * c[r,k-1] = 1 / (1 + exp(-(w . [h[r,k-1,:]; W1[x_{k-1},:]]) / temps[k-1])),
 * evaluated in float64 and rounded to float32.  h: [R, gamma, H] bfloat16;
 * w: [H + 256] float32; temps: [gamma] float32 (> 0); W1 [V, 256] in p->dtype;
 * anchors [R], tokens [R, gamma] int32.  Output c: [R, gamma] float32.
 * Limits: 1 <= H <= 65536. */
int dspark_confidence(const dspark_problem* p, int32_t H, const uint16_t* h, const float* w,
                      const float* temps, const void* W1, const int32_t* anchors,
                      const int32_t* tokens, float* c, void* stream);

/* Stages 3-4 -- prefix-survival products and the hardware-aware prefix
 * scheduler (Algorithm 1).  [P1 §3.2.2]
 *   a[r,j-1] = a[r,j-2] * c[r,j-1] in binary32, a[r,0] = c[r,0]
 *   candidates (r, j) in order of the key (-a[r,j-1], r, j); start from l = 0,
 *   B = R, tau = R, Theta = R * sps[R-1]; take candidates while
 *   Theta' = tau' * sps[B'-1] > Theta (strict), B' = B + 1, tau' = tau + a;
 *   stop at the first non-improvement (causal).  tau is accumulated exactly in
 *   units of 2^-38 (each a rounded to nearest-even), Theta = double(tau) * SPS.
 * c: [R, gamma] float32 in [0, 1]; sps: [n_sps] float32, sps[B-1] = SPS(B),
 * n_sps >= R*(gamma+1).  Outputs: a [R, gamma] float32; lengths [R] int32;
 * stats [4] float64 = (B, tau, Theta, n_selected); theta_path [R*gamma+1]
 * float64 or NULL (Theta before any candidate, then after each examined
 * candidate up to and including the stopping one, NaN afterwards).
 * Limit: R*gamma <= 16384.  No workspace is needed. */
int dspark_schedule(int32_t R, int32_t gamma, const float* c, const float* sps, int32_t n_sps,
                    float* a, int32_t* lengths, double* stats, double* theta_path, void* stream);

/* Production variant of the scheduler: capacity.  [P1 §5.2]
 * The deployed scheduler sets a round's capacity K from confidences two
 * rounds old and leaves out the early-stopping break, so that the search is
 * not caught in a local optimum at a throughput cliff of an irregular SPS(B).
 * Here: a = prefix products of c (as in dspark_schedule), candidates in the
 * same survival order, Theta_i = tau_i * sps[R+i-1] after the first i
 * candidates (i = 0..R*gamma, tau as in dspark_schedule); K = the smallest i
 * with the largest Theta_i, written to K[0] on the device (a later round reads
 * it there with no host synchronisation).  lengths [R]: the top-K verify
 * lengths on these same confidences; stats [4] = (B, tau, Theta, K) at K;
 * theta_path [R*gamma+1] float64 or NULL: every Theta_i.  sps entries must be
 * finite and >= 0.  Limit: R*gamma <= 16384. */
int dspark_schedule_capacity(int32_t R, int32_t gamma, const float* c, const float* sps,
                             int32_t n_sps, float* a, int32_t* K, int32_t* lengths,
                             double* stats, double* theta_path, void* stream);

/* Production variant of the scheduler: top-K.  [P1 §5.2]
 * Verify the first min(K[0], R*gamma) candidates (K[0] < 0 counts as 0) in the
 * survival order of this round's c; K is a device int32 (normally written by
 * dspark_schedule_capacity two rounds earlier).  a [R, gamma] float32;
 * lengths [R] int32 (prefixes, since a request's survival never rises);
 * stats [4] = (B, tau, Theta, taken), Theta = tau * sps[B-1].
 * Limit: R*gamma <= 16384. */
int dspark_schedule_topk(int32_t R, int32_t gamma, const float* c, const int32_t* K,
                         const float* sps, int32_t n_sps, float* a, int32_t* lengths,
                         double* stats, void* stream);

/* Static-threshold verify lengths.  [P1 §4.3.3]
 * a = binary32 prefix products of c [R, gamma]; lengths[r] = the largest j
 * with a[r,i-1] >= theta (compared in binary64) for every i <= j.
 * theta must not be NaN.  Limits: 1 <= R <= 65536, 1 <= gamma <= 64. */
int dspark_schedule_threshold(int32_t R, int32_t gamma, const float* c, double theta, float* a,
                              int32_t* lengths, void* stream);

/* Acceptance statistics of one verified round.  [P1 §4.3.1, §4.3.3]
 * accept_mask [R, gamma] (dspark_verify's: 1 accepted, 0 rejected, 255 not
 * verified) or NULL.  Position k counts only rollouts whose positions 1..k-1
 * were all accepted: reached[k-1] = requests with positions 1..k-1 accepted
 * and position k verified, accepted[k-1] = those that accepted position k
 * (int64 [gamma] each).  Threshold sweep (n_thr in [0, 1024]; a [R, gamma]
 * survival products, n_accept [R] the accepted lengths of a verify of all
 * gamma positions, thresholds [n_thr] float64): sweep_verified[g] = sum_r
 * l_r(thresholds[g]) with l_r as in dspark_schedule_threshold, and
 * sweep_accepted[g] = sum_r min(n_accept[r], l_r) -- the tokens a verify
 * limited by that threshold checks and accepts.  One workgroup for the mask and
 * one per threshold; no workspace. */
int dspark_acceptance_stats(int32_t R, int32_t gamma, const uint8_t* accept_mask, const float* a,
                            const int32_t* n_accept, const double* thresholds, int32_t n_thr,
                            int64_t* reached, int64_t* accepted, int64_t* sweep_verified,
                            int64_t* sweep_accepted, void* stream);

/* Sequential Temperature Scaling fit.  [P1 §3.2.1]
 * Calibrates the prefix survival on N held-out rollouts by a left-to-right
 * grid search: for j = 1..gamma, with the temperatures of positions < j fixed,
 *   a_j(T) = fl32(a_{j-1} * fl32(1 / (1 + exp(-s[n,j-1] / T)))) (binary64
 *            sigmoid rounded to binary32; a_0 = 1),
 *   N * ECE_j(T) = sum over bins b of |sum_{n in b} (y[n,j-1] - a_j(T))|, bins
 *            = min(floor(a * bins), bins - 1) over [0, 1], every a rounded to
 *            the nearest multiple of 2^-40 (exact integer sums),
 * and T_j = the grid value with the smallest ECE (lowest index on ties).
 * s: [N, gamma] float64 confidence-head scores (the logit before the sigmoid);
 * y: [N, gamma] uint8 survival labels (1 iff positions 1..j were all
 * accepted); grid: [G] float64 candidate temperatures (> 0).
 * Outputs: temps [gamma] float32 (T_j); ece_units, ece1_units [gamma] int64:
 * N * ECE in units of 2^-40 at T_j and at T = 1 (earlier positions
 * calibrated); a [N, gamma] float32, the calibrated survival.
 * ws: dspark_sts_workspace_bytes(N, gamma, G, bins) bytes, 256-byte aligned
 * (0 = bad sizes).  Limits: 1 <= N <= 2^20, 1 <= gamma <= 64, 1 <= G <= 1024,
 * 1 <= bins <= 64.  3 * gamma + 1 launches. */
size_t dspark_sts_workspace_bytes(int32_t N, int32_t gamma, int32_t G, int32_t bins);
int dspark_sts_fit(int32_t N, int32_t gamma, const double* s, const uint8_t* y, int32_t G,
                   const double* grid, int32_t bins, float* temps, int64_t* ece_units,
                   int64_t* ece1_units, float* a, void* ws, size_t ws_bytes, void* stream);

/* Device-side check of the values the host cannot see, the preconditions
 * above (a debugging aid, off the hot path: one pass over every tensor given).
 * counts: int64 [6] in device memory, overwritten with the number of
 *   0: anchors [R] outside [0, V)
 *   1: tokens [R, gamma] outside [0, V)
 *   2: entries of U [R, gamma, V] that are NaN or +inf (-inf masks an entry)
 *   3: entries of T [R, gamma+1, V] that are NaN or +inf
 *   4: entries of W1 [V, 256] and W2 [256, V] (as given to dspark_pack_w2)
 *      that are NaN or infinite
 *   5: confidences c [R, gamma] (float32) outside [0, 1] or NaN.
 * Any tensor may be NULL (its count stays 0).  U, T, W1 and W2 are in p->dtype
 * and must be aligned to their element size, the int32 / float32 tensors to 4
 * bytes and counts to 8. */
int dspark_check_inputs(const dspark_problem* p, const void* U, const void* T, const void* W1,
                        const void* W2, const int32_t* anchors, const int32_t* tokens,
                        const float* c, int64_t* counts, void* stream);

/* Message for the last failing call on this thread ("" if none). */
const char* dspark_last_error(void);

/* Per-kernel timing with HIP events (tracing; off by default).
 * dspark_timing_enable(1) clears the record and brackets every kernel the
 * library enqueues from then on with a pair of events on that kernel's
 * stream; dspark_timing_enable(0) stops recording.  dspark_timing_report
 * waits for the recorded events and writes one line per kernel name,
 * "name launches total_ms\n", into buf (NUL-terminated, truncated to cap),
 * then clears the record; with buf NULL it only returns the size and keeps
 * the record.  Returns the bytes needed (excluding the NUL) or a negative
 * dspark_status. */
int dspark_timing_enable(int on);
int dspark_timing_report(char* buf, size_t cap);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H_ */
