// kernels.h -- host-side launchers shared between the kernel translation units
// and the C-ABI layer.  Every launcher only enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

constexpr int kRank = 256;       // Markov-head rank (summary page §3.1 default)
constexpr int kTile = 32;        // vocabulary entries per MFMA tile
constexpr int kSteps = kRank / 16;

enum BiasMode { kModeDraft = 0, kModeCstar = 1, kModeResidual = 2 };

// Bytes of the packed W2 tiles (bf16: 16 KB MFMA tiles of 32 tokens; binary32:
// the transposed matrix padded to whole tiles).  The per-tile max|W2| array
// (one float per tile) follows them in the same buffer.
__host__ __device__ inline int64_t w2_tiles_bytes(bool bf16, int ntiles) {
  return bf16 ? (int64_t)ntiles * kSteps * 64 * 16 : (int64_t)ntiles * kTile * kRank * 4;
}
__host__ __device__ inline float* w2_tile_absmax(void* W2p, bool bf16, int ntiles) {
  return reinterpret_cast<float*>(static_cast<char*>(W2p) + w2_tiles_bytes(bf16, ntiles));
}
__host__ __device__ inline const float* w2_tile_absmax(const void* W2p, bool bf16, int ntiles) {
  return reinterpret_cast<const float*>(static_cast<const char*>(W2p) + w2_tiles_bytes(bf16, ntiles));
}

// Error bound of the binary32 contraction.  The split passes form
// B_v = sum_i W1[x, i] W2[i, v] with binary32 products and sums starting from
// zero (256 roundings at most), then z_v = U_v + B_v with one more rounding:
// |z_v - exact| <= 256 u S_v + u |z_v|, u = 2^-24, S_v = sum_i |W1[x,i] W2[i,v]|
// <= ||W1[x]||_1 max_{i, v in tile} |W2[i,v]|.  kContractErr = 2^-15 covers
// 256 u twice over (the rounding of the L1 norm itself included).
constexpr float kContractErr = 0x1p-15f;

// Brackets one kernel launch with HIP events when library timing is enabled
// (dspark_timing_enable); a no-op otherwise.
class TimingScope {
 public:
  TimingScope(const char* name, hipStream_t stream);
  ~TimingScope();

 private:
  int slot_;
  hipStream_t stream_;
};

// Partial results of a two-level Gumbel-max draw, one record per (row, split).
// Block b (vocabulary entries [32b, 32b+32)) has a binary32 score whose exact
// binary64 value lies in [lo_b, hi_b].  The record keeps the split's largest
// lower bound, its largest upper bound with that block, and the second largest
// upper bound; a later binary64 pass rescores every block that can still win.
struct BlockCands {
  float* lo;
  float* hi1;
  int32_t* b1;
  float* hi2;
};

// Arguments of one split-vocabulary pass over a set of (request, position)
// rows: bias B = W1[x_{k-1}] W2 plus backbone logits U, consumed by a
// mode-specific epilogue.  Partial records are indexed [row * nsplit + split].
// Matrix-core B operands of the draft: the W1 row of row r's previous token,
// bf16, in the lane order of the bias pass (16-byte chunk c = 16h + s of the
// row, elements [128h + 8s, 128h + 8s + 8), goes to lane (r % 32) + 32h of
// step s of 32-row group r / 32), so that a wave loads its 32 rows' operands
// with 16 lane-contiguous 1 KB loads.  Index of that chunk, in 16-byte units:
__host__ __device__ inline int64_t bop_chunk(int r, int s, int h) {
  return ((int64_t)(r >> 5) * kSteps + s) * 64 + (r & 31) + 32 * h;
}

struct BiasPassArgs {
  int R, gamma, V;
  uint64_t seed;
  int k;                      // draft: 1-based block position of every row
  const int32_t* row_ids;     // verify passes: row id r*gamma + (k-1); null in draft
  const int32_t* row_count;   // verify passes: device count of valid rows
  int nrows;                  // row capacity
  const void* U;
  const void* T;
  const void* W1;
  const void* W2p;
  const int32_t* anchors;
  const int32_t* tokens;
  const void* bop;            // draft, bf16: B operands (bop_chunk order), or null: gather W1 rows
  const double* lse_d;        // [R*gamma]
  const double* lse_t;        // [R*(gamma+1)]
  int ntiles;                 // ceil(V / 32)
  int vec_ok;                 // U/T rows 16-byte aligned: vector loads allowed
  int tiles_per_stage;        // tiles per pipeline stage (split granularity)
  int nsplit;                 // vocabulary splits; with `dyn`, the launched split columns
  int rec_stride;             // partial records per row (>= every split count the pass uses)
  int dyn;                    // splits follow the device row count (active_split_count)
  float* pm;                  // draft: running max per partial
  double* ps;                 // draft: sum of exp; cstar: sum of min(p^d, p^t)
  BlockCands cand;            // draft: blocks of p^d; residual: blocks of max(0, p^t - p^d)
  BlockCands cand_f;          // residual: blocks of p^t (empty-residual fallback)
  float* wpos;                // residual: residual mass seen by the split
  float* zout;                // draft, optional: every logit z = U + B [R, gamma, V]
};

struct BiasGeometry {
  int rows_per_block;  // 256
  int row_blocks;
  int tiles_per_stage;
  int nsplit;
};
BiasGeometry bias_geometry(int mode, bool bf16, int nrows, int V);
// Splits of the small-batch draft and residual passes (at most 32 rows, bf16; tile-granular
// splits, one per workgroup), or 0 when the batch is larger.
int small_pass_splits(int nrows, int V);

// First tile of split `s` of a pass with `nsplit` splits over ntiles tiles
// grouped in stages of `tps` tiles (split s covers [split_tile(s), split_tile(s+1))).
__host__ __device__ inline int split_tile(int s, int nsplit, int ntiles, int tps) {
  const int nstages = (ntiles + tps - 1) / tps;
  const int st = (int)((int64_t)s * nstages / nsplit);
  const int t = st * tps;
  return t < ntiles ? t : ntiles;
}

// Splits of a pass whose active row count is known on the device only: the
// `grid` launched workgroups go to the row blocks (256 rows) that hold active
// rows, `grid / blocks` vocabulary splits each, at most `max_split`.  The count
// is rounded down to a multiple of 8 when that idles at most 1/8 of the
// workgroups: with workgroup id = block * splits + split, every row block of a
// split then runs on one XCD (ids are dealt to the 8 XCDs in turn) and shares
// that XCD's L2 copy of the W2 tiles.
__host__ __device__ inline int active_split_count(int grid, int active_rows, int max_split) {
  constexpr int kBlockRows = 256;
  const int blocks = active_rows > kBlockRows ? (active_rows + kBlockRows - 1) / kBlockRows : 1;
  int ns = grid / blocks;
  ns = ns < max_split ? ns : max_split;
  const int ns8 = ns & ~7;
  if (ns8 > 0 && 8 * (ns - ns8) <= ns) ns = ns8;
  return ns > 1 ? ns : 1;
}

hipError_t launch_bias_pass(int mode, bool bf16, const BiasPassArgs& a, hipStream_t stream);

// Binary64 final stage of a two-level draw: merges the split records of each
// row, rescores the blocks that can still win and draws the member.
enum SelectMode { kSelDraft = 0, kSelResidual = 1, kSelBonus = 2 };
struct SelectArgs {
  int R, gamma, V;
  uint64_t seed;
  int k;                      // draft position (draft mode)
  int ntiles, nsplit, tiles_per_stage;
  const int32_t* row_ids;     // residual: r*gamma + (k*-1); bonus: r*(gamma+1) + l_r
  const int32_t* row_count;   // device count of rows in row_ids
  const void* U;
  const void* T;
  const void* W1;
  const void* W2p;
  const int32_t* anchors;
  const int32_t* tokens;
  const double* lse_d;        // residual mode
  const double* lse_t;        // residual mode
  const float* pm;            // draft: lse partials
  const double* ps;
  BlockCands cand;
  BlockCands cand_f;
  const float* wpos;
  void* bop_out;              // draft, bf16: B operands for the next position (bop_chunk order) or null
  const void* bop_in;         // draft, bf16: this position's B operands (written by the previous select) or null
  int32_t* out_tokens;        // draft: tokens [R, gamma]; residual / bonus: out_token [R]
  double* out_lse;            // draft
  double* out_logq;           // draft
};
hipError_t launch_select(int mode, bool bf16, const SelectArgs& a, hipStream_t stream);
// Residual and bonus draws of a verify in one launch (a: residual list, b: bonus list;
// the two lists hold every request once).
hipError_t launch_select_final(bool bf16, const SelectArgs& ar, const SelectArgs& ab,
                               hipStream_t stream);


// ---- verification helpers ------------------------------------------------
struct VerifyWs {
  int32_t* row_ids;     // [R*gamma]
  int32_t* counts;      // [4]: rows, residual rows, bonus rows, spare
  int32_t* req_off;     // [R] first row of request r in row_ids
  int32_t* req_len;     // [R] clamped verify length
  int32_t* req_slot;    // [R] slot of r in the residual or bonus list
  int32_t* req_mode;    // [R] 1 residual, 2 bonus
  int32_t* resid_ids;   // [R] row ids r*gamma + (k*-1)
  int32_t* bonus_ids;   // [R] target row ids r*(gamma+1) + l_r
  float* lt_m;          // [R*gamma*ns_t] target log-sum-exp partials
  double* lt_s;
  double* lse_t;        // [R*(gamma+1)] merged, NaN where not computed
  double* c_s;          // [R*gamma*ns_c] c* partial sums
  BlockCands r_cand;    // [R*ns_r] residual draw records
  BlockCands r_candf;   // [R*ns_r] its p^t fallback records
  float* r_wpos;        // [R*ns_r]
  BlockCands b_cand;    // [R*ns_b] bonus draw records
  int ns_t, ns_c, ns_r, ns_b;  // ns_t, ns_c: target-lse / c* records per row (their stride)
  int grid_t, grid_c;         // workgroups of the target-lse / c* pass (split counts follow the rows)
  int vec_ok;           // T rows 16-byte aligned: vector loads allowed
  int all_rows;         // every position verified: the target-lse pass writes the identity
                        // row map, the per-request bookkeeping and the counts
};

// Vocabulary splits of the target-lse pass over `active` rows (known on the
// device only): about 2048 workgroups in all, at least 2048 entries per split,
// at most grid / active splits (the launched workgroups), whole 8-entry chunks
// of *chunk entries.  Never more splits for more rows.
__host__ __device__ inline int lse_split_count(int active, int grid, int V, int* chunk) {
  const int rows = active > 1 ? active : 1;
  int ns = (2048 + rows - 1) / rows;
  const int max_split = (V + 2047) / 2048;
  if (ns > max_split) ns = max_split;
  if (ns > grid / rows) ns = grid / rows;
  if (ns < 1) ns = 1;
  int c = (V + ns - 1) / ns;
  c = (c + 7) & ~7;
  *chunk = c;
  return (V + c - 1) / c;
}

hipError_t launch_build_rows(int R, int gamma, const int32_t* lengths, const VerifyWs& w,
                             hipStream_t stream);
hipError_t launch_target_lse(bool bf16, int R, int gamma, int V, const void* T,
                             const VerifyWs& w, hipStream_t stream);
hipError_t launch_decide(bool bf16, int R, int gamma, int V, uint64_t seed, const void* T,
                         const int32_t* tokens, const double* logq, const VerifyWs& w,
                         int32_t* n_accept, uint8_t* accept_mask, double* lse_t_out,
                         hipStream_t stream);
hipError_t launch_bonus(bool bf16, int R, int gamma, int V, uint64_t seed, const void* T,
                        const VerifyWs& w, float* cstar, hipStream_t stream);

// ---- other stages ---------------------------------------------------------
hipError_t launch_pack_w2(bool bf16, int V, const void* W2, void* W2p, hipStream_t stream);
hipError_t launch_logpd(int rows, int V, const double* lse, float* zl, hipStream_t stream);
// Device-side input check: counts (int64, device) of the kCheckCounts classes
// of dspark_check_inputs, overwritten.
constexpr int kCheckCounts = 6;
hipError_t launch_check_inputs(bool bf16, int R, int gamma, int V, const void* U, const void* T,
                               const void* W1, const void* W2, const int32_t* anchors,
                               const int32_t* tokens, const float* c, int64_t* counts,
                               hipStream_t stream);
hipError_t launch_confidence(bool w1_bf16, int R, int gamma, int V, int H, const uint16_t* h,
                             const float* w, const float* temps, const void* W1,
                             const int32_t* anchors, const int32_t* tokens, float* c,
                             hipStream_t stream);
hipError_t launch_schedule(int R, int gamma, const float* c, const float* sps, float* a,
                           int32_t* lengths, double* stats, double* theta_path,
                           hipStream_t stream);
hipError_t launch_schedule_capacity(int R, int gamma, const float* c, const float* sps,
                                    float* a, int32_t* K, int32_t* lengths, double* stats,
                                    double* theta_path, hipStream_t stream);
hipError_t launch_schedule_topk(int R, int gamma, const float* c, const int32_t* K,
                                const float* sps, float* a, int32_t* lengths, double* stats,
                                hipStream_t stream);

// ---- Sequential Temperature Scaling fit -------------------------------------
constexpr int kStsMaxBins = 64;
constexpr int kStsMaxGrid = 1024;
size_t sts_workspace_bytes(int gamma, int G, int bins);
hipError_t launch_sts_fit(int N, int gamma, const double* s, const uint8_t* y, int G,
                          const double* grid, int bins, float* temps, int64_t* ece_units,
                          int64_t* ece1_units, float* a, void* ws, hipStream_t stream);

// ---- static threshold and acceptance statistics ---------------------------
constexpr int kMaxThresholds = 1024;
hipError_t launch_threshold(int R, int gamma, const float* c, double theta, float* a,
                            int32_t* lengths, hipStream_t stream);
hipError_t launch_acceptance_stats(int R, int gamma, const uint8_t* mask, const float* a,
                                   const int32_t* n_accept, const double* thresholds, int n_thr,
                                   int64_t* reached, int64_t* accepted, int64_t* sweep_verified,
                                   int64_t* sweep_accepted, hipStream_t stream);

}  // namespace dspark
