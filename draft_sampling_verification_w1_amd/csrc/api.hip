// api.hip -- the C ABI (include/dspark.h): host-side validation, workspace
// carving and the launch sequence of each stage.  Host code only.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "dspark.h"
#include "kernels.h"

using namespace dspark;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return DSPARK_OK;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(DSPARK_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

int check_problem(const dspark_problem* p) {
  if (!p) return fail(DSPARK_ERR_ARG, "problem is NULL");
  if (p->dtype != DSPARK_F32 && p->dtype != DSPARK_BF16)
    return fail(DSPARK_ERR_DTYPE, "dtype %d is not DSPARK_F32 or DSPARK_BF16", p->dtype);
  if (p->reserved != 0) return fail(DSPARK_ERR_ARG, "reserved field must be 0");
  if (p->R < 1 || p->R > 65536) return fail(DSPARK_ERR_SHAPE, "R=%d outside [1, 65536]", p->R);
  if (p->gamma < 1 || p->gamma > 64)
    return fail(DSPARK_ERR_SHAPE, "gamma=%d outside [1, 64]", p->gamma);
  if (p->V < 1 || p->V >= (1 << 26)) return fail(DSPARK_ERR_SHAPE, "V=%d outside [1, 2^26)", p->V);
  if (p->rank != kRank) return fail(DSPARK_ERR_SHAPE, "rank=%d, only %d is supported", p->rank, kRank);
  if ((int64_t)p->R * p->gamma > (1 << 20))
    return fail(DSPARK_ERR_SHAPE, "R*gamma=%lld exceeds 2^20", (long long)p->R * p->gamma);
  return DSPARK_OK;
}

// Workspace layout.  Draft and verify run one after the other on a stream,
// so they share one buffer (the size is the larger of the two layouts).
struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  }
};

struct CandLayout {
  size_t lo, hi1, b1, hi2;
};

CandLayout take_cands(Carver& c, size_t n) {
  CandLayout L;
  L.lo = c.take(n * sizeof(float));
  L.hi1 = c.take(n * sizeof(float));
  L.b1 = c.take(n * sizeof(int32_t));
  L.hi2 = c.take(n * sizeof(float));
  return L;
}

BlockCands cands_at(void* ws, const CandLayout& L);

struct DraftLayout {
  BiasGeometry g;
  size_t pm, ps, bop, bytes;
  CandLayout cand;
};

DraftLayout draft_layout(const dspark_problem* p) {
  DraftLayout L;
  L.g = bias_geometry(kModeDraft, p->dtype == DSPARK_BF16, p->R, p->V);
  // the small-batch pass (at most 32 rows, bf16) may use more, tile-granular splits
  const int ns_small = p->dtype == DSPARK_BF16 ? small_pass_splits(p->R, p->V) : 0;
  const size_t n = (size_t)p->R * (ns_small > L.g.nsplit ? ns_small : L.g.nsplit);
  Carver c;
  L.pm = c.take(n * sizeof(float));
  L.ps = c.take(n * sizeof(double));
  L.cand = take_cands(c, n);
  // B operands of every row a bias workgroup covers (whole blocks of rows)
  L.bop = c.take((size_t)L.g.row_blocks * L.g.rows_per_block * kRank * 2);
  L.bytes = c.off;
  return L;
}

// Splits per bonus row: about 2048 workgroups in all, whole 32-token blocks.
int bonus_splits(int R, int V) {
  const int ntiles = (V + kTile - 1) / kTile;
  const int ns = (2048 + R - 1) / R;
  return ns < 1 ? 1 : (ns > ntiles ? ntiles : ns);
}

struct VerifyLayout {
  BiasGeometry gc, gr;
  int ns_r, small_r;  // residual pass: splits (records per row); 1 = the small-batch pass
  int grid_c, rec_c;  // c* pass: workgroups launched, records per row
  int grid_t, ns_t, ns_b;  // target lse: workgroups launched, records per row
  size_t row_ids, counts, req_off, req_len, req_slot, req_mode, resid_ids, bonus_ids;
  size_t lt_m, lt_s, lse_t, c_s, r_wpos, bytes;
  CandLayout r_cand, r_candf, b_cand;
};

VerifyLayout verify_layout(const dspark_problem* p) {
  VerifyLayout L;
  const size_t R = p->R, rows = (size_t)p->R * p->gamma;
  L.gc = bias_geometry(kModeCstar, p->dtype == DSPARK_BF16, (int)rows, p->V);
  L.gr = bias_geometry(kModeResidual, p->dtype == DSPARK_BF16, p->R, p->V);
  // at most 32 requests (bf16): the residual rows go through the small-batch
  // pass, on its tile-granular splits
  const int ns_small = p->dtype == DSPARK_BF16 ? small_pass_splits(p->R, p->V) : 0;
  L.small_r = ns_small > 0 ? 1 : 0;
  L.ns_r = ns_small > 0 ? ns_small : L.gr.nsplit;
  // the c* pass spreads its workgroups over the row blocks that hold verified
  // rows (known on the device only): up to one split per workgroup
  L.grid_c = L.gc.nsplit * L.gc.row_blocks;
  const int c_stages = ((p->V + kTile - 1) / kTile + L.gc.tiles_per_stage - 1) / L.gc.tiles_per_stage;
  L.rec_c = L.grid_c < c_stages ? L.grid_c : c_stages;
  // target lse: splits for every position set the grid; fewer verified rows
  // take more splits each (at most the count for one row: the record stride)
  int chunk;
  L.grid_t = (int)rows * lse_split_count((int)rows, 1 << 30, p->V, &chunk);
  L.ns_t = lse_split_count(1, L.grid_t, p->V, &chunk);
  L.ns_b = bonus_splits(p->R, p->V);
  Carver c;
  L.row_ids = c.take(rows * 4);
  L.counts = c.take(4 * 4);
  L.req_off = c.take(R * 4);
  L.req_len = c.take(R * 4);
  L.req_slot = c.take(R * 4);
  L.req_mode = c.take(R * 4);
  L.resid_ids = c.take(R * 4);
  L.bonus_ids = c.take(R * 4);
  L.lt_m = c.take(rows * L.ns_t * sizeof(float));
  L.lt_s = c.take(rows * L.ns_t * sizeof(double));
  L.lse_t = c.take(R * (p->gamma + 1) * sizeof(double));
  L.c_s = c.take(rows * L.rec_c * sizeof(double));
  L.r_cand = take_cands(c, R * L.ns_r);
  L.r_candf = take_cands(c, R * L.ns_r);
  L.r_wpos = c.take(R * L.ns_r * sizeof(float));
  L.b_cand = take_cands(c, R * L.ns_b);
  L.bytes = c.off;
  return L;
}

size_t workspace_bytes(const dspark_problem* p) {
  const size_t a = draft_layout(p).bytes, b = verify_layout(p).bytes;
  return a > b ? a : b;
}

int check_ws(const dspark_problem* p, void* ws, size_t ws_bytes) {
  const size_t need = workspace_bytes(p);
  if (!ws) return fail(DSPARK_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if ((uintptr_t)ws % kAlign) return fail(DSPARK_ERR_WORKSPACE, "workspace not %zu-byte aligned", kAlign);
  if (ws_bytes < need)
    return fail(DSPARK_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  return DSPARK_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Vector loads of U / T rows need 16-byte aligned rows: aligned bases and a
// row length that keeps every row start aligned.
int rows_vec_ok(const dspark_problem* p, const void* U, const void* T) {
  const int per = p->dtype == DSPARK_BF16 ? 8 : 4;
  return (p->V % per == 0) && (!U || aligned16(U)) && (!T || aligned16(T));
}

int check_weights(const void* W1, const void* W2p) {
  if (!aligned16(W1)) return fail(DSPARK_ERR_ARG, "W1 must be 16-byte aligned");
  if (!aligned16(W2p)) return fail(DSPARK_ERR_ARG, "W2p must be 16-byte aligned");
  return DSPARK_OK;
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

BlockCands cands_at(void* ws, const CandLayout& L) {
  BlockCands c;
  c.lo = at<float>(ws, L.lo);
  c.hi1 = at<float>(ws, L.hi1);
  c.b1 = at<int32_t>(ws, L.b1);
  c.hi2 = at<float>(ws, L.hi2);
  return c;
}

// Packed tiles, then one float per tile (max |W2| over the tile).
size_t packed_bytes(const dspark_problem* p) {
  const int ntiles = (p->V + kTile - 1) / kTile;
  return (size_t)w2_tiles_bytes(p->dtype == DSPARK_BF16, ntiles) + (size_t)ntiles * sizeof(float);
}

// ---- per-kernel timing (tracing) -----------------------------------------
struct TimingRecord {
  const char* name;
  hipEvent_t start, stop;
  bool stopped;  // the stop event was recorded
};

std::mutex g_timing_mu;
bool g_timing_on = false;
// Set while a call that must not allocate runs on this thread: no timing events
// are created or recorded for its kernels (creating events can allocate).
thread_local bool g_no_events = false;
std::vector<TimingRecord> g_timing_recs;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t pooled_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void recycle_records() {
  for (auto& r : g_timing_recs) {
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_timing_recs.clear();
}

}  // namespace

namespace dspark {

TimingScope::TimingScope(const char* name, hipStream_t stream) : slot_(-1), stream_(stream) {
  if (g_no_events) return;
  std::lock_guard<std::mutex> lock(g_timing_mu);
  if (!g_timing_on) return;
  TimingRecord r{name, pooled_event(), pooled_event(), false};
  if (!r.start || !r.stop || hipEventRecord(r.start, stream) != hipSuccess) return;
  g_timing_recs.push_back(r);
  slot_ = (int)g_timing_recs.size() - 1;
}

TimingScope::~TimingScope() {
  if (slot_ < 0) return;
  std::lock_guard<std::mutex> lock(g_timing_mu);
  if (slot_ < (int)g_timing_recs.size()) {
    TimingRecord& r = g_timing_recs[slot_];
    r.stopped = hipEventRecord(r.stop, stream_) == hipSuccess;
  }
}

}  // namespace dspark

namespace {

// ---- scratch of the no-allocation draft entry point ---------------------------
// A fixed device array (each GPU the library runs on holds its own copy until
// the process ends).  Host code never passes the array's name to a kernel: its
// device address comes from hipGetSymbolAddress, once per device, with that
// device current.  Calls on one GPU share the array (they must not overlap).
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "draft_step_noalloc: current device");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DSPARK_ERR_ARG, "draft_step_noalloc: device %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "draft_step_noalloc: scratch address");
    if (!ptr || (uintptr_t)ptr % kAlign)
      return fail(DSPARK_ERR_HIP, "draft_step_noalloc: scratch address not %zu-byte aligned", kAlign);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DSPARK_OK;
}

// ---- the draft stage: argument checks and launch sequence --------------------
int check_draft_args(const dspark_problem* p, const void* U, const void* W1, const void* W2p,
                     const int32_t* anchors, const int32_t* tokens, const double* lse,
                     const double* logq) {
  if (int e = check_problem(p)) return e;
  if (!U || !W1 || !W2p || !anchors || !tokens || !lse || !logq)
    return fail(DSPARK_ERR_ARG, "draft_step: tensor pointers must be non-NULL");
  if (int e = check_weights(W1, W2p)) return e;
  return DSPARK_OK;
}

// Enqueues every draft position; ws holds at least draft_layout(p).bytes.
int draft_launch(const dspark_problem* p, const void* U, const void* W1, const void* W2p,
                 const int32_t* anchors, int32_t* tokens, double* lse, double* logq,
                 float* logpd, void* ws, void* stream) {
  const bool bf16 = p->dtype == DSPARK_BF16;
  const DraftLayout L = draft_layout(p);
  hipStream_t s = (hipStream_t)stream;
  BiasPassArgs a = {};
  a.R = p->R;
  a.gamma = p->gamma;
  a.V = p->V;
  a.seed = p->seed;
  a.nrows = p->R;
  a.U = U;
  a.W1 = W1;
  a.W2p = W2p;
  a.anchors = anchors;
  a.tokens = tokens;
  a.ntiles = (p->V + kTile - 1) / kTile;
  a.vec_ok = rows_vec_ok(p, U, nullptr);
  a.tiles_per_stage = L.g.tiles_per_stage;
  a.nsplit = L.g.nsplit;
  if (const int ns = bf16 ? small_pass_splits(p->R, p->V) : 0) {
    // at most 32 rows: the small-batch pass, tile-granular splits
    a.tiles_per_stage = 1;
    a.nsplit = ns;
  }
  a.rec_stride = a.nsplit;
  a.pm = at<float>(ws, L.pm);
  a.ps = at<double>(ws, L.ps);
  a.cand = cands_at(ws, L.cand);
  a.zout = logpd;
  SelectArgs q = {};
  q.R = p->R;
  q.gamma = p->gamma;
  q.V = p->V;
  q.seed = p->seed;
  q.ntiles = a.ntiles;
  q.nsplit = a.nsplit;
  q.tiles_per_stage = a.tiles_per_stage;
  q.U = U;
  q.W1 = W1;
  q.W2p = W2p;
  q.anchors = anchors;
  q.tokens = tokens;
  q.pm = a.pm;
  q.ps = a.ps;
  q.cand = a.cand;
  q.out_tokens = tokens;
  q.out_lse = lse;
  q.out_logq = logq;
  // bf16: each select writes the drafted tokens' W1 rows as the next
  // position's matrix-core operands; the first position gathers the anchors'
  void* bop = bf16 ? at<void>(ws, L.bop) : nullptr;
  for (int k = 1; k <= p->gamma; ++k) {
    a.k = k;
    q.k = k;
    a.bop = k > 1 ? bop : nullptr;
    q.bop_out = k < p->gamma ? bop : nullptr;
    q.bop_in = a.bop;
    hipError_t e = launch_bias_pass(kModeDraft, bf16, a, s);
    if (e != hipSuccess) return hip_fail(e, "draft pass");
    e = launch_select(kSelDraft, bf16, q, s);
    if (e != hipSuccess) return hip_fail(e, "draft select");
  }
  if (logpd) {
    hipError_t e = launch_logpd(p->R * p->gamma, p->V, lse, logpd, s);
    if (e != hipSuccess) return hip_fail(e, "draft log p^d");
  }
  return ok();
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int dspark_timing_enable(int on) {
  std::lock_guard<std::mutex> lock(g_timing_mu);
  if (on) recycle_records();
  g_timing_on = on != 0;
  return ok();
}

__attribute__((visibility("default"))) int dspark_timing_report(char* buf, size_t cap) {
  std::lock_guard<std::mutex> lock(g_timing_mu);
  std::map<std::string, std::pair<long, double>> agg;
  std::vector<std::string> order;
  for (auto& r : g_timing_recs) {
    if (!r.stopped) return hip_fail(hipErrorInvalidValue, "timing report: a stop event was not recorded");
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return hip_fail(e, "timing report");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return hip_fail(e, "timing report");
    auto it = agg.find(r.name);
    if (it == agg.end()) {
      order.push_back(r.name);
      agg[r.name] = {1, ms};
    } else {
      it->second.first += 1;
      it->second.second += ms;
    }
  }
  std::string out;
  char line[256];
  for (auto& name : order) {
    snprintf(line, sizeof line, "%s %ld %.6f\n", name.c_str(), agg[name].first, agg[name].second);
    out += line;
  }
  if (buf && cap) {  // a size query (buf NULL) keeps the record
    recycle_records();
    const size_t n = out.size() < cap - 1 ? out.size() : cap - 1;
    memcpy(buf, out.data(), n);
    buf[n] = '\0';
  }
  g_last_error.clear();
  return (int)out.size();
}

__attribute__((visibility("default"))) const char* dspark_last_error(void) {
  return g_last_error.c_str();
}

__attribute__((visibility("default"))) size_t dspark_w2_packed_bytes(const dspark_problem* p) {
  if (check_problem(p) != DSPARK_OK) return 0;
  return packed_bytes(p);
}

__attribute__((visibility("default"))) int dspark_pack_w2(const dspark_problem* p, const void* W2,
                                                          void* W2p, void* stream) {
  if (int e = check_problem(p)) return e;
  if (!W2 || !W2p) return fail(DSPARK_ERR_ARG, "W2 and W2p must be non-NULL");
  if ((uintptr_t)W2p % kAlign) return fail(DSPARK_ERR_ARG, "W2p must be %zu-byte aligned", kAlign);
  hipError_t e = launch_pack_w2(p->dtype == DSPARK_BF16, p->V, W2, W2p, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "pack_w2");
  return ok();
}

__attribute__((visibility("default"))) size_t dspark_workspace_bytes(const dspark_problem* p) {
  if (check_problem(p) != DSPARK_OK) return 0;
  return workspace_bytes(p);
}

__attribute__((visibility("default"))) int dspark_draft_step(
    const dspark_problem* p, const void* U, const void* W1, const void* W2p,
    const int32_t* anchors, int32_t* tokens, double* lse, double* logq, float* logpd, void* ws,
    size_t ws_bytes, void* stream) {
  if (int e = check_draft_args(p, U, W1, W2p, anchors, tokens, lse, logq)) return e;
  if (int e = check_ws(p, ws, ws_bytes)) return e;
  return draft_launch(p, U, W1, W2p, anchors, tokens, lse, logq, logpd, ws, stream);
}

__attribute__((visibility("default"))) int dspark_draft_step_noalloc(
    const dspark_problem* p, const void* U, const void* W1, const void* W2p,
    const int32_t* anchors, int32_t* tokens, double* lse, double* logq, float* logpd,
    void* stream) {
  if (int e = check_draft_args(p, U, W1, W2p, anchors, tokens, lse, logq)) return e;
  const size_t need = draft_layout(p).bytes;
  if (need > kNoAllocScratchBytes)
    return fail(DSPARK_ERR_WORKSPACE,
                "draft_step_noalloc: the problem needs %zu bytes of draft scratch, more than the "
                "library's fixed %zu (use dspark_draft_step with a workspace)",
                need, kNoAllocScratchBytes);
  void* scratch_ptr = nullptr;
  if (int e = noalloc_scratch(&scratch_ptr)) return e;
  g_no_events = true;
  const int e = draft_launch(p, U, W1, W2p, anchors, tokens, lse, logq, logpd, scratch_ptr, stream);
  g_no_events = false;
  return e;
}

__attribute__((visibility("default"))) int dspark_verify(
    const dspark_problem* p, const void* U, const void* W1, const void* W2p,
    const int32_t* anchors, const int32_t* tokens, const double* lse_d, const double* logq,
    const void* T, const int32_t* lengths, float* cstar, int32_t* n_accept, int32_t* out_token,
    uint8_t* accept_mask, double* lse_t, void* ws, size_t ws_bytes, void* stream) {
  if (int e = check_problem(p)) return e;
  if (!U || !W1 || !W2p || !anchors || !tokens || !lse_d || !logq || !T || !cstar || !n_accept ||
      !out_token)
    return fail(DSPARK_ERR_ARG, "verify: tensor pointers must be non-NULL");
  if (int e = check_weights(W1, W2p)) return e;
  if (int e = check_ws(p, ws, ws_bytes)) return e;
  const bool bf16 = p->dtype == DSPARK_BF16;
  const VerifyLayout L = verify_layout(p);
  hipStream_t s = (hipStream_t)stream;
  VerifyWs w;
  w.row_ids = at<int32_t>(ws, L.row_ids);
  w.counts = at<int32_t>(ws, L.counts);
  w.req_off = at<int32_t>(ws, L.req_off);
  w.req_len = at<int32_t>(ws, L.req_len);
  w.req_slot = at<int32_t>(ws, L.req_slot);
  w.req_mode = at<int32_t>(ws, L.req_mode);
  w.resid_ids = at<int32_t>(ws, L.resid_ids);
  w.bonus_ids = at<int32_t>(ws, L.bonus_ids);
  w.lt_m = at<float>(ws, L.lt_m);
  w.lt_s = at<double>(ws, L.lt_s);
  w.lse_t = at<double>(ws, L.lse_t);
  w.c_s = at<double>(ws, L.c_s);
  w.r_cand = cands_at(ws, L.r_cand);
  w.r_candf = cands_at(ws, L.r_candf);
  w.r_wpos = at<float>(ws, L.r_wpos);
  w.b_cand = cands_at(ws, L.b_cand);
  w.ns_t = L.ns_t;
  w.ns_c = L.rec_c;
  w.grid_c = L.grid_c;
  w.ns_r = L.ns_r;
  w.ns_b = L.ns_b;
  w.grid_t = L.grid_t;
  w.vec_ok = rows_vec_ok(p, nullptr, T);
  w.all_rows = lengths == nullptr ? 1 : 0;

  hipError_t e = hipSuccess;
  if (!w.all_rows) {
    e = launch_build_rows(p->R, p->gamma, lengths, w, s);
    if (e != hipSuccess) return hip_fail(e, "verify rows");
  }
  e = launch_target_lse(bf16, p->R, p->gamma, p->V, T, w, s);
  if (e != hipSuccess) return hip_fail(e, "target lse");
  e = launch_decide(bf16, p->R, p->gamma, p->V, p->seed, T, tokens, logq, w, n_accept, accept_mask,
                    lse_t, s);
  if (e != hipSuccess) return hip_fail(e, "decide");

  BiasPassArgs a = {};
  a.R = p->R;
  a.gamma = p->gamma;
  a.V = p->V;
  a.seed = p->seed;
  a.U = U;
  a.T = T;
  a.W1 = W1;
  a.W2p = W2p;
  a.anchors = anchors;
  a.tokens = tokens;
  a.lse_d = lse_d;
  a.lse_t = w.lse_t;
  a.ntiles = (p->V + kTile - 1) / kTile;
  a.vec_ok = rows_vec_ok(p, U, T);
  // c* over every verified row
  a.row_ids = w.row_ids;
  a.row_count = w.counts + 0;
  a.nrows = p->R * p->gamma;
  a.tiles_per_stage = L.gc.tiles_per_stage;
  a.nsplit = L.gc.nsplit;
  a.rec_stride = L.rec_c;
  a.dyn = 1;
  a.ps = w.c_s;
  e = launch_bias_pass(kModeCstar, bf16, a, s);
  if (e != hipSuccess) return hip_fail(e, "cstar pass");
  // residual draw at each request's first rejection: block records ...
  a.row_ids = w.resid_ids;
  a.row_count = w.counts + 1;
  a.nrows = p->R;
  a.tiles_per_stage = L.small_r ? 1 : L.gr.tiles_per_stage;
  a.nsplit = L.ns_r;
  a.rec_stride = L.ns_r;
  a.dyn = 0;
  a.ps = nullptr;
  a.cand = w.r_cand;
  a.cand_f = w.r_candf;
  a.wpos = w.r_wpos;
  e = launch_bias_pass(kModeResidual, bf16, a, s);
  if (e != hipSuccess) return hip_fail(e, "residual pass");
  // ... and the bonus draw's block records
  e = launch_bonus(bf16, p->R, p->gamma, p->V, p->seed, T, w, cstar, s);  // also finalizes c*
  if (e != hipSuccess) return hip_fail(e, "bonus pass");
  SelectArgs q = {};
  q.R = p->R;
  q.gamma = p->gamma;
  q.V = p->V;
  q.seed = p->seed;
  q.ntiles = a.ntiles;
  q.U = U;
  q.T = T;
  q.W1 = W1;
  q.W2p = W2p;
  q.anchors = anchors;
  q.tokens = tokens;
  q.lse_d = lse_d;
  q.lse_t = w.lse_t;
  q.out_tokens = out_token;
  q.row_ids = w.resid_ids;
  q.row_count = w.counts + 1;
  q.nsplit = L.ns_r;
  q.tiles_per_stage = L.small_r ? 1 : L.gr.tiles_per_stage;
  q.cand = w.r_cand;
  q.cand_f = w.r_candf;
  q.wpos = w.r_wpos;
  SelectArgs qb = q;
  qb.row_ids = w.bonus_ids;
  qb.row_count = w.counts + 2;
  qb.nsplit = L.ns_b;
  qb.tiles_per_stage = 1;
  qb.cand = w.b_cand;
  e = launch_select_final(bf16, q, qb, s);
  if (e != hipSuccess) return hip_fail(e, "residual / bonus select");
  return ok();
}

__attribute__((visibility("default"))) int dspark_confidence(
    const dspark_problem* p, int32_t H, const uint16_t* h, const float* w, const float* temps,
    const void* W1, const int32_t* anchors, const int32_t* tokens, float* c, void* stream) {
  if (int e = check_problem(p)) return e;
  if (H < 1 || H > 65536) return fail(DSPARK_ERR_SHAPE, "H=%d outside [1, 65536]", H);
  if (!h || !w || !temps || !W1 || !anchors || !tokens || !c)
    return fail(DSPARK_ERR_ARG, "confidence: tensor pointers must be non-NULL");
  hipError_t e = launch_confidence(p->dtype == DSPARK_BF16, p->R, p->gamma, p->V, H, h, w, temps,
                                   W1, anchors, tokens, c, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "confidence");
  return ok();
}

__attribute__((visibility("default"))) int dspark_check_inputs(
    const dspark_problem* p, const void* U, const void* T, const void* W1, const void* W2,
    const int32_t* anchors, const int32_t* tokens, const float* c, int64_t* counts, void* stream) {
  if (int e = check_problem(p)) return e;
  if (!counts) return fail(DSPARK_ERR_ARG, "check_inputs: counts must be non-NULL");
  const uintptr_t esz = p->dtype == DSPARK_BF16 ? 2 : 4;
  const void* logits[4] = {U, T, W1, W2};
  for (const void* q : logits)
    if ((uintptr_t)q % esz)
      return fail(DSPARK_ERR_ARG, "check_inputs: U, T, W1, W2 must be aligned to %d bytes", (int)esz);
  if ((uintptr_t)anchors % 4 || (uintptr_t)tokens % 4 || (uintptr_t)c % 4 || (uintptr_t)counts % 8)
    return fail(DSPARK_ERR_ARG, "check_inputs: misaligned anchors, tokens, c or counts");
  hipError_t e = launch_check_inputs(p->dtype == DSPARK_BF16, p->R, p->gamma, p->V, U, T, W1, W2,
                                     anchors, tokens, c, counts, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "check_inputs");
  return ok();
}

__attribute__((visibility("default"))) int dspark_schedule(int32_t R, int32_t gamma,
                                                           const float* c, const float* sps,
                                                           int32_t n_sps, float* a,
                                                           int32_t* lengths, double* stats,
                                                           double* theta_path, void* stream) {
  if (R < 1 || gamma < 1) return fail(DSPARK_ERR_SHAPE, "R=%d, gamma=%d must be >= 1", R, gamma);
  if ((int64_t)R * gamma > 16384)
    return fail(DSPARK_ERR_SHAPE, "R*gamma=%lld exceeds 16384", (long long)R * gamma);
  if ((int64_t)n_sps < (int64_t)R * (gamma + 1))
    return fail(DSPARK_ERR_RANGE, "SPS table has %d entries, R*(gamma+1)=%lld needed", n_sps,
                (long long)R * (gamma + 1));
  if (!c || !sps || !a || !lengths || !stats)
    return fail(DSPARK_ERR_ARG, "schedule: tensor pointers must be non-NULL");
  hipError_t e = launch_schedule(R, gamma, c, sps, a, lengths, stats, theta_path, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "schedule");
  return ok();
}

__attribute__((visibility("default"))) int dspark_schedule_capacity(
    int32_t R, int32_t gamma, const float* c, const float* sps, int32_t n_sps, float* a,
    int32_t* K, int32_t* lengths, double* stats, double* theta_path, void* stream) {
  if (R < 1 || gamma < 1) return fail(DSPARK_ERR_SHAPE, "R=%d, gamma=%d must be >= 1", R, gamma);
  if ((int64_t)R * gamma > 16384)
    return fail(DSPARK_ERR_SHAPE, "R*gamma=%lld exceeds 16384", (long long)R * gamma);
  if ((int64_t)n_sps < (int64_t)R * (gamma + 1))
    return fail(DSPARK_ERR_RANGE, "SPS table has %d entries, R*(gamma+1)=%lld needed", n_sps,
                (long long)R * (gamma + 1));
  if (!c || !sps || !a || !K || !lengths || !stats)
    return fail(DSPARK_ERR_ARG, "schedule_capacity: tensor pointers must be non-NULL");
  hipError_t e = launch_schedule_capacity(R, gamma, c, sps, a, K, lengths, stats, theta_path,
                                          (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "schedule_capacity");
  return ok();
}

__attribute__((visibility("default"))) int dspark_schedule_topk(int32_t R, int32_t gamma,
                                                                const float* c, const int32_t* K,
                                                                const float* sps, int32_t n_sps,
                                                                float* a, int32_t* lengths,
                                                                double* stats, void* stream) {
  if (R < 1 || gamma < 1) return fail(DSPARK_ERR_SHAPE, "R=%d, gamma=%d must be >= 1", R, gamma);
  if ((int64_t)R * gamma > 16384)
    return fail(DSPARK_ERR_SHAPE, "R*gamma=%lld exceeds 16384", (long long)R * gamma);
  if ((int64_t)n_sps < (int64_t)R * (gamma + 1))
    return fail(DSPARK_ERR_RANGE, "SPS table has %d entries, R*(gamma+1)=%lld needed", n_sps,
                (long long)R * (gamma + 1));
  if (!c || !K || !sps || !a || !lengths || !stats)
    return fail(DSPARK_ERR_ARG, "schedule_topk: tensor pointers must be non-NULL");
  hipError_t e = launch_schedule_topk(R, gamma, c, K, sps, a, lengths, stats, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "schedule_topk");
  return ok();
}

__attribute__((visibility("default"))) int dspark_schedule_threshold(int32_t R, int32_t gamma,
                                                                     const float* c, double theta,
                                                                     float* a, int32_t* lengths,
                                                                     void* stream) {
  if (R < 1 || R > 65536 || gamma < 1 || gamma > 64)
    return fail(DSPARK_ERR_SHAPE, "R=%d, gamma=%d outside [1, 65536] x [1, 64]", R, gamma);
  if (theta != theta) return fail(DSPARK_ERR_RANGE, "threshold is NaN");
  if (!c || !a || !lengths)
    return fail(DSPARK_ERR_ARG, "schedule_threshold: tensor pointers must be non-NULL");
  hipError_t e = launch_threshold(R, gamma, c, theta, a, lengths, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "schedule_threshold");
  return ok();
}

__attribute__((visibility("default"))) int dspark_acceptance_stats(
    int32_t R, int32_t gamma, const uint8_t* accept_mask, const float* a,
    const int32_t* n_accept, const double* thresholds, int32_t n_thr, int64_t* reached,
    int64_t* accepted, int64_t* sweep_verified, int64_t* sweep_accepted, void* stream) {
  if (R < 1 || R > 65536 || gamma < 1 || gamma > 64)
    return fail(DSPARK_ERR_SHAPE, "R=%d, gamma=%d outside [1, 65536] x [1, 64]", R, gamma);
  if (n_thr < 0 || n_thr > kMaxThresholds)
    return fail(DSPARK_ERR_SHAPE, "n_thr=%d outside [0, %d]", n_thr, kMaxThresholds);
  if (!accept_mask && n_thr == 0)
    return fail(DSPARK_ERR_ARG, "acceptance_stats: nothing to compute");
  if (accept_mask && (!reached || !accepted))
    return fail(DSPARK_ERR_ARG, "acceptance_stats: reached and accepted must be non-NULL");
  if (n_thr > 0 && (!a || !n_accept || !thresholds || !sweep_verified || !sweep_accepted))
    return fail(DSPARK_ERR_ARG, "acceptance_stats: sweep pointers must be non-NULL");
  hipError_t e = launch_acceptance_stats(R, gamma, accept_mask, a, n_accept, thresholds, n_thr,
                                         reached, accepted, sweep_verified, sweep_accepted,
                                         (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "acceptance_stats");
  return ok();
}

__attribute__((visibility("default"))) size_t dspark_sts_workspace_bytes(int32_t N, int32_t gamma,
                                                                        int32_t G, int32_t bins) {
  if (N < 1 || N > (1 << 20) || gamma < 1 || gamma > 64 || G < 1 || G > kStsMaxGrid || bins < 1 ||
      bins > kStsMaxBins)
    return 0;
  return sts_workspace_bytes(gamma, G, bins);
}

__attribute__((visibility("default"))) int dspark_sts_fit(int32_t N, int32_t gamma, const double* s,
                                                          const uint8_t* y, int32_t G,
                                                          const double* grid, int32_t bins,
                                                          float* temps, int64_t* ece_units,
                                                          int64_t* ece1_units, float* a, void* ws,
                                                          size_t ws_bytes, void* stream) {
  if (N < 1 || N > (1 << 20) || gamma < 1 || gamma > 64)
    return fail(DSPARK_ERR_SHAPE, "N=%d, gamma=%d outside [1, 2^20] x [1, 64]", N, gamma);
  if (G < 1 || G > kStsMaxGrid || bins < 1 || bins > kStsMaxBins)
    return fail(DSPARK_ERR_SHAPE, "G=%d, bins=%d outside [1, %d] x [1, %d]", G, bins, kStsMaxGrid,
                kStsMaxBins);
  if (!s || !y || !grid || !temps || !ece_units || !ece1_units || !a)
    return fail(DSPARK_ERR_ARG, "sts_fit: tensor pointers must be non-NULL");
  const size_t need = sts_workspace_bytes(gamma, G, bins);
  if (!ws) return fail(DSPARK_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if ((uintptr_t)ws % kAlign) return fail(DSPARK_ERR_WORKSPACE, "workspace not %zu-byte aligned", kAlign);
  if (ws_bytes < need)
    return fail(DSPARK_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  hipError_t e = launch_sts_fit(N, gamma, s, y, G, grid, bins, temps, ece_units, ece1_units, a, ws,
                                (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sts_fit");
  return ok();
}

}  // extern "C"
