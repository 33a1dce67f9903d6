// libmtp C ABI: host-side validation (fail closed before any enqueue), the
// workspace layout, and the kernel sequences of the draft-head step, the
// pending-pair flush, verification and rollback.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/mtp.h"
#include "kernels.h"

using namespace mtp;

namespace {
thread_local hipError_t g_last_hip = hipSuccess;

// Event pairs bracketing the launches of one kernel class while timing is on
// (benchmarks).
struct KernelTimer {
  std::mutex mu;
  std::vector<hipEvent_t> start, stop;
  int used = 0;
  int kind = -1;
  bool on = false;
  bool paused = false;
} g_timer;
}  // namespace

void mtp::time_mark(int kind, bool before, hipStream_t s, int* slot) {
  std::lock_guard<std::mutex> lk(g_timer.mu);
  if (!g_timer.on || g_timer.kind != kind) { *slot = -1; return; }
  if (before) {
    if (g_timer.paused) { *slot = -1; return; }
    if (g_timer.used >= static_cast<int>(g_timer.start.size())) { *slot = -1; return; }
    *slot = g_timer.used++;
    hipEventRecord(g_timer.start[*slot], s);
  } else if (*slot >= 0) {
    hipEventRecord(g_timer.stop[*slot], s);
  }
}

namespace {
}  // namespace

#define MTP_TRY(expr)                  \
  do {                                 \
    const hipError_t e_ = (expr);      \
    if (e_ != hipSuccess) {            \
      g_last_hip = e_;                 \
      return MTP_E_HIP;                \
    }                                  \
  } while (0)

struct mtp_head {
  mtp_head_config cfg;
  mtp_head_weights w;
  int wt;   // weight type of projections / norms / embedding
  int lmt;  // lm_head type
};

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kHeadBytes = 256;   // reserved at offset 0
constexpr int kVerifyChunk = 4096;   // logits per verify workgroup
constexpr int kFlushWgs = 512;       // flush attention workgroups (about two per compute unit)

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int epc_of(int t) { return t == W_F32 ? 4 : (t == W_BF16 ? 8 : 16); }

int lpr_for(int K, int t) {
  const int nch = K / epc_of(t);
  int l = 64;
  while (l > 8 && nch % l) l >>= 1;
  return (nch % l == 0 && nch >= l) ? l : 0;
}

// The unembedding streams many short rows, one row block after another.  With
// int8 rows a lane covering at least 16 chunks keeps a block's loads in full
// batches instead of one batch and a one-chunk tail that waits a whole memory
// round trip by itself (H 5120: 320 chunks, 16 lanes of 20 rather than 64 of
// 5; measured 145 -> 133 us, with 32 lanes of 10 137 us).  bf16 rows keep 64
// lanes (10 chunks each; 32 lanes of 20 measured slower).
int lpr_unembed(int K, int t) {
  int l = lpr_for(K, t);
  if (t != W_I8) return l;
  const int nch = K / epc_of(t);
  while (l > 8 && nch / l < 16 && nch % (l / 2) == 0) l >>= 1;
  return l;
}

int nr_for(int rows) {
  if (rows <= 4) return rows < 1 ? 1 : rows;
  return rows <= 8 ? 8 : 16;
}

int kp_for(int K, int t, int nr) {
  // staged inputs in LDS: 128 KB of fp32, or 144 KB of bf16 for few-row passes
  // with bf16 weights (four rows of 17408, the 27B-shaped down projection's
  // input, in one phase)
  const int budget = (nr > 1 && t == W_BF16 ? 73728 : 32768) / nr;
  if (K <= budget) return K;
  const int q = lpr_for(K, t) * epc_of(t);
  int kp = budget / q * q;
  return kp > 0 ? kp : q;
}

// Key chunks per (row, kv head): about 256 attention workgroups per query row,
// at least 32 keys per chunk.
int nchunk_for(const mtp_head_config& c, int capacity) {
  int target = (256 + c.n_kv_heads - 1) / c.n_kv_heads;
  const int fine = (capacity + 31) / 32;
  if (target > fine) target = fine;
  return target < 1 ? 1 : target;
}

struct Layout {
  size_t x, qkv, qr, part_o, part_ml, o, x1, m, g, amax, xa, gpart, uxa, ulog, lo, lx, lb, total;
  int nchunk;
};

// Flushes of more rows than gemv_max_rows go through the MFMA tiles.  Small
// heads keep the GEMV passes up to 16 rows (one launch per projection; every
// kernel there is latency-bound).  Large heads switch past one row: the
// weight-streaming MFMA product reads each weight once with coalesced loads
// for any row count, while the few-row GEMV passes stage every row per
// workgroup and run at fewer waves per SIMD (27B shape, fc + q/k/v of a flush:
// 3 rows 94 us as GEMV passes, 5 rows 67 us as products).
constexpr int kGemvMaxRows = 16;
constexpr int kGemvMaxRowsLarge = 1;
constexpr int kLargeHidden = 2048;

int gemv_max_rows(const mtp_head_config& c) {
  return c.hidden >= kLargeHidden ? kGemvMaxRowsLarge : kGemvMaxRows;
}

// Three sessions and more: their unembedding runs as one matrix-core product
// over the sessions' normalised last rows (the lm_head streamed once for every
// session) instead of few-row GEMV launches (27B shape, rounds of B sessions:
// B=2 4397 vs 4311 draft tokens/s for the GEMV, B=3 5957 vs 6057, B=4 7460 vs
// 7867).  bf16 lm_head.
constexpr int kUnembedProductSlots = 3;
bool unembed_product(const mtp_head_config& c, int slots) {
  const int mv[1] = {c.vocab};
  return slots >= kUnembedProductSlots && c.lm_head_dtype == MTP_BF16 && gemm_supported(c.vocab, c.hidden, mv, 1);
}

// With the unembedding as a product (bf16 weights too), o_proj and the MLP run
// as products over the sessions' gathered last rows as well: each weight
// streamed once for every session rather than once per launch of four.
bool last_rows_product(const mtp_head_config& c, int slots) {
  if (!unembed_product(c, slots) || c.weight_dtype != MTP_BF16) return false;
  const int H = c.hidden, I = c.intermediate;
  const int mh[1] = {H}, mi[1] = {I};
  return gemm_supported(H, c.n_q_heads * c.head_dim, mh, 1) && gemm_supported(I, H, mi, 1) &&
         gemm_supported(H, I, mh, 1);
}

// upper bound on the unembedding GEMV's workgroup count (one argmax key each)
size_t amax_parts(const mtp_head_config& c) { return static_cast<size_t>(c.vocab) / 4 + 2048; }

// rows: workspace rows (every session's rows, flattened); slots: unembedding
// rows of one launch (one per session), each with its own argmax keys
Layout layout(const mtp_head_config& c, int rows, int capacity, int slots = 1) {
  Layout L{};
  const size_t H = c.hidden, D = c.head_dim, hq = c.n_q_heads, hkv = c.n_kv_heads, I = c.intermediate;
  L.nchunk = nchunk_for(c, capacity);
  size_t off = kHeadBytes;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  L.x = take(rows * H * 4);
  L.qkv = take(rows * (hq + 2 * hkv) * D * 4);
  L.qr = take(rows * hq * D * 4);
  L.part_o = take(rows * hq * L.nchunk * D * 4);
  L.part_ml = take(rows * hq * L.nchunk * 2 * 4);
  L.o = take(rows * hq * D * 4);
  L.x1 = take(rows * H * 4);
  L.m = take(rows * I * 4);
  L.g = take(rows * H * 4);
  L.amax = take(static_cast<size_t>(slots) * amax_parts(c) * 8);
  const bool mfma_rows = rows > gemv_max_rows(c);
  L.xa = mfma_rows ? take(rows * 2 * H * 2) : off;             // bf16 normalised rows (MFMA path)
  size_t part = 0;                                             // split partial sums (MFMA path)
  if (mfma_rows) {
    const int mq[3] = {static_cast<int>(hq * D), static_cast<int>(hkv * D), static_cast<int>(hkv * D)};
    const int mh[1] = {static_cast<int>(H)};
    const int mi[2] = {static_cast<int>(I), static_cast<int>(I)};
    const int qkv_rows = static_cast<int>((hq + 2 * hkv) * D);
    part = std::max({gemm_part_floats(rows, H, 2 * H, mh, 1, false),
                     gemm_part_floats(rows, qkv_rows, H, mq, 3, false),
                     gemm_part_floats(rows, H, hq * D, mh, 1, false),
                     gemm_part_floats(rows, I, H, mi, 2, true),
                     gemm_part_floats(rows, H, I, mh, 1, false)});
  }
  const bool up = unembed_product(c, slots);
  if (up) {
    const int mv[1] = {c.vocab};
    part = std::max(part, gemm_part_floats(slots, c.vocab, static_cast<int>(H), mv, 1, false));
  }
  const bool lp = last_rows_product(c, slots);
  if (lp) {
    const int mh[1] = {static_cast<int>(H)};
    const int mi[2] = {static_cast<int>(I), static_cast<int>(I)};
    part = std::max({part, gemm_part_floats(slots, H, hq * D, mh, 1, false),
                     gemm_part_floats(slots, I, H, mi, 2, true), gemm_part_floats(slots, H, I, mh, 1, false)});
  }
  L.gpart = part ? take(part * 4) : off;
  L.uxa = up ? take(static_cast<size_t>(slots) * H * 2) : off;             // normalised last rows, bf16
  L.ulog = up ? take(static_cast<size_t>(slots) * c.vocab * 4) : off;      // their logits
  L.lo = lp ? take(static_cast<size_t>(slots) * hq * D * 2) : off;         // gathered o rows, bf16
  L.lx = lp ? take(static_cast<size_t>(slots) * H * 4) : off;              // gathered x rows
  L.lb = lp ? take(static_cast<size_t>(slots) * H * 2) : off;              // MLP input rows, bf16
  L.total = off;
  return L;
}

bool dtype_ok(int t, bool allow_i8) { return t == MTP_F32 || t == MTP_BF16 || (allow_i8 && t == MTP_I8G128); }

int validate_cfg(const mtp_head_config* c) {
  if (!c) return MTP_E_INVALID_ARG;
  if (c->hidden <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      c->intermediate <= 0 || c->vocab <= 0)
    return MTP_E_INVALID_ARG;
  if (!(c->rms_eps >= 0.f) || !std::isfinite(c->rms_eps) || !(c->rope_theta > 0.f) ||
      !std::isfinite(c->rope_theta))
    return MTP_E_INVALID_ARG;
  if (!dtype_ok(c->weight_dtype, false) || !dtype_ok(c->act_dtype, false) ||
      !dtype_ok(c->kv_dtype, false) || !dtype_ok(c->lm_head_dtype, true))
    return MTP_E_INVALID_ARG;
  if (c->hidden % 64 || c->intermediate % 64) return MTP_E_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256) return MTP_E_UNSUPPORTED;
  if (c->n_q_heads % c->n_kv_heads) return MTP_E_UNSUPPORTED;
  const int g = c->n_q_heads / c->n_kv_heads;
  if (g != 1 && g != 2 && g != 3 && g != 4 && g != 6 && g != 8) return MTP_E_UNSUPPORTED;
  if (c->lm_head_dtype == MTP_I8G128 && c->hidden % 128) return MTP_E_UNSUPPORTED;
  if (static_cast<long long>(c->vocab) * c->hidden >= (1ll << 40)) return MTP_E_UNSUPPORTED;
  return MTP_OK;
}

int validate_kv(const mtp_head* h, const mtp_kv* kv) {
  if (!kv || !kv->k || !kv->v || !kv->state || kv->capacity <= 0) return MTP_E_INVALID_ARG;
  if (kv->capacity > (1 << 20)) return MTP_E_UNSUPPORTED;
  (void)h;
  return MTP_OK;
}

inline char* wsp(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

// Independent sessions in one call; batch 1 is the single-session path.  With
// batch > 1 session b's K/V start b * kv_sb elements in and its state words at
// state + 4 b; its pending token j is tokens[b * tok_sb + j], its hidden row
// b * hid_sb + j and its count n_dev[b * ndev_sb]; its outputs (hidden, logits,
// argmax) go to row b * out_sb of each output.  Workspace rows are flattened
// b * n_max + j.
struct Sessions {
  int batch = 1;
  int tok_sb = 0, hid_sb = 0, out_sb = 0, ndev_sb = 0;
  long long kv_sb = 0;
  bool multi() const { return batch > 1; }
};
const Sessions kOneSession{};

// unembedding rows per launch (one per session; the GEMV row counts are 1, 2, 3, 4, 8, 16)
int slots_of(const Sessions& ss) { return ss.multi() ? nr_for(ss.batch) : 1; }
// Past four sessions the one-row-per-session GEMVs (the unembedding, and o_proj
// and the MLP after a LAST-mode flush) run as launches of four sessions each:
// the few-row GEMV's staged-input reads from LDS grow with its row count and
// bound it past four rows (the 27B unembedding: 8 rows 752 us against 2 x 289
// us for two launches of four; 16 rows 5.5 ms against 4 x 289 us).
constexpr int kLastRowGroup = 4;
int last_row_nr(int slots) { return slots > kLastRowGroup ? kLastRowGroup : slots; }

GemvArgs base_gemv(const mtp_head* h, const mtp_kv* kv, const Sessions& ss = kOneSession) {
  GemvArgs a;
  std::memset(&a, 0, sizeof(a));
  a.nw_bf16 = h->wt == W_BF16;
  a.eps = h->cfg.rms_eps;
  a.kv_state = kv->state;
  a.batch = ss.batch;
  a.tok_sb = ss.tok_sb; a.hid_sb = ss.hid_sb; a.out_sb = ss.out_sb; a.ndev_sb = ss.ndev_sb;
  return a;
}

// One GEMV launch, bracketed for the benchmark timer when `kind` >= 0.
hipError_t timed_gemv(const GemvArgs& a, int wt, int nr, hipStream_t s, int* grid_out, int kind) {
  int slot = -1;
  if (kind >= 0) time_mark(kind, true, s, &slot);
  const hipError_t e = launch_gemv(a, wt, nr, s, grid_out);
  if (kind >= 0) time_mark(kind, false, s, &slot);
  return e;
}

hipError_t run_gemv(GemvArgs a, int wt, int rows_total, int row_sel, hipStream_t s,
                    int* grid_out = nullptr, int kind = TIME_PROJECTION) {
  // ROWS_RANGE: blocks of up to 16 activation rows share one pass over the weights
  // ROW_LAST: the last row of each session (one slot per session)
  a.row_sel = row_sel;
  if (row_sel == ROW_LAST) {
    const int nr = last_row_nr(a.batch > 1 ? nr_for(a.batch) : 1);
    a.kp = kp_for(a.K, wt, nr);
    a.grid_stride = a.kp == a.K;
    for (int b = 0; b < (a.batch > 1 ? a.batch : 1); b += nr) {   // sessions b .. b + nr - 1
      a.row_base = b;
      hipError_t e = timed_gemv(a, wt, nr, s, b == 0 ? grid_out : nullptr, kind);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const int nr = nr_for(rows_total);
  a.kp = kp_for(a.K, wt, nr);
  a.grid_stride = a.kp == a.K;
  for (int b = 0; b < rows_total; b += nr) {
    a.row_base = b;
    hipError_t e = timed_gemv(a, wt, nr, s, nullptr, kind);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t timed_gemm(const GemmArgs& g, hipStream_t s, const RowNorm* rn = nullptr, bool* normed = nullptr,
                      int* split_left = nullptr) {
  int slot = -1;
  time_mark(TIME_PROJECTION, true, s, &slot);
  const hipError_t e = launch_gemm(g, s, rn, normed, split_left);
  time_mark(TIME_PROJECTION, false, s, &slot);
  return e;
}

// Several sessions: the products run over every flattened row (rows past a
// session's count were prepared as zeros and are never read back).
GemmArgs base_gemm(const mtp_kv* kv, int n_max, const int32_t* n_dev, float* part,
                   const Sessions& ss = kOneSession) {
  GemmArgs g;
  std::memset(&g, 0, sizeof(g));
  g.n_max = ss.multi() ? ss.batch * n_max : n_max;
  g.n_dev = ss.multi() ? nullptr : n_dev;
  g.kv_state = ss.multi() ? nullptr : kv->state;
  g.part = part;
  return g;
}

PrepArgs base_prep(const mtp_head* h, const mtp_kv* kv, int n_max, const int32_t* n_dev, uint16_t* out,
                   const Sessions& ss = kOneSession) {
  PrepArgs p;
  std::memset(&p, 0, sizeof(p));
  p.n_max = n_max;
  p.n_dev = n_dev;
  p.kv_state = kv->state;
  p.nw_bf16 = h->wt == W_BF16;
  p.eps = h->cfg.rms_eps;
  p.out = out;
  p.batch = ss.batch;
  p.tok_sb = ss.tok_sb; p.hid_sb = ss.hid_sb; p.ndev_sb = ss.ndev_sb;
  return p;
}

// The unembedding launch: logits = W_lm RMSNorm(g; w_norm) of the last row with
// the per-workgroup argmax keys.
GemvArgs unembed_args(const mtp_head* h, const mtp_kv* kv, const Layout& L, int n_max, const int32_t* n_dev,
                      const float* g, float* logits, void* ws, const Sessions& ss = kOneSession) {
  const mtp_head_config& c = h->cfg;
  GemvArgs a = base_gemv(h, kv, ss);
  a.w[0] = h->w.lm_head; a.m[0] = c.vocab; a.M = c.vocab; a.K = c.hidden; a.lpr = lpr_unembed(c.hidden, h->lmt);
  a.scales = static_cast<const uint16_t*>(h->w.lm_head_scales);
  a.n_max = n_max; a.n_dev = n_dev;
  a.in_mode = IN_RMS; a.x = g; a.ldx = c.hidden; a.nw = h->w.norm;
  a.out_mode = OUT_LOGITS; a.logits = logits;
  a.amax_part = reinterpret_cast<unsigned long long*>(wsp(ws, L.amax));
  a.row_sel = ROW_LAST;
  a.row_base = 0;
  a.kp = kp_for(a.K, h->lmt, last_row_nr(slots_of(ss)));   // rows per launch (launches of four past four)
  a.grid_stride = a.kp == a.K;
  return a;
}

// The head forward for n rows (n_max host bound, n_dev device count; a device
// count below n_min sets MTP_DEV_COUNT).  mode: KV_ONLY / LAST / ALL.
// hidden_out: [1 or n, H] in act dtype (nullable).
// fold_in (nullable): the previous step's argmax merge and append commit, run
// by this call's fc pass when that pass is a one-row GEMV, else launched first.
// defer_out (nullable): this call's own merge is returned instead of launched,
// for a following call to fold (the argmax keys it reads sit in the workspace
// after the rows a one-row call writes before its fc pass ends).
int head_forward(const mtp_head* h, const mtp_kv* kv, const int32_t* tokens, const void* hiddens,
                 int n_max, const int32_t* n_dev, int mode, int set_base, void* hidden_out,
                 float* logits, int32_t* argmax, void* ws, hipStream_t s, int n_min = 0,
                 const Sessions& ss = kOneSession, const FinishArgs* fold_in = nullptr,
                 FinishArgs* defer_out = nullptr) {
  const mtp_head_config& c = h->cfg;
  // a folded merge not yet enqueued when this call returns (an error before its
  // fc pass) is launched on the way out, so the previous step still commits
  struct FoldGuard {
    const FinishArgs* f;
    hipStream_t s;
    ~FoldGuard() {
      if (f) (void)launch_finish(*f, s);
    }
  } guard{fold_in && fold_in->state ? fold_in : nullptr, s};
  const int rows_total = ss.multi() ? ss.batch * n_max : n_max;   // workspace rows
  const int slots = slots_of(ss);
  const Layout L = layout(c, rows_total, kv->capacity, slots);
  if (ss.multi() && mode != MTP_FLUSH_LAST) return MTP_E_UNSUPPORTED;
  // host-checkable limits before anything is enqueued: the unembedding's
  // workgroups each write one argmax key per slot into a buffer of amax_parts
  // entries per slot
  if (mode != MTP_FLUSH_KV_ONLY) {
    GemvArgs u = unembed_args(h, kv, L, n_max, n_dev, nullptr, nullptr, ws, ss);
    u.dry_run = 1;
    int grid = 0;
    MTP_TRY(launch_gemv(u, h->lmt, last_row_nr(slots), s, &grid));
    if (grid < 1 || static_cast<size_t>(grid) > amax_parts(c)) return MTP_E_UNSUPPORTED;
  }
  const int H = c.hidden, D = c.head_dim, hq = c.n_q_heads, hkv = c.n_kv_heads, I = c.intermediate;
  const int qkv_rows = (hq + 2 * hkv) * D;
  float* x = reinterpret_cast<float*>(wsp(ws, L.x));
  float* qkv = reinterpret_cast<float*>(wsp(ws, L.qkv));
  float* qr = reinterpret_cast<float*>(wsp(ws, L.qr));
  float* o = reinterpret_cast<float*>(wsp(ws, L.o));
  float* x1 = reinterpret_cast<float*>(wsp(ws, L.x1));
  float* m = reinterpret_cast<float*>(wsp(ws, L.m));
  float* g = reinterpret_cast<float*>(wsp(ws, L.g));
  uint16_t* xa = reinterpret_cast<uint16_t*>(wsp(ws, L.xa));
  float* gpart = reinterpret_cast<float*>(wsp(ws, L.gpart));
  // many rows with bf16 weights: normalised rows + MFMA tiles instead of GEMV passes
  const bool mfma = h->wt == W_BF16 && rows_total > gemv_max_rows(c);
  if (mfma) {
    const int mq[3] = {hq * D, hkv * D, hkv * D};
    const int mh[1] = {H};
    const int mi[1] = {I};
    if (!gemm_supported(H, 2 * H, mh, 1) || !gemm_supported(qkv_rows, H, mq, 3) ||
        !gemm_supported(H, hq * D, mh, 1) || !gemm_supported(I, H, mi, 1) || !gemm_supported(H, I, mh, 1))
      return MTP_E_UNSUPPORTED;
  }
  // 1. x = W_fc [RMSNorm(E[t]) | RMSNorm(h)]
  bool normed_qkv = false, normed_mlp = false, normed_g = false;
  const bool have_fold = fold_in && fold_in->state;
  const bool fold = have_fold && fold_in->parts && !mfma && !ss.multi() && rows_total == 1;
  if (have_fold && !fold) {
    guard.f = nullptr;
    MTP_TRY(launch_finish(*fold_in, s));
  }
  if (mfma) {
    PrepArgs p = base_prep(h, kv, n_max, n_dev, xa, ss);
    p.in_mode = IN_EMBED; p.K = 2 * H; p.ld_out = 2 * H;
    p.nw = h->w.pre_fc_norm_embedding; p.nw2 = h->w.pre_fc_norm_hidden;
    p.tok = tokens; p.vocab_tok = c.vocab; p.err = kv->state + 3;
    p.embed = h->w.embed; p.embed_bf16 = 1;
    p.hid = hiddens; p.hid_bf16 = c.act_dtype == MTP_BF16; p.ld_hid = H;
    MTP_TRY(launch_rows_prep(p, s));
    GemmArgs m1 = base_gemm(kv, n_max, n_dev, gpart, ss);
    m1.w[0] = static_cast<const uint16_t*>(h->w.fc); m1.m[0] = H; m1.M = H; m1.K = 2 * H;
    m1.a = xa; m1.lda = 2 * H; m1.out_mode = OUT_F32; m1.y = x; m1.ldy = H;
    // a split-K reduce also writes the q/k/v input rows, RMSNorm(x; w_in)
    const RowNorm rn{h->w.input_layernorm, h->wt == W_BF16, c.rms_eps, xa, H};
    MTP_TRY(timed_gemm(m1, s, &rn, &normed_qkv));
  }
  GemvArgs a = base_gemv(h, kv, ss);
  a.w[0] = h->w.fc; a.m[0] = H; a.M = H; a.K = 2 * H; a.lpr = lpr_for(2 * H, h->wt);
  a.n_max = n_max; a.n_dev = n_dev;
  a.in_mode = IN_EMBED; a.nw = h->w.pre_fc_norm_embedding; a.nw2 = h->w.pre_fc_norm_hidden;
  a.tok = tokens; a.vocab_tok = c.vocab; a.err = kv->state + 3;
  a.embed = h->w.embed; a.embed_bf16 = h->wt == W_BF16;
  a.hid = hiddens; a.hid_bf16 = c.act_dtype == MTP_BF16; a.ld_hid = H;
  a.out_mode = OUT_F32; a.y = x; a.ldy = H;
  if (fold) {
    a.fin_parts = fold_in->parts; a.fin_nparts = fold_in->nparts; a.fin_amax = fold_in->amax_out;
    a.fin_ndev = fold_in->n_dev; a.fin_nmax = fold_in->n_max; a.fin_set_base = fold_in->set_base;
    a.fin_state = fold_in->state;
    guard.f = nullptr;   // the fc pass below carries it
  }
  if (!mfma) MTP_TRY(run_gemv(a, h->wt, rows_total, ROWS_RANGE, s));

  // LAST mode: the norm/RoPE/append runs inside the attention kernel, which
  // also sums the q/k/v product's split-K partials
  const bool fuse_rope = mode == MTP_FLUSH_LAST;
  int qkv_split = 1;

  // 2. q, k, v = W_{q,k,v} RMSNorm(x; w_in)
  if (mfma) {
    if (!normed_qkv) {
      PrepArgs p = base_prep(h, kv, n_max, n_dev, xa, ss);
      p.in_mode = IN_RMS; p.K = H; p.ld_out = H; p.x = x; p.ldx = H; p.nw = h->w.input_layernorm;
      MTP_TRY(launch_rows_prep(p, s));
    }
    GemmArgs m2 = base_gemm(kv, n_max, n_dev, gpart, ss);
    m2.w[0] = static_cast<const uint16_t*>(h->w.q_proj); m2.m[0] = hq * D;
    m2.w[1] = static_cast<const uint16_t*>(h->w.k_proj); m2.m[1] = hkv * D;
    m2.w[2] = static_cast<const uint16_t*>(h->w.v_proj); m2.m[2] = hkv * D;
    m2.M = qkv_rows; m2.K = H; m2.a = xa; m2.lda = H; m2.out_mode = OUT_F32; m2.y = qkv; m2.ldy = qkv_rows;
    // the attention's split sums take 32-bit offsets into the partials
    const bool defer = fuse_rope && D >= kSplitMinHeadDim &&
                       gemm_part_floats(rows_total, qkv_rows, H, m2.m, 3, false) * 4 < (size_t{1} << 31);
    MTP_TRY(timed_gemm(m2, s, nullptr, nullptr, defer ? &qkv_split : nullptr));
  }
  a = base_gemv(h, kv, ss);
  a.w[0] = h->w.q_proj; a.m[0] = hq * D;
  a.w[1] = h->w.k_proj; a.m[1] = hkv * D;
  a.w[2] = h->w.v_proj; a.m[2] = hkv * D;
  a.M = qkv_rows; a.K = H; a.lpr = lpr_for(H, h->wt);
  a.n_max = n_max; a.n_dev = n_dev;
  a.in_mode = IN_RMS; a.x = x; a.ldx = H; a.nw = h->w.input_layernorm;
  a.out_mode = OUT_F32; a.y = qkv; a.ldy = qkv_rows;
  if (!mfma) MTP_TRY(run_gemv(a, h->wt, rows_total, ROWS_RANGE, s));

  // 3. q/k norm + RoPE, append K/V at slots len + j, advance len
  RopeArgs r;
  std::memset(&r, 0, sizeof(r));
  r.qkv = qkv; r.ld_qkv = qkv_rows; r.q_out = qr;
  r.q_norm = h->w.q_norm; r.k_norm = h->w.k_norm; r.nw_bf16 = h->wt == W_BF16;
  r.eps = c.rms_eps; r.theta = c.rope_theta; r.hq = hq; r.hkv = hkv; r.d = D;
  r.kc = kv->k; r.vc = kv->v; r.kv_bf16 = c.kv_dtype == MTP_BF16; r.capacity = kv->capacity;
  r.state = kv->state; r.n_max = n_max; r.n_dev = n_dev; r.n_min = n_min;
  if (!fuse_rope) MTP_TRY(launch_rope_append(r, s));
  FinishArgs f;
  std::memset(&f, 0, sizeof(f));
  f.state = kv->state; f.n_max = n_max; f.n_dev = n_dev; f.set_base = set_base;
  f.batch = ss.batch; f.out_sb = ss.out_sb; f.ndev_sb = ss.ndev_sb;
  if (mode == MTP_FLUSH_KV_ONLY) {
    if (defer_out) std::memset(defer_out, 0, sizeof(*defer_out));   // nothing left to fold
    MTP_TRY(launch_finish(f, s));
    return MTP_OK;
  }

  const int rsel = (mode == MTP_FLUSH_ALL) ? ROWS_RANGE : ROW_LAST;
  const bool mfma_out = mfma && rsel == ROWS_RANGE;   // o, MLP over every row
  // several sessions' last rows: o, the MLP and the unembedding as products
  // over the gathered rows [batch, .] (outputs kept compact until the hidden copy)
  const bool lprod = ss.multi() && rsel == ROW_LAST && last_rows_product(c, slots);
  LastRowsArgs gr;
  std::memset(&gr, 0, sizeof(gr));
  gr.n_max = n_max; gr.n_dev = n_dev; gr.ndev_sb = ss.ndev_sb; gr.state = kv->state; gr.batch = ss.batch;
  gr.nw_bf16 = h->wt == W_BF16; gr.eps = c.rms_eps; gr.rows = ss.batch;
  auto last_gemm = [&](const void* a_rows, int lda) {
    GemmArgs g;
    std::memset(&g, 0, sizeof(g));
    g.n_max = ss.batch; g.part = gpart; g.a = a_rows; g.lda = lda;
    return g;
  };
  uint16_t* lo = reinterpret_cast<uint16_t*>(wsp(ws, L.lo));
  float* lx = reinterpret_cast<float*>(wsp(ws, L.lx));
  uint16_t* lb = reinterpret_cast<uint16_t*>(wsp(ws, L.lb));

  // 4. attention over the draft KV
  AttnArgs t;
  std::memset(&t, 0, sizeof(t));
  t.q = qr; t.kc = kv->k; t.vc = kv->v; t.kv_bf16 = c.kv_dtype == MTP_BF16; t.capacity = kv->capacity;
  t.state = kv->state; t.hq = hq; t.hkv = hkv; t.d = D; t.n_max = n_max; t.n_dev = n_dev; t.n_min = n_min;
  t.row_sel = rsel; t.nchunk = L.nchunk;
  // several sessions' last rows: about the same ~256 workgroups in all (a
  // decode-attention workgroup fills its CU's wave slots, so more would queue)
  if (ss.multi() && rsel == ROW_LAST) t.nchunk = (L.nchunk + ss.batch - 1) / ss.batch;
  t.batch = ss.batch; t.kv_sb = ss.kv_sb; t.ndev_sb = ss.ndev_sb;
  if (fuse_rope) {
    t.fuse_rope = 1; t.qkv = qkv; t.ld_qkv = qkv_rows; t.q_norm = h->w.q_norm; t.k_norm = h->w.k_norm;
    t.qkv_nsp = qkv_split;
    if (qkv_split > 1) {   // partials [split, n_max, qkv_rows]
      t.qkv = gpart;
      t.qkv_pstride = rows_total * qkv_rows;   // every session's rows, b * n_max + j
    }
    t.nw_bf16 = h->wt == W_BF16; t.eps = c.rms_eps; t.theta = c.rope_theta;
  }
  if (mfma_out && c.kv_dtype == MTP_BF16) {
    // matrix-core flush attention: workgroups of 64 query vectors over
    // kFlushWgs workgroups in all (key chunks of at least one block each)
    const int qblocks = (n_max * (hq / hkv) + 63) / 64;
    int ns = kFlushWgs / (qblocks * hkv);
    ns = ns > kFlushMaxChunks ? kFlushMaxChunks : ns;
    t.mfma = 1;
    t.nchunk = ns < 1 ? 1 : (ns > L.nchunk ? L.nchunk : ns);
  }
  t.part_o = reinterpret_cast<float*>(wsp(ws, L.part_o));
  t.part_ml = reinterpret_cast<float*>(wsp(ws, L.part_ml));
  t.o = o;
  t.o_bf16 = mfma_out;   // the many-row o product reads bf16 rows
  if (lprod) {           // the o product's rows, gathered by the merge
    t.o = reinterpret_cast<float*>(lo); t.o_bf16 = 1; t.o_compact = 1;
    t.xg = x; t.xg_out = lx; t.ld_xg = H;
  }
  MTP_TRY(launch_attention(t, s));

  // 5. x1 = x + W_o o
  a = base_gemv(h, kv, ss);
  a.w[0] = h->w.o_proj; a.m[0] = H; a.M = H; a.K = hq * D; a.lpr = lpr_for(hq * D, h->wt);
  a.n_max = n_max; a.n_dev = n_dev;
  a.in_mode = IN_F32; a.x = o; a.ldx = hq * D;
  a.out_mode = OUT_RESID; a.res = x; a.ldres = H; a.y = x1; a.ldy = H;
  if (mfma_out) {
    GemmArgs m5 = base_gemm(kv, n_max, n_dev, gpart, ss);
    m5.w[0] = static_cast<const uint16_t*>(h->w.o_proj); m5.m[0] = H; m5.M = H; m5.K = hq * D;
    m5.a = o; m5.lda = hq * D;
    m5.out_mode = OUT_RESID; m5.res = x; m5.ldres = H; m5.y = x1; m5.ldy = H;
    // a split-K reduce also writes the MLP input rows, RMSNorm(x1; w_post)
    const RowNorm rn{h->w.post_attention_layernorm, h->wt == W_BF16, c.rms_eps, xa, H};
    MTP_TRY(timed_gemm(m5, s, &rn, &normed_mlp));
  } else if (lprod) {
    GemmArgs m5 = last_gemm(lo, hq * D);
    m5.w[0] = static_cast<const uint16_t*>(h->w.o_proj); m5.m[0] = H; m5.M = H; m5.K = hq * D;
    m5.out_mode = OUT_RESID; m5.res = lx; m5.ldres = H; m5.y = x1; m5.ldy = H;
    const RowNorm rn{h->w.post_attention_layernorm, h->wt == W_BF16, c.rms_eps, lb, H};
    MTP_TRY(timed_gemm(m5, s, &rn, &normed_mlp));
  } else {
    MTP_TRY(run_gemv(a, h->wt, rows_total, rsel, s));
  }

  // 6. m = silu(W_g b) * (W_u b), b = RMSNorm(x1; w_post)
  a = base_gemv(h, kv, ss);
  a.w[0] = h->w.gate_proj; a.m[0] = I; a.w[1] = h->w.up_proj; a.m[1] = I;
  a.M = I; a.K = H; a.lpr = lpr_for(H, h->wt);
  a.n_max = n_max; a.n_dev = n_dev;
  a.in_mode = IN_RMS; a.x = x1; a.ldx = H; a.nw = h->w.post_attention_layernorm;
  a.out_mode = OUT_SWIGLU; a.y = m; a.ldy = I;
  if (mfma_out) {
    if (!normed_mlp) {
      PrepArgs p = base_prep(h, kv, n_max, n_dev, xa, ss);
      p.in_mode = IN_RMS; p.K = H; p.ld_out = H; p.x = x1; p.ldx = H; p.nw = h->w.post_attention_layernorm;
      MTP_TRY(launch_rows_prep(p, s));
    }
    GemmArgs m6 = base_gemm(kv, n_max, n_dev, gpart, ss);
    m6.w[0] = static_cast<const uint16_t*>(h->w.gate_proj); m6.m[0] = I;
    m6.w[1] = static_cast<const uint16_t*>(h->w.up_proj); m6.m[1] = I;
    m6.M = I; m6.K = H; m6.a = xa; m6.lda = H; m6.out_mode = OUT_SWIGLU; m6.y = m; m6.ldy = I; m6.y_bf16 = 1;
    MTP_TRY(timed_gemm(m6, s));
  } else if (lprod) {
    if (!normed_mlp) {
      LastRowsArgs gb = gr;
      gb.x = x1; gb.compact_in = 1; gb.K = H; gb.nw = h->w.post_attention_layernorm; gb.out = lb;
      MTP_TRY(launch_last_rows_norm(gb, s));
    }
    GemmArgs m6 = last_gemm(lb, H);
    m6.w[0] = static_cast<const uint16_t*>(h->w.gate_proj); m6.m[0] = I;
    m6.w[1] = static_cast<const uint16_t*>(h->w.up_proj); m6.m[1] = I;
    m6.M = I; m6.K = H; m6.out_mode = OUT_SWIGLU; m6.y = m; m6.ldy = I; m6.y_bf16 = 1;
    MTP_TRY(timed_gemm(m6, s));
  } else {
    MTP_TRY(run_gemv(a, h->wt, rows_total, rsel, s));
  }

  // 7. g = x1 + W_d m  (also written to hidden_out in the activation dtype)
  a = base_gemv(h, kv, ss);
  a.w[0] = h->w.down_proj; a.m[0] = H; a.M = H; a.K = I; a.lpr = lpr_for(I, h->wt);
  a.n_max = n_max; a.n_dev = n_dev;
  a.in_mode = IN_F32; a.x = m; a.ldx = I;
  a.out_mode = OUT_RESID; a.res = x1; a.ldres = H; a.y = g; a.ldy = H;
  a.y2 = hidden_out; a.y2_bf16 = c.act_dtype == MTP_BF16; a.ldy2 = H;
  if (mfma_out) {
    GemmArgs m7 = base_gemm(kv, n_max, n_dev, gpart, ss);
    m7.w[0] = static_cast<const uint16_t*>(h->w.down_proj); m7.m[0] = H; m7.M = H; m7.K = I;
    m7.a = m; m7.lda = I;
    m7.out_mode = OUT_RESID; m7.res = x1; m7.ldres = H; m7.y = g; m7.ldy = H;
    m7.y2 = hidden_out; m7.y2_bf16 = c.act_dtype == MTP_BF16; m7.ldy2 = H;
    MTP_TRY(timed_gemm(m7, s));
  } else if (lprod) {   // g rows compact; a split-K reduce also writes the unembedding's input rows
    GemmArgs m7 = last_gemm(m, I);
    m7.w[0] = static_cast<const uint16_t*>(h->w.down_proj); m7.m[0] = H; m7.M = H; m7.K = I;
    m7.out_mode = OUT_RESID; m7.res = x1; m7.ldres = H; m7.y = g; m7.ldy = H;
    const RowNorm rn{h->w.norm, h->wt == W_BF16, c.rms_eps, reinterpret_cast<uint16_t*>(wsp(ws, L.uxa)), H};
    MTP_TRY(timed_gemm(m7, s, &rn, &normed_g));
  } else {
    MTP_TRY(run_gemv(a, h->wt, rows_total, rsel, s));
  }

  // 8. logits = W_lm RMSNorm(g; w_norm) of the last row, with its argmax
  if (ss.multi() && unembed_product(c, slots)) {
    // the sessions' last rows normalised, one product over them, the chunk keys
    LastRowsArgs lr;
    std::memset(&lr, 0, sizeof(lr));
    lr.x = g; lr.K = H; lr.n_max = n_max; lr.n_dev = n_dev; lr.ndev_sb = ss.ndev_sb; lr.state = kv->state;
    lr.batch = ss.batch; lr.nw = h->w.norm; lr.nw_bf16 = h->wt == W_BF16; lr.eps = c.rms_eps;
    lr.out = reinterpret_cast<uint16_t*>(wsp(ws, L.uxa)); lr.rows = ss.batch;
    if (lprod) {   // g gathered already; each valid session's row also goes to hidden_out
      lr.compact_in = 1;
      lr.copy = hidden_out; lr.copy_bf16 = c.act_dtype == MTP_BF16;
      lr.copy_ld = static_cast<long long>(ss.out_sb) * H;
    }
    if (!normed_g) MTP_TRY(launch_last_rows_norm(lr, s));
    GemmArgs mu;
    std::memset(&mu, 0, sizeof(mu));
    mu.w[0] = static_cast<const uint16_t*>(h->w.lm_head); mu.m[0] = c.vocab; mu.M = c.vocab; mu.K = H;
    mu.n_max = ss.batch; mu.part = gpart;
    mu.a = lr.out; mu.lda = H; mu.out_mode = OUT_F32;
    mu.y = reinterpret_cast<float*>(wsp(ws, L.ulog)); mu.ldy = c.vocab;
    int tslot = -1;
    time_mark(TIME_UNEMBED, true, s, &tslot);
    const hipError_t eu = launch_gemm(mu, s);
    time_mark(TIME_UNEMBED, false, s, &tslot);
    MTP_TRY(eu);
    ArgmaxRowsArgs am;
    std::memset(&am, 0, sizeof(am));
    am.logits = mu.y; am.V = c.vocab; am.ld = c.vocab; am.n_dev = n_dev; am.ndev_sb = ss.ndev_sb;
    am.n_max = n_max; am.state = kv->state; am.batch = ss.batch;
    am.parts = reinterpret_cast<unsigned long long*>(wsp(ws, L.amax)); am.nparts = argmax_rows_parts(c.vocab);
    am.logits_out = logits; am.out_sb = ss.out_sb;
    if (normed_g) {   // the hidden copy of each valid session, with the chunk keys
      am.copy_src = g; am.K = H; am.copy = hidden_out; am.copy_bf16 = c.act_dtype == MTP_BF16;
      am.copy_ld = static_cast<long long>(ss.out_sb) * H;
    }
    MTP_TRY(launch_argmax_rows(am, s));
    f.parts = am.parts; f.nparts = am.nparts; f.amax_out = argmax;
    if (defer_out) {
      *defer_out = f;
      return MTP_OK;
    }
    MTP_TRY(launch_finish(f, s));
    return MTP_OK;
  }
  a = unembed_args(h, kv, L, n_max, n_dev, g, logits, ws, ss);
  int tslot = -1, grid = 0;
  time_mark(TIME_UNEMBED, true, s, &tslot);
  const int unr = last_row_nr(slots);
  MTP_TRY(launch_gemv(a, h->lmt, unr, s, &grid));
  for (int g0 = unr; g0 < (ss.multi() ? ss.batch : 1); g0 += unr) {
    // sessions g0 .. g0 + unr - 1; their keys continue the [session][grid] layout
    // (every launch of the same row count has the same grid)
    GemvArgs u = a;
    u.row_base = a.row_base + g0;
    u.amax_part = a.amax_part + static_cast<size_t>(g0) * grid;
    MTP_TRY(launch_gemv(u, h->lmt, unr, s, nullptr));
  }
  time_mark(TIME_UNEMBED, false, s, &tslot);
  // 9. argmax of the partial keys, commit the append (len, round base)
  f.parts = a.amax_part; f.nparts = grid; f.amax_out = argmax;
  if (defer_out) {
    *defer_out = f;
    return MTP_OK;
  }
  MTP_TRY(launch_finish(f, s));
  return MTP_OK;
}

}  // namespace

extern "C" {

const char* mtp_last_error(void) { return hipGetErrorString(g_last_hip); }

const char* mtp_status_string(int status) {
  switch (status) {
    case MTP_OK: return "MTP_OK";
    case MTP_E_INVALID_ARG: return "MTP_E_INVALID_ARG";
    case MTP_E_UNSUPPORTED: return "MTP_E_UNSUPPORTED";
    case MTP_E_NOT_BOUND: return "MTP_E_NOT_BOUND";
    case MTP_E_CAPACITY: return "MTP_E_CAPACITY";
    case MTP_E_HIP: return "MTP_E_HIP";
    case MTP_E_DEVICE: return "MTP_E_DEVICE";
    case MTP_E_WORKSPACE: return "MTP_E_WORKSPACE";
    default: return "MTP_E_UNKNOWN";
  }
}

int mtp_head_create(const mtp_head_config* cfg, const mtp_head_weights* w, mtp_head** out) {
  if (!out || !w) return MTP_E_INVALID_ARG;
  int st = validate_cfg(cfg);
  if (st != MTP_OK) return st;
  if (!w->embed || !w->lm_head) return MTP_E_NOT_BOUND;
  if (cfg->lm_head_dtype == MTP_I8G128 && !w->lm_head_scales) return MTP_E_INVALID_ARG;
  const void* req[] = {w->pre_fc_norm_embedding, w->pre_fc_norm_hidden, w->fc, w->input_layernorm,
                       w->q_proj, w->k_proj, w->v_proj, w->q_norm, w->k_norm, w->o_proj,
                       w->post_attention_layernorm, w->gate_proj, w->up_proj, w->down_proj, w->norm};
  for (const void* p : req)
    if (!p) return MTP_E_INVALID_ARG;
  mtp_head* h = new (std::nothrow) mtp_head;
  if (!h) return MTP_E_INVALID_ARG;
  h->cfg = *cfg;
  h->w = *w;
  h->wt = cfg->weight_dtype == MTP_BF16 ? W_BF16 : W_F32;
  h->lmt = cfg->lm_head_dtype == MTP_I8G128 ? W_I8 : (cfg->lm_head_dtype == MTP_BF16 ? W_BF16 : W_F32);
  // every GEMV shape must split into whole 16-byte chunks per lane
  const int H = cfg->hidden;
  if (!lpr_for(2 * H, h->wt) || !lpr_for(H, h->wt) || !lpr_for(cfg->intermediate, h->wt) ||
      !lpr_for(cfg->n_q_heads * cfg->head_dim, h->wt) || !lpr_for(H, h->lmt)) {
    delete h;
    return MTP_E_UNSUPPORTED;
  }
  *out = h;
  return MTP_OK;
}

void mtp_head_destroy(mtp_head* head) { delete head; }

size_t mtp_workspace_bytes(const mtp_head_config* cfg, int32_t max_rows, int32_t max_capacity) {
  if (validate_cfg(cfg) != MTP_OK || max_rows < 1 || max_rows > MTP_MAX_FLUSH || max_capacity < 1)
    return 0;
  return layout(*cfg, max_rows, max_capacity).total;
}

int mtp_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws || ws_bytes == 0) return MTP_E_INVALID_ARG;
  MTP_TRY(launch_fill_zero(ws, ws_bytes, stream));
  return MTP_OK;
}

int mtp_draft_step(const mtp_head* head, const mtp_kv* kv, const int32_t* token_dev,
                   const void* hidden_in_dev, void* hidden_out_dev, float* logits_dev,
                   int32_t* argmax_dev, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!head || !token_dev || !hidden_in_dev || !hidden_out_dev || !ws) return MTP_E_INVALID_ARG;
  if (hidden_in_dev == hidden_out_dev) return MTP_E_INVALID_ARG;
  int st = validate_kv(head, kv);
  if (st != MTP_OK) return st;
  if (ws_bytes < layout(head->cfg, 1, kv->capacity).total) return MTP_E_WORKSPACE;
  return head_forward(head, kv, token_dev, hidden_in_dev, 1, nullptr, MTP_FLUSH_LAST, 0,
                      hidden_out_dev, logits_dev, argmax_dev, ws, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The library's own scratch for mtp_draft_step_static: one array per device
// (each GPU the library runs on holds its own copy until the process ends).
// Host code never passes `scratch` itself to a kernel -- in host code that
// name is a stand-in, not a device address; the address comes from
// hipGetSymbolAddress once per device and is kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[MTP_STATIC_SCRATCH_BYTES];

namespace {
struct ScratchTable {
  std::mutex mu;
  std::map<int, void*> addr;   // device ordinal -> address of that device's scratch
} g_scratch;

// The current device's scratch address (looked up on the first call there).
hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_scratch.mu);
  auto it = g_scratch.addr.find(dev);
  if (it == g_scratch.addr.end()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    it = g_scratch.addr.emplace(dev, ptr).first;
  }
  *out = it->second;
  return hipSuccess;
}
}  // namespace

extern "C" {

int mtp_draft_step_static(const mtp_head* head, const mtp_kv* kv, const int32_t* token_dev,
                          const void* hidden_in_dev, void* hidden_out_dev, float* logits_dev,
                          int32_t* argmax_dev, hipStream_t stream) {
  if (!head || !token_dev || !hidden_in_dev || !hidden_out_dev) return MTP_E_INVALID_ARG;
  if (hidden_in_dev == hidden_out_dev) return MTP_E_INVALID_ARG;
  int st = validate_kv(head, kv);
  if (st != MTP_OK) return st;
  // the step's scratch must fit the static array (host check, nothing enqueued)
  if (layout(head->cfg, 1, kv->capacity).total > static_cast<size_t>(MTP_STATIC_SCRATCH_BYTES))
    return MTP_E_WORKSPACE;
  void* ws = nullptr;
  MTP_TRY(static_scratch(&ws));
  // every scratch value the step reads it first writes in the same call: no
  // clearing is needed between calls
  return head_forward(head, kv, token_dev, hidden_in_dev, 1, nullptr, MTP_FLUSH_LAST, 0, hidden_out_dev,
                      logits_dev, argmax_dev, ws, stream);
}

int mtp_flush_pairs(const mtp_head* head, const mtp_kv* kv, const int32_t* tokens_dev,
                    const void* hiddens_dev, int32_t n_max, const int32_t* n_dev, int32_t out_mode,
                    int32_t set_round_base, void* hidden_out_dev, float* logits_last_dev,
                    int32_t* argmax_last_dev, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!head || !tokens_dev || !hiddens_dev || !ws) return MTP_E_INVALID_ARG;
  if (out_mode != MTP_FLUSH_KV_ONLY && out_mode != MTP_FLUSH_LAST && out_mode != MTP_FLUSH_ALL)
    return MTP_E_INVALID_ARG;
  if (n_max < 1) return MTP_E_INVALID_ARG;
  if (n_max > MTP_MAX_FLUSH) return MTP_E_CAPACITY;
  int st = validate_kv(head, kv);
  if (st != MTP_OK) return st;
  if (!n_dev && n_max > kv->capacity) return MTP_E_CAPACITY;
  if (ws_bytes < layout(head->cfg, n_max, kv->capacity).total) return MTP_E_WORKSPACE;
  if (hidden_out_dev && hidden_out_dev == hiddens_dev) return MTP_E_INVALID_ARG;
  return head_forward(head, kv, tokens_dev, hiddens_dev, n_max, n_dev, out_mode,
                      set_round_base ? 1 : 0, hidden_out_dev, logits_last_dev, argmax_last_dev, ws,
                      stream);
}

int mtp_draft_chain(const mtp_head* head, const mtp_kv* kv, const int32_t* pend_tokens_dev,
                    const void* pend_hiddens_dev, int32_t n_max, const int32_t* n_dev, int32_t n_draft,
                    int32_t* drafts_dev, void* hiddens_out_dev, float* draft_logits_dev, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  if (!head || !pend_tokens_dev || !pend_hiddens_dev || !drafts_dev || !hiddens_out_dev || !ws)
    return MTP_E_INVALID_ARG;
  if (n_draft < 1 || n_draft > MTP_MAX_DRAFT || n_max < 1) return MTP_E_INVALID_ARG;
  if (n_max > MTP_MAX_FLUSH) return MTP_E_CAPACITY;
  int st = validate_kv(head, kv);
  if (st != MTP_OK) return st;
  if (ws_bytes < layout(head->cfg, n_max, kv->capacity).total) return MTP_E_WORKSPACE;
  if (hiddens_out_dev == pend_hiddens_dev) return MTP_E_INVALID_ARG;
  const mtp_head_config& c = head->cfg;
  const size_t row_bytes = static_cast<size_t>(c.hidden) * (c.act_dtype == MTP_BF16 ? 2 : 4);
  char* hout = static_cast<char*>(hiddens_out_dev);
  // the flush of the pending pairs gives d_0 and g_0
  // (a pending count of 0 is a device error here: a round always has a pending pair)
  // each step's argmax merge and append commit run inside the next step's fc
  // pass (the token it embeds); the last step's run on their own
  FinishArgs pend;
  std::memset(&pend, 0, sizeof(pend));
  st = head_forward(head, kv, pend_tokens_dev, pend_hiddens_dev, n_max, n_dev, MTP_FLUSH_LAST, 1, hout,
                    draft_logits_dev, drafts_dev, ws, stream, 1, kOneSession, nullptr,
                    n_draft > 1 ? &pend : nullptr);
  if (st != MTP_OK) return st;
  // chained steps: (d_{i-1}, g_{i-1}) -> d_i, g_i
  for (int i = 1; i < n_draft; ++i) {
    FinishArgs next;
    std::memset(&next, 0, sizeof(next));
    st = head_forward(head, kv, drafts_dev + (i - 1), hout + (i - 1) * row_bytes, 1, nullptr, MTP_FLUSH_LAST, 0,
                      hout + i * row_bytes, draft_logits_dev ? draft_logits_dev + static_cast<size_t>(i) * c.vocab
                                                             : nullptr,
                      drafts_dev + i, ws, stream, 0, kOneSession, &pend, i + 1 < n_draft ? &next : nullptr);
    if (st != MTP_OK) return st;
    pend = next;
  }
  return MTP_OK;
}

size_t mtp_batch_workspace_bytes(const mtp_head_config* cfg, int32_t batch, int32_t max_rows,
                                 int32_t max_capacity) {
  if (validate_cfg(cfg) != MTP_OK || batch < 1 || batch > MTP_MAX_BATCH || max_rows < 1 ||
      max_rows > MTP_MAX_FLUSH || max_capacity < 1)
    return 0;
  Sessions ss;
  ss.batch = batch;
  return layout(*cfg, batch * max_rows, max_capacity, slots_of(ss)).total;
}

int mtp_draft_chain_batch(const mtp_head* head, const mtp_kv* kv, int32_t batch, const int32_t* pend_tokens_dev,
                          const void* pend_hiddens_dev, int32_t n_max, const int32_t* n_dev, int32_t n_dev_stride,
                          int32_t n_draft, int32_t* drafts_dev, void* hiddens_out_dev, float* draft_logits_dev,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!head || !pend_tokens_dev || !pend_hiddens_dev || !drafts_dev || !hiddens_out_dev || !ws)
    return MTP_E_INVALID_ARG;
  if (batch < 1 || batch > MTP_MAX_BATCH) return MTP_E_INVALID_ARG;
  if (n_draft < 1 || n_draft > MTP_MAX_DRAFT || n_max < 1) return MTP_E_INVALID_ARG;
  if (n_dev && n_dev_stride < 1) return MTP_E_INVALID_ARG;
  if (n_max > MTP_MAX_FLUSH) return MTP_E_CAPACITY;
  int st = validate_kv(head, kv);
  if (st != MTP_OK) return st;
  if (!n_dev && n_max > kv->capacity) return MTP_E_CAPACITY;
  const mtp_head_config& c = head->cfg;
  if (ws_bytes < mtp_batch_workspace_bytes(&c, batch, n_max, kv->capacity)) return MTP_E_WORKSPACE;
  const size_t row_bytes = static_cast<size_t>(c.hidden) * (c.act_dtype == MTP_BF16 ? 2 : 4);
  // the hidden outputs must not overlap the pending hiddens they are computed from
  const char* hs = static_cast<const char*>(pend_hiddens_dev);
  char* hout = static_cast<char*>(hiddens_out_dev);
  const size_t in_span = static_cast<size_t>(batch) * n_max * row_bytes;
  const size_t out_span = static_cast<size_t>(batch) * n_draft * row_bytes;
  if (hout < hs + in_span && hs < hout + out_span) return MTP_E_INVALID_ARG;
  Sessions ss;
  ss.batch = batch;
  ss.kv_sb = static_cast<long long>(c.n_kv_heads) * kv->capacity * c.head_dim;
  ss.tok_sb = n_max;
  ss.hid_sb = n_max;
  ss.out_sb = n_draft;
  ss.ndev_sb = n_dev_stride;
  // every session's pending pairs in one flush: d_0 and g_0 of each session
  st = head_forward(head, kv, pend_tokens_dev, pend_hiddens_dev, n_max, n_dev, MTP_FLUSH_LAST, 1, hout,
                    draft_logits_dev, drafts_dev, ws, stream, 1, ss);
  if (st != MTP_OK) return st;
  // chained steps, one row per session: (d_{i-1}, g_{i-1}) -> d_i, g_i
  Sessions sc = ss;
  sc.tok_sb = n_draft;
  sc.hid_sb = n_draft;
  sc.ndev_sb = 0;
  for (int i = 1; i < n_draft; ++i) {
    st = head_forward(head, kv, drafts_dev + (i - 1), hout + (i - 1) * row_bytes, 1, nullptr, MTP_FLUSH_LAST, 0,
                      hout + i * row_bytes,
                      draft_logits_dev ? draft_logits_dev + static_cast<size_t>(i) * c.vocab : nullptr,
                      drafts_dev + i, ws, stream, 0, sc);
    if (st != MTP_OK) return st;
  }
  return MTP_OK;
}

int mtp_repair_pending(const int32_t* out_tokens_dev, const int32_t* out_counts_dev,
                       const void* target_hiddens_dev, int32_t hidden, int32_t act_dtype, int32_t n_draft,
                       int32_t* pend_tokens_dev, void* pend_hiddens_dev, int32_t* pend_count_dev,
                       hipStream_t stream) {
  if (!out_tokens_dev || !out_counts_dev || !target_hiddens_dev || !pend_tokens_dev || !pend_hiddens_dev ||
      !pend_count_dev)
    return MTP_E_INVALID_ARG;
  if (hidden < 1 || n_draft < 1 || n_draft > MTP_MAX_DRAFT) return MTP_E_INVALID_ARG;
  if (act_dtype != MTP_F32 && act_dtype != MTP_BF16) return MTP_E_INVALID_ARG;
  const size_t row_bytes = static_cast<size_t>(hidden) * (act_dtype == MTP_BF16 ? 2 : 4);
  // the pending rows must not overlap the rows they are copied from
  const char* hs = static_cast<const char*>(target_hiddens_dev);
  const char* hd = static_cast<const char*>(pend_hiddens_dev);
  const size_t span = (n_draft + 1) * row_bytes;
  if (hd < hs + span && hs < hd + span) return MTP_E_INVALID_ARG;
  MTP_TRY(launch_repair(out_tokens_dev, out_counts_dev, target_hiddens_dev, static_cast<int>(row_bytes / 2),
                        n_draft, pend_tokens_dev, pend_hiddens_dev, pend_count_dev, stream));
  return MTP_OK;
}

int mtp_repair_pending_batch(int32_t batch, const int32_t* out_tokens_dev, const int32_t* out_counts_dev,
                             const void* target_hiddens_dev, int32_t hidden, int32_t act_dtype, int32_t n_draft,
                             int32_t* pend_tokens_dev, void* pend_hiddens_dev, int32_t* pend_counts_dev,
                             hipStream_t stream) {
  if (!out_tokens_dev || !out_counts_dev || !target_hiddens_dev || !pend_tokens_dev || !pend_hiddens_dev ||
      !pend_counts_dev)
    return MTP_E_INVALID_ARG;
  if (batch < 1 || batch > MTP_MAX_BATCH) return MTP_E_INVALID_ARG;
  if (hidden < 1 || n_draft < 1 || n_draft > MTP_MAX_DRAFT) return MTP_E_INVALID_ARG;
  if (act_dtype != MTP_F32 && act_dtype != MTP_BF16) return MTP_E_INVALID_ARG;
  const size_t row_bytes = static_cast<size_t>(hidden) * (act_dtype == MTP_BF16 ? 2 : 4);
  const char* hs = static_cast<const char*>(target_hiddens_dev);
  const char* hd = static_cast<const char*>(pend_hiddens_dev);
  const size_t span = static_cast<size_t>(batch) * (n_draft + 1) * row_bytes;
  if (hd < hs + span && hs < hd + span) return MTP_E_INVALID_ARG;
  MTP_TRY(launch_repair(out_tokens_dev, out_counts_dev, target_hiddens_dev, static_cast<int>(row_bytes / 2),
                        n_draft, pend_tokens_dev, pend_hiddens_dev, pend_counts_dev, stream, batch));
  return MTP_OK;
}

size_t spec_verify_workspace_bytes(int32_t n_draft, int32_t vocab) {
  if (n_draft < 0 || n_draft > MTP_MAX_DRAFT || vocab < 1) return 0;
  const size_t nb = (static_cast<size_t>(vocab) + kVerifyChunk - 1) / kVerifyChunk;
  return kHeadBytes + align_up((n_draft + 1) * nb * 8) +
         align_up(verify_sampled_scratch_bytes(n_draft, vocab, kVerifyChunk));
}

}  // extern "C"

namespace {
// spec_verify over `batch` independent sessions (arrays session-major, one
// workspace of spec_verify_workspace_bytes per session)
int verify_sessions(const spec_sampling* sp, int32_t batch, int32_t n_draft, int32_t vocab,
                    const float* target_logits_dev, const float* draft_logits_dev,
                    const int32_t* draft_tokens_dev, int32_t* history_dev, int32_t* history_state_dev,
                    const float* uniforms_dev, int32_t* out_tokens_dev, int32_t* out_counts_dev,
                    void* ws, size_t ws_bytes, hipStream_t stream, int32_t* kv_state = nullptr,
                    int32_t kv_to_len = 0, int32_t kv_keep = 0, int32_t* report = nullptr) {
  if (!sp || !target_logits_dev || !history_dev || !history_state_dev || !out_tokens_dev ||
      !out_counts_dev || !ws)
    return MTP_E_INVALID_ARG;
  if (batch < 1 || batch > MTP_MAX_BATCH) return MTP_E_INVALID_ARG;
  if (n_draft < 0 || n_draft > MTP_MAX_DRAFT || vocab < 1) return MTP_E_INVALID_ARG;
  if (n_draft > 0 && !draft_tokens_dev) return MTP_E_INVALID_ARG;
  if (sp->window < 1 || sp->window > 1024) return MTP_E_INVALID_ARG;
  if (!(sp->temperature >= 0.f) || !std::isfinite(sp->temperature)) return MTP_E_INVALID_ARG;
  if (!(sp->repeat_penalty > 0.f) || !std::isfinite(sp->repeat_penalty)) return MTP_E_INVALID_ARG;
  if (!(sp->top_p > 0.f) || !(sp->min_p >= 0.f) || !(sp->min_p <= 1.f) || sp->top_k < 0)
    return MTP_E_INVALID_ARG;
  const size_t per = spec_verify_workspace_bytes(n_draft, vocab);
  if (per == 0 || ws_bytes < static_cast<size_t>(batch) * per) return MTP_E_WORKSPACE;
  const bool greedy = sp->temperature == 0.f;
  if (greedy != (draft_logits_dev == nullptr) && n_draft > 0) return MTP_E_INVALID_ARG;
  if (!greedy && !uniforms_dev) return MTP_E_INVALID_ARG;
  if (!greedy && !verify_sampled_supported(sp->top_k, vocab)) return MTP_E_UNSUPPORTED;
  VerifyArgs a;
  std::memset(&a, 0, sizeof(a));
  a.n_draft = n_draft; a.vocab = vocab;
  a.temperature = sp->temperature; a.penalty = sp->repeat_penalty; a.top_p = sp->top_p;
  a.min_p = sp->min_p; a.top_k = sp->top_k; a.window = sp->window;
  a.ln_min_p = sp->min_p > 0.f ? static_cast<float>(std::log(static_cast<double>(sp->min_p))) : -INFINITY;
  a.target = target_logits_dev; a.draft = draft_logits_dev; a.drafts = draft_tokens_dev;
  a.ring = history_dev; a.ring_state = history_state_dev; a.uniforms = uniforms_dev;
  a.out_tokens = out_tokens_dev; a.out_counts = out_counts_dev;
  a.chunk = kVerifyChunk;
  const size_t nb = (static_cast<size_t>(vocab) + kVerifyChunk - 1) / kVerifyChunk;
  a.parts = reinterpret_cast<unsigned long long*>(wsp(ws, kHeadBytes));
  a.scratch = wsp(ws, kHeadBytes + align_up((n_draft + 1) * nb * 8));
  a.batch = batch;
  a.sess_bytes = per;
  a.kv_state = kv_state;
  a.kv_to_len = kv_to_len;
  a.kv_keep = kv_keep;
  a.report = report;
  const hipError_t e = greedy ? launch_verify_greedy(a, stream) : launch_verify_sampled(a, stream);
  if (e == hipErrorNotSupported) return MTP_E_UNSUPPORTED;
  MTP_TRY(e);
  return MTP_OK;
}
}  // namespace

extern "C" {

int spec_verify(const spec_sampling* sp, int32_t n_draft, int32_t vocab,
                const float* target_logits_dev, const float* draft_logits_dev,
                const int32_t* draft_tokens_dev, int32_t* history_dev, int32_t* history_state_dev,
                const float* uniforms_dev, int32_t* out_tokens_dev, int32_t* out_counts_dev,
                void* ws, size_t ws_bytes, hipStream_t stream) {
  return verify_sessions(sp, 1, n_draft, vocab, target_logits_dev, draft_logits_dev, draft_tokens_dev, history_dev,
                         history_state_dev, uniforms_dev, out_tokens_dev, out_counts_dev, ws, ws_bytes, stream);
}

int spec_verify_rollback(const spec_sampling* sp, int32_t n_draft, int32_t vocab,
                         const float* target_logits_dev, const float* draft_logits_dev,
                         const int32_t* draft_tokens_dev, int32_t* history_dev, int32_t* history_state_dev,
                         const float* uniforms_dev, int32_t* out_tokens_dev, int32_t* out_counts_dev,
                         void* ws, size_t ws_bytes, const mtp_kv* kv, int32_t to_len, int32_t keep_accepted,
                         int32_t* report_dev, hipStream_t stream) {
  // the rollback's own argument rules (kv_rollback), checked before anything is enqueued
  if (!kv || !kv->state || kv->capacity <= 0) return MTP_E_INVALID_ARG;
  if (to_len < MTP_TO_ROUND_BASE) return MTP_E_INVALID_ARG;
  if (to_len > kv->capacity) return MTP_E_CAPACITY;
  if (keep_accepted != 0 && keep_accepted != 1) return MTP_E_INVALID_ARG;
  if (keep_accepted && to_len != MTP_TO_ROUND_BASE) return MTP_E_INVALID_ARG;
  return verify_sessions(sp, 1, n_draft, vocab, target_logits_dev, draft_logits_dev, draft_tokens_dev, history_dev,
                         history_state_dev, uniforms_dev, out_tokens_dev, out_counts_dev, ws, ws_bytes, stream,
                         kv->state, to_len, keep_accepted, report_dev);
}

int spec_verify_batch(const spec_sampling* sp, int32_t batch, int32_t n_draft, int32_t vocab,
                      const float* target_logits_dev, const float* draft_logits_dev,
                      const int32_t* draft_tokens_dev, int32_t* history_dev, int32_t* history_state_dev,
                      const float* uniforms_dev, int32_t* out_tokens_dev, int32_t* out_counts_dev,
                      void* ws, size_t ws_bytes, hipStream_t stream) {
  return verify_sessions(sp, batch, n_draft, vocab, target_logits_dev, draft_logits_dev, draft_tokens_dev,
                         history_dev, history_state_dev, uniforms_dev, out_tokens_dev, out_counts_dev, ws, ws_bytes,
                         stream);
}

int mtp_timing_begin(int32_t kind, int32_t max_launches) {
  if (max_launches < 1 || max_launches > (1 << 20)) return MTP_E_INVALID_ARG;
  if (kind < MTP_TIME_UNEMBED || kind > MTP_TIME_PROJECTION) return MTP_E_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_timer.mu);
  for (hipEvent_t e : g_timer.start) hipEventDestroy(e);
  for (hipEvent_t e : g_timer.stop) hipEventDestroy(e);
  g_timer.start.assign(max_launches, nullptr);
  g_timer.stop.assign(max_launches, nullptr);
  for (int i = 0; i < max_launches; ++i) {
    // Timing only: no system-scope fence (no cache write-back between the
    // bracketed launch and its neighbours).
    const unsigned fl = hipEventDisableSystemFence;
    if (hipEventCreateWithFlags(&g_timer.start[i], fl) != hipSuccess ||
        hipEventCreateWithFlags(&g_timer.stop[i], fl) != hipSuccess) {
      g_last_hip = hipErrorOutOfMemory;
      g_timer.on = false;
      return MTP_E_HIP;
    }
  }
  g_timer.used = 0;
  g_timer.kind = kind;
  g_timer.on = true;
  g_timer.paused = false;
  return MTP_OK;
}

int mtp_timing_pause(int32_t paused) {
  std::lock_guard<std::mutex> lk(g_timer.mu);
  g_timer.paused = paused != 0;
  return MTP_OK;
}

int mtp_timing_elapsed(int32_t first, int32_t count, float* total_ms) {
  if (!total_ms || first < 0 || count < 0) return MTP_E_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_timer.mu);
  if (first + count > g_timer.used) return MTP_E_INVALID_ARG;
  float sum = 0.f;
  for (int i = first; i < first + count; ++i) {
    MTP_TRY(hipEventSynchronize(g_timer.stop[i]));
    float ms = 0.f;
    MTP_TRY(hipEventElapsedTime(&ms, g_timer.start[i], g_timer.stop[i]));
    sum += ms;
  }
  *total_ms = sum;
  return MTP_OK;
}

int mtp_timing_end(float* total_ms, int32_t* launches) {
  if (!total_ms || !launches) return MTP_E_INVALID_ARG;
  float sum = 0.f;
  int used = 0;
  {
    std::lock_guard<std::mutex> lk(g_timer.mu);
    g_timer.on = false;
    used = g_timer.used;
  }
  const int st = mtp_timing_elapsed(0, used, &sum);
  std::lock_guard<std::mutex> lk(g_timer.mu);
  for (hipEvent_t e : g_timer.start) hipEventDestroy(e);
  for (hipEvent_t e : g_timer.stop) hipEventDestroy(e);
  g_timer.start.clear();
  g_timer.stop.clear();
  g_timer.used = 0;
  if (st != MTP_OK) return st;
  *total_ms = sum;
  *launches = used;
  return MTP_OK;
}

int kv_rollback(const mtp_kv* kv, int32_t to_len, const int32_t* n_accepted_dev, int32_t n_draft,
                hipStream_t stream) {
  if (!kv || !kv->state || kv->capacity <= 0) return MTP_E_INVALID_ARG;
  if (to_len < MTP_TO_ROUND_BASE) return MTP_E_INVALID_ARG;
  if (to_len > kv->capacity) return MTP_E_CAPACITY;
  if (n_draft < 0 || n_draft > MTP_MAX_DRAFT) return MTP_E_INVALID_ARG;
  if (n_accepted_dev && to_len != MTP_TO_ROUND_BASE) return MTP_E_INVALID_ARG;
  MTP_TRY(launch_rollback(kv->state, to_len, n_accepted_dev, n_draft, kv->capacity, stream));
  return MTP_OK;
}

int kv_rollback_batch(const mtp_kv* kv, int32_t batch, int32_t to_len, const int32_t* counts_dev, int32_t n_draft,
                      hipStream_t stream) {
  if (!kv || !kv->state || kv->capacity <= 0) return MTP_E_INVALID_ARG;
  if (batch < 1 || batch > MTP_MAX_BATCH) return MTP_E_INVALID_ARG;
  if (to_len < MTP_TO_ROUND_BASE) return MTP_E_INVALID_ARG;
  if (to_len > kv->capacity) return MTP_E_CAPACITY;
  if (n_draft < 0 || n_draft > MTP_MAX_DRAFT) return MTP_E_INVALID_ARG;
  if (counts_dev && to_len != MTP_TO_ROUND_BASE) return MTP_E_INVALID_ARG;
  MTP_TRY(launch_rollback(kv->state, to_len, counts_dev, n_draft, kv->capacity, stream, batch, 2));
  return MTP_OK;
}

}  // extern "C"
