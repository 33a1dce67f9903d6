// Host-visible launch interfaces of the gfx950 kernels (C++ linkage, used by
// the C ABI in api.cpp).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtp {

// Benchmark timing hook (defined with the C ABI): brackets one launch of kernel
// class `kind` with events on `s` when that class is being timed.  *slot
// carries the event slot from the `before` call to the `after` call.
void time_mark(int kind, bool before, hipStream_t s, int* slot);
enum TimeKind { TIME_UNEMBED = 0, TIME_ATTENTION = 1, TIME_VERIFY = 2, TIME_PROJECTION = 3 };

enum WType { W_F32 = 0, W_BF16 = 1, W_I8 = 2 };
enum InMode { IN_F32 = 0, IN_RMS = 1, IN_EMBED = 2 };
enum OutMode { OUT_F32 = 0, OUT_RESID = 1, OUT_SWIGLU = 2, OUT_LOGITS = 3 };
enum RowSel { ROWS_RANGE = 0, ROW_LAST = 1 };

// y[j, r] = sum_k W[r, k] * in(j)[k] for activation rows j, weight rows r.
struct GemvArgs {
  const void* w[3];        // up to three stacked matrices (rows concatenated)
  int m[3];                // rows of each
  int M;                   // output rows (SWIGLU: rows of one of the pair)
  int K;                   // columns
  const uint16_t* scales;  // W_I8: fp16 scales [M, K/128]
  int lpr;                 // lanes per weight row (8..64, divides K/elements-per-16B)
  int kp;                  // columns staged in LDS per phase
  int grid_stride;         // single phase: workgroups loop over row blocks
  // activation rows: j in [row_base, row_base + NR) and j < n, or j = n - 1
  int row_sel;
  int row_base;
  int n_max;
  const int32_t* n_dev;    // nullable device count
  // input
  int in_mode;
  const float* x;
  int ldx;
  const void* nw;          // IN_RMS norm weight / IN_EMBED embedding-half norm
  const void* nw2;         // IN_EMBED hidden-half norm
  int nw_bf16;
  float eps;
  const int32_t* tok;      // IN_EMBED: token ids, valid in [0, vocab_tok)
  int vocab_tok;
  int32_t* err;            // IN_EMBED: state[3], set to 4 on a token out of range
  const void* embed;
  int embed_bf16;
  const void* hid;
  int hid_bf16;
  int ld_hid;
  // output
  int out_mode;
  float* y;
  int ldy;
  const float* res;
  int ldres;
  void* y2;                // optional copy in act dtype (ROW_LAST: written at row 0)
  int y2_bf16;
  int ldy2;
  float* logits;           // OUT_LOGITS (nullable)
  unsigned long long* amax_part;  // OUT_LOGITS: one argmax key per workgroup
  const int32_t* kv_state; // nullable: skip everything when state[3] != 0
  int dry_run;             // compute the launch shape only (*grid_out), enqueue nothing
  // batch > 1: independent sessions in one launch.  n_max is the rows per
  // session and workspace rows are flattened b * n_max + j; session b's state
  // words are kv_state + 4 b (a set error word drops its rows) and its count
  // n_dev[b * ndev_sb]; its token j is tok[b * tok_sb + j], its hidden row
  // b * hid_sb + j.  ROW_LAST: slot r is session row_base + r, whose hidden copy
  // and logits go to row b * out_sb of y2 and logits ([rows, vocab]).
  int batch;
  int tok_sb, hid_sb, out_sb, ndev_sb;
  // IN_EMBED with one session and one row: the previous step's argmax merge
  // and append commit folded into this launch (fin_parts nullable).  The token
  // is the argmax of fin_parts[0, fin_nparts) when that step had rows (fin_n =
  // clamp(*fin_ndev or fin_nmax, 0, fin_nmax) > 0), else tok[0]; workgroup 0
  // stores it at fin_amax and commits fin_state[0] += fin_n (fin_state[1] = the
  // new length when fin_set_base).  Nothing in this launch reads those words.
  const unsigned long long* fin_parts;
  int fin_nparts;
  int32_t* fin_amax;
  const int32_t* fin_ndev;
  int fin_nmax;
  int fin_set_base;
  int32_t* fin_state;
  // Up to four activation rows, single phase (set by the launcher; more than
  // one row only over large matrices): each wave's first
  // pf chunks per lane of every row slot of its first row block are loaded
  // straight into LDS at byte offset pf_off of the dynamic LDS before the input
  // staging (their memory latency overlaps it; no registers are held).
  int pf;
  int pf_off;
};

// *grid_out (nullable) receives the number of workgroups launched.
hipError_t launch_gemv(const GemvArgs& a, int wtype, int nr, hipStream_t s, int* grid_out = nullptr);

// Normalised bf16 input rows for the matrix-core projections: RMSNorm(x; nw)
// (IN_RMS) or [RMSNorm(E[tok]; nw) | RMSNorm(hid; nw2)] (IN_EMBED, K = 2H), one
// row per activation row j < n.
struct PrepArgs {
  int in_mode;
  int K;
  int n_max;
  const int32_t* n_dev;
  const int32_t* kv_state;   // skip everything when state[3] != 0
  const float* x;
  int ldx;
  const void* nw;
  const void* nw2;
  int nw_bf16;
  float eps;
  const int32_t* tok;
  int vocab_tok;
  int32_t* err;              // state[3], set to 4 on a token out of range
  const void* embed;
  int embed_bf16;
  const void* hid;
  int hid_bf16;
  int ld_hid;
  uint16_t* out;             // [n_max, ld_out] bf16
  int ld_out;
  // batch > 1: n_max rows per session, batch * n_max rows in all (flattened
  // b * n_max + j); rows past a session's count (or of a session whose error
  // word is set) are written as zeros; session b's token j is tok[b * tok_sb +
  // j], its hidden row b * hid_sb + j, its count n_dev[b * ndev_sb], its state
  // words kv_state + 4 b.
  int batch;
  int tok_sb, hid_sb, ndev_sb;
};
hipError_t launch_rows_prep(const PrepArgs& a, hipStream_t s);

// Several sessions' last rows normalised into bf16 rows (the batched
// unembedding's product input): out row b = bf16(x * nw * inv_rms) of session
// b's last row x (flattened rows b * n_max + j), zeros past the batch, for a
// session with no row or with its error word set.  One workgroup per row.
struct LastRowsArgs {
  const float* x;            // [batch * n_max, K], or [batch, K] when compact_in
  int K;
  int n_max;
  const int32_t* n_dev;      // session b's count n_dev[b * ndev_sb] (null: n_max)
  int ndev_sb;
  const int32_t* state;      // session b's state words state + 4 b
  int batch;
  const void* nw;
  int nw_bf16;
  float eps;
  uint16_t* out;             // [rows, K] bf16
  int rows;                  // >= batch
  int compact_in;            // session b's row is x + b K (already gathered)
  void* copy;                // nullable: the row itself of each valid session at copy + b copy_ld
  int copy_bf16;
  long long copy_ld;
};
hipError_t launch_last_rows_norm(const LastRowsArgs& a, hipStream_t s);

// The argmax key of every 4096-logit chunk of each session's logits row
// (parts[b * nparts + c]; 0 for a session without a row), the row copied to
// logits_out + b * out_sb * V when that is set and the session has a row.
struct ArgmaxRowsArgs {
  const float* logits;       // [batch, ld]
  int V;
  int ld;
  const int32_t* n_dev;
  int ndev_sb;
  int n_max;
  const int32_t* state;
  int batch;
  unsigned long long* parts;
  int nparts;                // argmax_rows_parts(V)
  float* logits_out;         // nullable
  int out_sb;
  // nullable: each valid session's row copy_src + b K also goes to copy + b
  // copy_ld (the hidden copy), spread over the row's chunk blocks
  const float* copy_src;
  int K;
  void* copy;
  int copy_bf16;
  long long copy_ld;
};
int argmax_rows_parts(int V);
hipError_t launch_argmax_rows(const ArgmaxRowsArgs& a, hipStream_t s);

// Y[j, c] = sum_k A[j, k] W[c, k] over activation rows j < n on bf16 MFMA tiles
// (64 rows x 64 columns per workgroup).  W: up to three stacked bf16 matrices
// (OUT_SWIGLU: w[0] gate and w[1] up, M rows each).  A: bf16 rows, or fp32 rows
// rounded to bf16 on load (a_f32).  Requires M, K and every m[i] multiples of 64.
struct GemmArgs {
  const uint16_t* w[3];
  int m[3];
  int M;
  int K;
  int n_max;
  const int32_t* n_dev;
  const int32_t* kv_state;
  const void* a;
  int a_f32;
  int lda;
  int out_mode;              // OUT_F32, OUT_RESID or OUT_SWIGLU
  float* y;
  int ldy;
  const float* res;
  int ldres;
  void* y2;                  // optional copy of y in the activation dtype
  int y2_bf16;
  int ldy2;
  float* part;               // split partial sums [split, n_max, M] (gemm_part_floats)
  int y_bf16;                // OUT_SWIGLU: y holds bf16 (ldy in bf16 elements)
  int sk_units;              // set by launch_gemm: stream-K steps per workgroup (0 = off)
};
// The next projection's input row, RMSNorm(y; nw) in bf16, produced by the
// product's split-K reduce when it runs (one launch instead of two).
struct RowNorm {
  const void* nw;            // norm weight [M]
  int nw_bf16;
  float eps;
  uint16_t* out;             // bf16 rows [n, ld_out]
  int ld_out;
};
// rn (nullable): also write RMSNorm(y) rows when the product reduces split-K
// partials; *normed (nullable) tells whether it did (else the caller preps).
// split_left (nullable): a plain split-K product (no rn) leaves its partials
// in a.part ([split, n_max, M]) unreduced and stores the split count there (1
// when the product ran unsplit, or reduced them itself): the caller's next
// kernel sums them.
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s, const RowNorm* rn = nullptr, bool* normed = nullptr,
                       int* split_left = nullptr);
bool gemm_supported(int M, int K, const int* m, int nmat);
// fp32 elements of the partial-sum workspace a product of `rows` rows needs
// (0 when it runs unsplit)
size_t gemm_part_floats(int rows, int M, int K, const int* m, int nmat, bool swiglu);

// q/k RMSNorm + RoPE for rows j < n at positions state[0] + j, append k, v to
// the cache, write roped q to `q_out`.  state[0] is advanced later by k_finish.
struct RopeArgs {
  const float* qkv;        // [rows, (Hq + 2 Hkv) * D]
  int ld_qkv;
  float* q_out;            // [rows, Hq * D]
  const void* q_norm;
  const void* k_norm;
  int nw_bf16;
  float eps;
  float theta;
  int hq, hkv, d;
  void* kc;
  void* vc;
  int kv_bf16;
  int capacity;
  int32_t* state;
  int n_max;
  const int32_t* n_dev;
  int n_min;               // a device count below n_min (or above n_max) sets MTP_DEV_COUNT
};
hipError_t launch_rope_append(const RopeArgs& a, hipStream_t s);

// Split-K attention of query rows over the draft KV, then a merge.
struct AttnArgs {
  const float* q;          // [rows, Hq * D] roped
  void* kc;
  void* vc;
  int kv_bf16;
  int capacity;
  int32_t* state;
  int hq, hkv, d;
  int n_max;
  const int32_t* n_dev;
  int n_min;               // fuse_rope: a device count below n_min sets MTP_DEV_COUNT
  // batch > 1 (ROW_LAST with fuse_rope only): session b's K/V start kv_sb
  // elements after session b - 1's, its state words are state + 4 b, its count
  // n_dev[b * ndev_sb]; its rows are the workspace rows b * n_max + j
  int batch;
  long long kv_sb;
  int ndev_sb;
  int row_sel;             // ROWS_RANGE: rows 0..n-1; ROW_LAST: row n-1
  int nchunk;              // chunks per (row, kv head)
  int mfma;                // ROWS_RANGE over bf16 K/V: the matrix-core flush kernel
  float* part_o;           // [rows, Hq, nchunk, D]
  float* part_ml;          // [rows, Hq, nchunk, 2]
  float* o;                // [rows, Hq * D] (bf16 when o_bf16)
  int o_bf16;
  // several sessions, ROW_LAST: the merge writes session b's o row at row b
  // (bf16, o_bf16 set) and copies its residual row xg[b * n_max + n - 1] to
  // xg_out[b] (ld_xg floats), zeros for a session without a row
  int o_compact;
  const float* xg;
  float* xg_out;
  int ld_xg;
  // ROW_LAST with fuse_rope: the q/k RMSNorm + RoPE and the K/V append of the
  // rows j < n run inside the attention kernel (no separate append launch); the
  // q/k/v projections of the rows are read from qkv, or, with qkv_nsp > 1, are
  // the sums in split order of the product's split-K partials qkv + q *
  // qkv_pstride, q < qkv_nsp (the reduce the product would have launched).
  int fuse_rope;
  const float* qkv;        // [rows, (Hq + 2 Hkv) * D]
  int ld_qkv;
  int qkv_pstride;
  int qkv_nsp;
  const void* q_norm;
  const void* k_norm;
  int nw_bf16;
  float eps;
  float theta;
};
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
// smallest head_dim whose fused prologue sums split partials (qkv_nsp > 1)
constexpr int kSplitMinHeadDim = 128;
// the matrix-core flush attention and its merge (chunks at most kFlushMaxChunks)
constexpr int kFlushMaxChunks = 128;
hipError_t launch_attention_flush(const AttnArgs& a, hipStream_t s);

// End of a step or flush: merge the unembedding's per-workgroup argmax keys
// (if any) into *amax_out and commit the append: state[0] += n (state[1] too
// when set_base).  One workgroup.
struct FinishArgs {
  int32_t* state;
  int n_max;
  const int32_t* n_dev;
  int set_base;
  const unsigned long long* parts;  // nullable
  int nparts;
  int32_t* amax_out;                // nullable
  // batch > 1: one workgroup per session b: state + 4 b, count n_dev[b *
  // ndev_sb], argmax keys parts[b * nparts ..], result amax_out[b * out_sb]
  int batch;
  int out_sb, ndev_sb;
};
hipError_t launch_finish(const FinishArgs& a, hipStream_t s);

// Greedy verification (argmax match) with repetition penalty.
struct VerifyArgs {
  int n_draft, vocab;
  float temperature, penalty, top_p, min_p;
  int top_k, window;
  float ln_min_p;
  const float* target;
  const float* draft;
  const int32_t* drafts;
  int32_t* ring;
  int32_t* ring_state;
  const float* uniforms;
  int32_t* out_tokens;
  int32_t* out_counts;
  unsigned long long* parts;   // [n_draft + 1][blocks per row] argmax keys
  void* scratch;               // sampled path candidates
  int chunk;                   // elements per workgroup
  // batch > 1: blockIdx.z is the session b; every per-session array above
  // advances by b times its own size (rows, drafts, ring, ring state,
  // uniforms, outputs) and parts / scratch by b * sess_bytes
  int batch;
  size_t sess_bytes;
  // The round's tail in the final kernel (one session): when kv_state is set,
  // the draft KV's state words roll back as kv_rollback(kv_to_len, kv_keep ?
  // &k : NULL) would; then, when report is set, the row {state words, k, k + 1,
  // committed run} is written there (system-scope stores).
  int32_t* kv_state;
  int kv_to_len, kv_keep;
  int32_t* report;
};
hipError_t launch_verify_greedy(const VerifyArgs& a, hipStream_t s);
hipError_t launch_verify_sampled(const VerifyArgs& a, hipStream_t s);
size_t verify_sampled_scratch_bytes(int n_draft, int vocab, int chunk);
// any top_k >= 0 (the whole-vocabulary path takes what the per-chunk
// candidates cannot hold)
bool verify_sampled_supported(int top_k, int vocab);

// batch sessions (state words state + 4 b, accepted count n_acc[b * acc_stride])
hipError_t launch_rollback(int32_t* state, int to_len, const int32_t* n_acc, int n_draft,
                           int capacity, hipStream_t s, int batch = 1, int acc_stride = 0);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_repair(const int32_t* out_tokens, const int32_t* out_counts, const void* hid, int elems16,
                         int n_draft, int32_t* pend_tokens, void* pend_hid, int32_t* pend_count, hipStream_t s,
                         int batch = 1);

}  // namespace mtp
