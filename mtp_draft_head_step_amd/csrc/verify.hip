// Speculative verification on gfx950.
//
// Greedy (temperature 0): the sampler is a point mass, so acceptance is
// "draft i equals the argmax of target row i" (with the repetition penalty
// applied to the row's window first).  Each row is split over many workgroups;
// the window tokens that fall in a workgroup's id range are marked in an LDS
// bitmap so the penalty costs one LDS read per logit.  Every workgroup writes
// its partial argmax key; a one-workgroup kernel merges them per row, resolves
// the accepted count, writes the committed run and pushes it into the ring.
#include "common.h"
#include "kernels.h"

namespace mtp {

constexpr int kVThreads = 256;
constexpr int kVMaxChunk = 8192;
constexpr int kVGreedyChunk = 4096;   // logits per greedy workgroup (the host's chunk)

// Token at position idx of (ring oldest-first ++ drafts).
__device__ __forceinline__ int window_token(const int32_t* ring, int head, int count, int window,
                                            const int32_t* drafts, int idx) {
  if (idx < count) {
    int p = head - count + idx;
    p %= window;
    if (p < 0) p += window;
    return ring[p];
  }
  return drafts[idx - count];
}

// The ring's state words as stored by the caller, brought into range: head in
// [0, window), count in [0, window].
__device__ __forceinline__ int ring_head(const VerifyArgs& a) {
  const int h = a.ring_state[0] % a.window;
  return h < 0 ? h + a.window : h;
}
__device__ __forceinline__ int ring_count(const VerifyArgs& a) { return min(max(a.ring_state[1], 0), a.window); }

__device__ __forceinline__ float penalise(float v, float pen) { return v > 0.f ? v / pen : v * pen; }

// Session blockIdx.z's view of the arguments (several independent sessions in
// one launch); the identity for one session.
__device__ __forceinline__ VerifyArgs at_session(VerifyArgs a) {
  if (a.batch <= 1) return a;
  const size_t b = blockIdx.z;
  const size_t n = a.n_draft, v = a.vocab;
  a.target += b * (n + 1) * v;
  if (a.draft) a.draft += b * n * v;
  if (a.drafts) a.drafts += b * n;
  a.ring += b * a.window;
  a.ring_state += 2 * b;
  if (a.uniforms) a.uniforms += b * (n + 1);
  a.out_tokens += b * (n + 1);
  a.out_counts += 2 * b;
  a.parts = reinterpret_cast<unsigned long long*>(reinterpret_cast<char*>(a.parts) + b * a.sess_bytes);
  a.scratch = static_cast<char*>(a.scratch) + b * a.sess_bytes;
  return a;
}

// The draft KV's state words {length, round base, word 2, error}, loaded with
// the final kernel's other inputs (zeros without a fused rollback).
struct KvWords {
  int len, base, w2, err;
};
__device__ __forceinline__ KvWords load_kv_words(const VerifyArgs& a) {
  KvWords w{0, 0, 0, 0};
  if (a.kv_state) {
    w.len = a.kv_state[0];
    w.base = a.kv_state[1];
    w.w2 = a.kv_state[2];
    w.err = a.kv_state[3];
  }
  return w;
}

// Stores the host may read once the kernel is done (host-coherent memory):
// system scope, so no cache level keeps them.
__device__ __forceinline__ void store_sys(int32_t* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// One thread commits a verified round: the run dr[0..k-1], tok goes to
// out_tokens and into the history ring, the counts {k, k + 1} and the ring's
// state words are stored; then the fused tail (see VerifyArgs): the draft-KV
// rollback with this k and the report row.
__device__ void commit_round(const VerifyArgs& a, const int32_t* dr, int k, int tok, KvWords w) {
  int h = ring_head(a), c = ring_count(a);
  int32_t* rep = a.report;
  for (int r = 0; r <= k; ++r) {
    const int t = r < k ? dr[r] : tok;
    a.out_tokens[r] = t;
    a.ring[h] = t;
    if (rep) store_sys(rep + 6 + r, t);
    h = (h + 1) % a.window;
    c = c + 1 < a.window ? c + 1 : a.window;
  }
  a.out_counts[0] = k;
  a.out_counts[1] = k + 1;
  a.ring_state[0] = h;
  a.ring_state[1] = c;
  if (!a.kv_state) return;
  if (w.err == 0) {
    const int to = rollback_length(a.kv_to_len, w.len, w.base, k, a.kv_keep != 0, a.n_draft);
    if (to < 0) {
      w.err = 2;
      a.kv_state[3] = 2;
    } else {
      w.len = to;
      a.kv_state[0] = to;
    }
  }
  if (rep) {
    store_sys(rep + 0, w.len);
    store_sys(rep + 1, w.base);
    store_sys(rep + 2, w.w2);
    store_sys(rep + 3, w.err);
    store_sys(rep + 4, k);
    store_sys(rep + 5, k + 1);
  }
}

__global__ __launch_bounds__(kVThreads) void k_verify_greedy(VerifyArgs a) {
  a = at_session(a);
  __shared__ uint32_t bits[kVMaxChunk / 32];
  __shared__ unsigned long long s_best[kVThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = blockIdx.y;
  const int lo = blockIdx.x * a.chunk;
  const int hi = min(a.vocab, lo + a.chunk);
  const bool pen = a.penalty != 1.0f;
  const int head = ring_head(a);
  const int count = ring_count(a);
  // the chunk's logits first (all loads in flight at once), then the window
  const float* row = a.target + static_cast<size_t>(i) * a.vocab;
  constexpr int kPer = kVGreedyChunk / kVThreads;
  float v[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int k = lo + tid + u * kVThreads;
    v[u] = k < hi ? row[k] : 0.f;
  }
  if (pen) {
    for (int w = tid; w < kVMaxChunk / 32; w += kVThreads) bits[w] = 0u;
    __syncthreads();
    const int total = count + i;
    const int start = total > a.window ? total - a.window : 0;
    for (int t = start + tid; t < total; t += kVThreads) {
      const int tok = window_token(a.ring, head, count, a.window, a.drafts, t);
      if (tok >= lo && tok < hi) atomicOr(&bits[(tok - lo) >> 5], 1u << ((tok - lo) & 31));
    }
    __syncthreads();
  }
  unsigned long long best = 0ull;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int k = lo + tid + u * kVThreads;
    if (k >= hi) continue;
    float x = v[u];
    if (pen && ((bits[(k - lo) >> 5] >> ((k - lo) & 31)) & 1u)) x = penalise(x, a.penalty);
    const unsigned long long key = argmax_key(x, static_cast<uint32_t>(k));
    best = key > best ? key : best;
  }
  best = wave_max_u64(best);
  if (lane == 0) s_best[wave] = best;
  __syncthreads();
  if (tid == 0) {
    unsigned long long b = s_best[0];
    for (int w = 1; w < kVThreads / 64; ++w) b = s_best[w] > b ? s_best[w] : b;
    a.parts[static_cast<size_t>(i) * gridDim.x + blockIdx.x] = b;
  }
}

// Every load first (one memory round trip): the argmax keys of all rows
// (flattened [rows][nb]), the drafts and the ring state; each row's maximum by
// LDS atomics (order-free), then thread 0 walks the acceptance.
__global__ __launch_bounds__(kVThreads) void k_verify_greedy_finish(VerifyArgs a, int nb) {
  a = at_session(a);
  __shared__ unsigned long long s_row[MTP_MAX_DRAFT_DEV + 1];
  __shared__ int s_dr[MTP_MAX_DRAFT_DEV];
  const int tid = threadIdx.x;
  const int n = a.n_draft;
  const int tot = (n + 1) * nb;
  constexpr int kPer = 4;
  unsigned long long v[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int e = tid + u * kVThreads;
    v[u] = e < tot ? a.parts[e] : 0ull;
  }
  const int dr = tid < n ? a.drafts[tid] : 0;
  const KvWords w = tid == 0 ? load_kv_words(a) : KvWords{0, 0, 0, 0};
  if (tid <= n) s_row[tid] = 0ull;
  if (tid < n) s_dr[tid] = dr;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int e = tid + u * kVThreads;
    if (e < tot) atomicMax(&s_row[e / nb], v[u]);
  }
  for (int e = tid + kPer * kVThreads; e < tot; e += kVThreads) atomicMax(&s_row[e / nb], a.parts[e]);
  __syncthreads();
  if (tid != 0) return;
  int k = n;
  for (int r = 0; r < n; ++r) {
    if (s_dr[r] != argmax_index(s_row[r])) { k = r; break; }
  }
  commit_round(a, s_dr, k, argmax_index(s_row[k]), w);
}

hipError_t launch_verify_greedy(const VerifyArgs& a, hipStream_t s) {
  if (a.chunk != kVGreedyChunk) return hipErrorInvalidValue;
  const unsigned bz = a.batch > 1 ? a.batch : 1;
  const int nb = (a.vocab + a.chunk - 1) / a.chunk;
  (void)hipGetLastError();
  int slot = -1;
  time_mark(TIME_VERIFY, true, s, &slot);
  hipLaunchKernelGGL(k_verify_greedy, dim3(nb, a.n_draft + 1, bz), dim3(kVThreads), 0, s, a);
  time_mark(TIME_VERIFY, false, s, &slot);
  hipLaunchKernelGGL(k_verify_greedy_finish, dim3(1, 1, bz), dim3(kVThreads), 0, s, a, nb);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Sampled verification (temperature > 0): Leviathan/Chen rejection sampling
// over transformed rows.  Rows 0..N are the target rows, N+1..2N the draft rows.
//  A. k_sample_chunk  (chunks x rows): a chunk's logits are penalised (window of
//     its row), divided by the temperature and turned into 64-bit keys (value
//     desc, id asc); a radix select finds the chunk's kk-th key and the kk keys
//     at or above it are kept (sorted when kk <= 64).
//  B. k_sample_row    (rows): the row's exact top-k: for k <= 64 the chunks'
//     lists arrive sorted and are folded by bitonic merges in registers (one
//     list per merge, a running top 64 per wave); larger k by a radix select
//     over every candidate.  Softmax over it, top-p prefix, min-p cut,
//     renormalise; the support is written sorted by token id.
//  C. k_sample_decide (1 thread): accept d_i iff u_i q_i(d_i) < p_i(d_i); at the
//     first rejection draw from normalise(max(0, p - q)) (p if that is zero) with
//     u_N by inverse CDF in ascending id; else the bonus from p_N; ring push.
constexpr int kSChunk = 4096;      // logits per phase-A workgroup
constexpr int kSMaxCand = 8192;    // phase-B merge capacity (keys)
constexpr int kSMaxTopK = 256;     // largest supported top_k

struct SampledScratch {
  unsigned long long* cand;  // [rows][nb * kk]
  int* cnt;                  // [rows]
  int* ids;                  // [rows][kSMaxTopK]
  float* probs;              // [rows][kSMaxTopK]
};

__host__ __device__ inline size_t align256(size_t v) { return (v + 255) / 256 * 256; }

__host__ __device__ inline SampledScratch sampled_scratch(void* base, int n_draft, int vocab) {
  const int rows = 2 * n_draft + 1;
  const int nb = (vocab + kSChunk - 1) / kSChunk;
  char* p = static_cast<char*>(base);
  SampledScratch s;
  s.cand = reinterpret_cast<unsigned long long*>(p);
  p += align256(static_cast<size_t>(rows) * nb * kSMaxTopK * 8);
  s.cnt = reinterpret_cast<int*>(p);
  p += align256(static_cast<size_t>(rows) * 4);
  s.ids = reinterpret_cast<int*>(p);
  p += align256(static_cast<size_t>(rows) * kSMaxTopK * 4);
  s.probs = reinterpret_cast<float*>(p);
  return s;
}

size_t full_scratch_bytes(int n_draft, int vocab);

// either path's scratch (both start at the same place)
size_t verify_sampled_scratch_bytes(int n_draft, int vocab, int chunk) {
  (void)chunk;
  const int rows = 2 * n_draft + 1;
  const size_t nb = (static_cast<size_t>(vocab) + kSChunk - 1) / kSChunk;
  const size_t radix =
      align256(rows * nb * kSMaxTopK * 8) + align256(rows * 4ull) + 2 * align256(rows * kSMaxTopK * 4ull) + 256;
  const size_t full = full_scratch_bytes(n_draft, vocab);
  return radix > full ? radix : full;
}

__device__ __forceinline__ float key_value(unsigned long long key) {
  const uint32_t k = static_cast<uint32_t>(key >> 32);
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// Radix select over the workgroup's 64-bit keys (N per thread, 0 = empty; real
// keys are distinct): returns the kk-th largest key T, so the top kk are
// exactly the keys >= T (kk <= number of real keys).  Eight-bit digits from the
// top; the low 32 bits are only examined when keys share T's high half beyond
// what is needed (equal scores).  Per digit: a 256-bin histogram of the keys
// still matching the prefix (LDS integer atomics), then one wave finds the bin
// holding the kk-th key with a suffix scan.
template <int N>
__device__ unsigned long long kth_largest(const unsigned long long (&key)[N], int kk, int* hist, int* sh) {
  const int tid = threadIdx.x, lane = tid & 63;
  unsigned long long prefix = 0ull, mask = 0ull;
  int need = kk;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int b = tid; b < 256; b += blockDim.x) hist[b] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < N; ++u)
      if (key[u] != 0ull && (key[u] & mask) == prefix) atomicAdd(&hist[(key[u] >> shift) & 255], 1);
    __syncthreads();
    if (tid < 64) {
      // lane l owns bins 4l..4l+3; inclusive suffix sums over lanes (bins from the top)
      const int b0 = hist[4 * lane], b1 = hist[4 * lane + 1], b2 = hist[4 * lane + 2], b3 = hist[4 * lane + 3];
      int suf = b0 + b1 + b2 + b3;
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_down(suf, o, 64);
        if (lane + o < 64) suf += v;
      }
      const int above = suf - (b0 + b1 + b2 + b3);    // keys in bins of higher lanes
      if (above < need && suf >= need) {               // the need-th key is in this lane's bins
        int acc = above, d = 4 * lane + 3;
        const int bins[4] = {b0, b1, b2, b3};
        for (int q = 3; q >= 0; --q) {
          d = 4 * lane + q;
          if (acc + bins[q] >= need) break;
          acc += bins[q];
        }
        sh[0] = d;
        sh[1] = acc;                                    // keys above the chosen bin
        sh[2] = bins[d - 4 * lane];                     // keys in the chosen bin
      }
    }
    __syncthreads();
    const int d = sh[0];
    need -= sh[1];
    prefix |= static_cast<unsigned long long>(d) << shift;
    mask |= 255ull << shift;
    const bool done = sh[2] == need;                    // every key with this prefix is taken
    __syncthreads();
    if (done) return prefix;                            // the smallest key with this prefix is >= prefix
  }
  return prefix;
}

// Descending bitonic sort of n (a power of two, <= 2 * blockDim) keys in LDS.
__device__ void bitonic_small(unsigned long long* s, int n) {
  for (int size = 2; size <= n; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < (n >> 1); t += blockDim.x) {
        const int i = 2 * t - (t & (stride - 1));
        const int j = i + stride;
        const bool desc = (i & size) == 0;
        const unsigned long long x = s[i], y = s[j];
        if ((x < y) == desc) { s[i] = y; s[j] = x; }
      }
      __syncthreads();
    }
}

// One key per lane of a wave (lane i: element i), sorted descending by a
// bitonic network of lane exchanges.
__device__ __forceinline__ unsigned long long sort64_desc(unsigned long long v, int lane) {
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1)
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const unsigned long long o = xor_lane_u64(v, stride, lane);
      const bool desc = (lane & size) == 0;
      const bool lower = (lane & stride) == 0;
      v = (lower == desc) ? (v > o ? v : o) : (v < o ? v : o);
    }
  return v;
}

// The 64 largest of a descending 64-key list a and an ascending one rb, one
// key per lane (lane i: element i): their elementwise maximum is bitonic and
// holds them; half-cleaners at strides 32..1 sort it descending.
__device__ __forceinline__ unsigned long long merge_top64(unsigned long long a, unsigned long long rb, int lane) {
  unsigned long long m = a > rb ? a : rb;
#pragma unroll
  for (int st = 32; st > 0; st >>= 1) {
    const unsigned long long o = xor_lane_u64(m, st, lane);
    m = (lane & st) ? (m < o ? m : o) : (m > o ? m : o);
  }
  return m;
}

// Descending sort of n (a power of two) nonzero keys in LDS.  Up to 64 keys one
// wave sorts them in registers (the same bitonic network over 64 lanes, the
// slots past n holding 0, which sorts last): no workgroup barrier per stage.
// Larger n: the workgroup network.
__device__ void sort_small(unsigned long long* s, int n) {
  if (n <= 64) {
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      unsigned long long v = lane < n ? s[lane] : 0ull;
#pragma unroll
      for (int size = 2; size <= 64; size <<= 1)
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
          const unsigned long long o = xor_lane_u64(v, stride, lane);
          const bool desc = (lane & size) == 0;
          const bool lower = (lane & stride) == 0;
          v = (lower == desc) ? (v > o ? v : o) : (v < o ? v : o);
        }
      if (lane < n) s[lane] = v;
    }
    __syncthreads();
    return;
  }
  bitonic_small(s, n);
}

constexpr int kSPer = kSChunk / kVThreads;   // chunk keys per thread

__global__ __launch_bounds__(kVThreads) void k_sample_chunk(VerifyArgs a, SampledScratch sc, int nb, int kk) {
  if (a.batch > 1) {
    a = at_session(a);
    sc = sampled_scratch(a.scratch, a.n_draft, a.vocab);
  }
  __shared__ uint32_t bits[kSChunk / 32];
  __shared__ int hist[256];
  __shared__ int sh[4];
  __shared__ int s_cnt;
  __shared__ unsigned long long s_sel[64];
  __shared__ unsigned long long s_acc[kVThreads / 64][64];
  __shared__ unsigned long long s_floor;
  const int tid = threadIdx.x;
  const int row = blockIdx.y;
  const int n = a.n_draft;
  const bool draft = row > n;
  const int i = draft ? row - (n + 1) : row;            // window index of the row
  const float* src = (draft ? a.draft : a.target) + static_cast<size_t>(i) * a.vocab;
  const int lo = blockIdx.x * kSChunk;
  const int hi = min(a.vocab, lo + kSChunk);
  // the chunk's logits first (all loads in flight), then the window
  float v[kSPer];
#pragma unroll
  for (int u = 0; u < kSPer; ++u) {
    const int k = lo + tid + u * kVThreads;
    v[u] = k < hi ? src[k] : 0.f;
  }
  const bool pen = a.penalty != 1.0f;
  if (pen) {
    const int head = ring_head(a), count = ring_count(a);
    for (int w = tid; w < kSChunk / 32; w += kVThreads) bits[w] = 0u;
    __syncthreads();
    const int total = count + i;
    const int start = total > a.window ? total - a.window : 0;
    for (int t = start + tid; t < total; t += kVThreads) {
      const int tok = window_token(a.ring, head, count, a.window, a.drafts, t);
      if (tok >= lo && tok < hi) atomicOr(&bits[(tok - lo) >> 5], 1u << ((tok - lo) & 31));
    }
    __syncthreads();
  }
  unsigned long long key[kSPer];
#pragma unroll
  for (int u = 0; u < kSPer; ++u) {
    const int t = tid + u * kVThreads;
    const int k = lo + t;
    key[u] = 0ull;                                       // below every real key
    if (k < hi) {
      float x = v[u];
      if (pen && ((bits[t >> 5] >> (t & 31)) & 1u)) x = penalise(x, a.penalty);
      key[u] = argmax_key(x / a.temperature, static_cast<uint32_t>(k));
    }
  }
  const int take = min(kk, hi - lo);
  unsigned long long* out = sc.cand + (static_cast<size_t>(row) * nb + blockIdx.x) * kk;
  if (kk <= 64) {
    // A floor under the take-th largest key: the take-th largest of the 256
    // threads' maxima (at least take keys reach it).  The keys at or above it
    // are usually few: when they fit one wave they are sorted there and the
    // radix select is skipped.
    const int lane = tid & 63, wave = tid >> 6;
    unsigned long long mx = key[0];
#pragma unroll
    for (int u = 1; u < kSPer; ++u) mx = key[u] > mx ? key[u] : mx;
    s_acc[wave][lane] = sort64_desc(mx, lane);
    if (tid == 0) s_cnt = 0;
    __syncthreads();
    if (wave == 0) {
      unsigned long long acc = s_acc[0][lane];
#pragma unroll
      for (int w = 1; w < kVThreads / 64; ++w) acc = merge_top64(acc, s_acc[w][63 - lane], lane);
      if (lane == take - 1) s_floor = acc;
      s_sel[lane] = 0ull;
    }
    __syncthreads();
    const unsigned long long fl = s_floor;
#pragma unroll
    for (int u = 0; u < kSPer; ++u)
      if (key[u] != 0ull && key[u] >= fl) {
        const int pos = atomicAdd(&s_cnt, 1);
        if (pos < 64) s_sel[pos] = key[u];
      }
    __syncthreads();
    if (s_cnt <= 64) {
      sort_small(s_sel, 64);                             // the first `take` are the chunk's top
      if (tid < kk) out[tid] = tid < take ? s_sel[tid] : 0ull;
      return;
    }
    __syncthreads();
  }
  const unsigned long long thr = kth_largest<kSPer>(key, take, hist, sh);
  if (kk <= 64) {
    // the chunk's keys sorted (value desc, id asc; zeros after), so the row
    // kernel merges sorted lists
    if (tid < 64) s_sel[tid] = 0ull;
    if (tid == 0) s_cnt = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kSPer; ++u)
      if (key[u] != 0ull && key[u] >= thr) {             // exactly `take` keys
        const int pos = atomicAdd(&s_cnt, 1);
        if (pos < 64) s_sel[pos] = key[u];
      }
    __syncthreads();
    sort_small(s_sel, 64);
    if (tid < kk) out[tid] = s_sel[tid];
    return;
  }
  if (tid == 0) s_cnt = 0;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kSPer; ++u)
    if (key[u] != 0ull && key[u] >= thr) {                // exactly `take` keys
      const int pos = atomicAdd(&s_cnt, 1);
      if (pos < kk) out[pos] = key[u];
    }
  for (int t = take + tid; t < kk; t += kVThreads) out[t] = 0ull;
}

constexpr int kSRowPer = kSMaxCand / kVThreads;   // merge keys per thread

// The row's top-k (s[0..nv), value desc, id asc) to its support: softmax
// weights, the top-p and min-p prefixes, renormalised, written by token id.
__device__ __forceinline__ void sample_row_tail(const VerifyArgs& a, const SampledScratch& sc, unsigned long long* s,
                                                float* sp, int* s_keep, int nv, int row) {
  const int tid = threadIdx.x;
  if (nv <= 64) {
    // one wave, entry j in lane j: softmax weights, their running sum by a
    // lane scan, the top-p and min-p cuts by ballots (the scores are sorted,
    // so each cut keeps a prefix), and the renormalisation
    if (tid < 64) {
      const int j = tid;
      const float y0 = key_value(s[0]);
      const float yj = j < nv ? key_value(s[j]) : 0.f;
      const float pj = j < nv ? expf(yj - y0) : 0.f;
      float c = pj;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float t = __shfl_up(c, o, 64);
        if (j >= o) c += t;
      }
      const float tot = __shfl(c, nv - 1, 64);
      int keep = nv;
      if (a.top_p < 1.0f) {
        const unsigned long long hit = __ballot(j < nv && c >= a.top_p * tot);
        if (hit) keep = __ffsll(static_cast<long long>(hit));   // first j reaching the mass, plus one
      }
      if (a.min_p > 0.0f) {
        const int m = __popcll(__ballot(j < keep && (yj - y0) >= a.ln_min_p));
        keep = m < keep ? m : keep;
      }
      const float z = __shfl(c, keep - 1, 64);
      const float inv = 1.0f / z;
      if (j < keep) sp[j] = pj * inv;
      if (j == 0) *s_keep = keep;
    }
  } else if (tid == 0) {
    const float y0 = key_value(s[0]);
    float tot = 0.f;
    for (int j = 0; j < nv; ++j) {
      sp[j] = expf(key_value(s[j]) - y0);
      tot += sp[j];
    }
    int keep = nv;
    if (a.top_p < 1.0f) {
      const float target = a.top_p * tot;
      float c = 0.f;
      for (int j = 0; j < nv; ++j) {
        c += sp[j];
        if (c >= target) { keep = j + 1; break; }
      }
    }
    if (a.min_p > 0.0f) {
      int m = 0;
      while (m < keep && (key_value(s[m]) - y0) >= a.ln_min_p) ++m;
      keep = m < keep ? m : keep;
    }
    float z = 0.f;
    for (int j = 0; j < keep; ++j) z += sp[j];
    const float inv = 1.0f / z;
    for (int j = 0; j < keep; ++j) sp[j] *= inv;
    *s_keep = keep;
  }
  __syncthreads();
  const int keep = *s_keep;
  // re-key the kept entries by token id (ascending) with their probability bits
  int k3 = 1;
  while (k3 < keep) k3 <<= 1;
  unsigned long long mine = ~0ull;                       // sorts after every real entry
  if (tid < k3 && tid < keep) {
    const uint32_t id = 0xFFFFFFFFu - static_cast<uint32_t>(s[tid]);
    mine = (static_cast<unsigned long long>(id) << 32) | __float_as_uint(sp[tid]);
  }
  __syncthreads();
  if (tid < k3) s[tid] = ~mine;                          // descending of ~v = ascending of v
  __syncthreads();
  sort_small(s, k3);
  for (int j = tid; j < keep; j += kVThreads) {
    const unsigned long long vv = ~s[j];
    sc.ids[static_cast<size_t>(row) * kSMaxTopK + j] = static_cast<int>(vv >> 32);
    sc.probs[static_cast<size_t>(row) * kSMaxTopK + j] = __uint_as_float(static_cast<uint32_t>(vv));
  }
  if (tid == 0) sc.cnt[row] = keep;
}

__global__ __launch_bounds__(kVThreads) void k_sample_row(VerifyArgs a, SampledScratch sc, int nb, int kk,
                                                         int topk) {
  if (a.batch > 1) {
    a = at_session(a);
    sc = sampled_scratch(a.scratch, a.n_draft, a.vocab);
  }
  __shared__ unsigned long long s[kSMaxTopK];
  __shared__ float sp[kSMaxTopK];
  __shared__ int hist[256];
  __shared__ int sh[4];
  __shared__ int s_keep, s_cnt;
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int ncand = nb * kk;
  const unsigned long long* cand = sc.cand + static_cast<size_t>(row) * ncand;
  if (kk <= 64 && topk <= 64) {
    // The chunks' candidate lists are sorted: wave w folds lists w, w + 4, ...
    // into a running top 64 (a list per merge, sixteen lists' loads in flight),
    // then wave 0 folds the four waves' lists.  The row's top-k is a prefix.
    __shared__ unsigned long long s_acc[kVThreads / 64][64];
    const int lane = tid & 63, wave = tid >> 6;
    unsigned long long acc = 0ull;
    constexpr int kL = 16;                              // lists per wave per round trip
    for (int c0 = wave; c0 < nb; c0 += kL * (kVThreads / 64)) {
      unsigned long long l[kL];
#pragma unroll
      for (int q = 0; q < kL; ++q) {
        const int c = c0 + q * (kVThreads / 64);
        const int e = 63 - lane;                        // the list reversed: ascending
        l[q] = (c < nb && e < kk) ? cand[static_cast<size_t>(c) * kk + e] : 0ull;
      }
#pragma unroll
      for (int q = 0; q < kL; ++q)
        if (c0 + q * (kVThreads / 64) < nb) acc = merge_top64(acc, l[q], lane);
    }
    s_acc[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 1; w < kVThreads / 64; ++w) acc = merge_top64(acc, s_acc[w][63 - lane], lane);
      s[lane] = acc;
      const int nreal = __popcll(__ballot(acc != 0ull));
      if (lane == 0) s_cnt = nreal;
    }
    __syncthreads();
    sample_row_tail(a, sc, s, sp, &s_keep, min(topk, s_cnt), row);
    return;
  }
  unsigned long long key[kSRowPer];
  int nreal = 0;
#pragma unroll
  for (int u = 0; u < kSRowPer; ++u) {
    const int t = tid + u * kVThreads;
    key[u] = t < ncand ? cand[t] : 0ull;
    nreal += key[u] != 0ull;
  }
  // real candidates in the row (<= vocab); the exact top-k of them
  nreal = wave_sum(static_cast<float>(nreal)) + 0.5f;   // small integers: exact in fp32
  if ((tid & 63) == 0) hist[tid >> 6] = nreal;
  __syncthreads();
  int total = 0;
  for (int w = 0; w < kVThreads / 64; ++w) total += hist[w];
  __syncthreads();
  const int nv = min(topk, total);
  const unsigned long long thr = kth_largest<kSRowPer>(key, nv, hist, sh);
  int k2 = 1;
  while (k2 < nv) k2 <<= 1;
  for (int t = tid; t < k2; t += kVThreads) s[t] = 0ull;
  if (tid == 0) s_cnt = 0;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kSRowPer; ++u)
    if (key[u] != 0ull && key[u] >= thr) {                // exactly nv keys
      const int pos = atomicAdd(&s_cnt, 1);
      if (pos < k2) s[pos] = key[u];
    }
  __syncthreads();
  sort_small(s, k2);                                     // the top-k by (value desc, id asc)
  sample_row_tail(a, sc, s, sp, &s_keep, nv, row);
}

__device__ float prob_in(const SampledScratch& sc, int row, int tok) {
  const int* ids = sc.ids + static_cast<size_t>(row) * kSMaxTopK;
  int lo = 0, hi = sc.cnt[row];
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (ids[mid] < tok) lo = mid + 1; else hi = mid;
  }
  return (lo < sc.cnt[row] && ids[lo] == tok) ? sc.probs[static_cast<size_t>(row) * kSMaxTopK + lo] : 0.f;
}

// Inverse CDF over the ascending-id union of rows ra and rb with weight
// max(0, p_a - p_b) (rb < 0: weight p_a): first id whose running sum exceeds
// u * total; the last positive-weight id if none does.  Returns -1 if total is 0.
__device__ int draw(const SampledScratch& sc, int ra, int rb, float u) {
  const int* ia = sc.ids + static_cast<size_t>(ra) * kSMaxTopK;
  const float* pa = sc.probs + static_cast<size_t>(ra) * kSMaxTopK;
  const int na = sc.cnt[ra];
  const int* ib = rb >= 0 ? sc.ids + static_cast<size_t>(rb) * kSMaxTopK : nullptr;
  const float* pb = rb >= 0 ? sc.probs + static_cast<size_t>(rb) * kSMaxTopK : nullptr;
  const int nbb = rb >= 0 ? sc.cnt[rb] : 0;
  // tokens only in row b have weight max(0, 0 - q) = 0: walk row a's ids only
  float total = 0.f;
  for (int x = 0, y = 0; x < na; ++x) {
    while (y < nbb && ib[y] < ia[x]) ++y;
    const float q = (y < nbb && ib[y] == ia[x]) ? pb[y] : 0.f;
    total += fmaxf(pa[x] - q, 0.f);
  }
  if (!(total > 0.f)) return -1;
  const float t = u * total;
  float cum = 0.f;
  int last = -1;
  for (int x = 0, y = 0; x < na; ++x) {
    while (y < nbb && ib[y] < ia[x]) ++y;
    const float q = (y < nbb && ib[y] == ia[x]) ? pb[y] : 0.f;
    const float w = fmaxf(pa[x] - q, 0.f);
    cum += w;
    if (w > 0.f) last = ia[x];
    if (t < cum) return ia[x];
  }
  return last;
}

__global__ void k_sample_decide(VerifyArgs a, SampledScratch sc) {
  if (a.batch > 1) {
    a = at_session(a);
    sc = sampled_scratch(a.scratch, a.n_draft, a.vocab);
  }
  if (threadIdx.x != 0) return;
  const KvWords w = load_kv_words(a);
  const int n = a.n_draft;
  int k = n, tok = -1;
  for (int i = 0; i < n; ++i) {
    const int d = a.drafts[i];
    const float p = prob_in(sc, i, d);
    const float q = prob_in(sc, n + 1 + i, d);
    if (a.uniforms[i] * q < p) continue;
    k = i;
    tok = draw(sc, i, n + 1 + i, a.uniforms[n]);
    if (tok < 0) tok = draw(sc, i, -1, a.uniforms[n]);
    break;
  }
  if (k == n) tok = draw(sc, n, -1, a.uniforms[n]);
  commit_round(a, a.drafts, k, tok, w);
}

// ---------------------------------------------------------------------------
// Sampled verification over the whole vocabulary (top_k = 0, or top_k past
// what the per-chunk candidates hold).  The kept set of a row is a prefix of
// its keys in (value desc, id asc) order, the shortest of three prefixes: the
// top_k largest, the shortest whose softmax mass (over the top-k set) reaches
// top_p, and the values with y - y_max >= ln(min_p) (fp32, as elsewhere).  So
// it is "keys >= T" for T the largest of the three cut keys.
//  F1. k_full_transform (chunks x rows): y = penalise(x) / T into a row buffer,
//      chunk maxima.
//  F2. k_full_select (rows, 1024 threads): y_max; the top-k cut by a radix
//      select on counts; the top-p cut by a radix select on masses, held as
//      integers (exp(y - y_max) in units of 2^-40) so every sum is exact and
//      independent of the order of the atomic adds; the min-p cut from the
//      smallest value that passes; the normaliser over the kept keys in fp64,
//      summed in a fixed order.
//  F3. k_full_decide (1024 threads): the accept tests (one thread), then each
//      draw as a fixed-order parallel inverse CDF over all ids (per-thread
//      id ranges, an exclusive scan of their fp64 sums, one thread walks the
//      range holding u * total).
constexpr int kFThreads = 1024;
constexpr double kFMassScale = 1099511627776.0;   // 2^40

struct FullScratch {
  float* y;                  // [rows][vocab]
  float* cmax;               // [rows][nb]
  float* ymax;               // [rows]
  double* z;                 // [rows] normaliser over the kept keys
  unsigned long long* cut;   // [rows] smallest kept key
};

__host__ __device__ inline FullScratch full_scratch(void* base, int n_draft, int vocab) {
  const int rows = 2 * n_draft + 1;
  const int nb = (vocab + kSChunk - 1) / kSChunk;
  char* p = static_cast<char*>(base);
  FullScratch f;
  f.y = reinterpret_cast<float*>(p);
  p += align256(static_cast<size_t>(rows) * vocab * 4);
  f.cmax = reinterpret_cast<float*>(p);
  p += align256(static_cast<size_t>(rows) * nb * 4);
  f.ymax = reinterpret_cast<float*>(p);
  p += align256(static_cast<size_t>(rows) * 4);
  f.z = reinterpret_cast<double*>(p);
  p += align256(static_cast<size_t>(rows) * 8);
  f.cut = reinterpret_cast<unsigned long long*>(p);
  return f;
}

size_t full_scratch_bytes(int n_draft, int vocab) {
  const size_t rows = 2 * static_cast<size_t>(n_draft) + 1;
  const size_t nb = (static_cast<size_t>(vocab) + kSChunk - 1) / kSChunk;
  return align256(rows * vocab * 4) + align256(rows * nb * 4) + align256(rows * 4) + align256(rows * 8) +
         align256(rows * 8) + 256;
}

__device__ __forceinline__ unsigned long long mass_fx(float y, float ymax) {
  return static_cast<unsigned long long>(static_cast<double>(__expf(y - ymax)) * kFMassScale);
}

__global__ __launch_bounds__(kVThreads) void k_full_transform(VerifyArgs a, FullScratch fs, int nb) {
  if (a.batch > 1) {
    a = at_session(a);
    fs = full_scratch(a.scratch, a.n_draft, a.vocab);
  }
  __shared__ uint32_t bits[kSChunk / 32];
  __shared__ float red[kVThreads / 64];
  const int tid = threadIdx.x;
  const int row = blockIdx.y;
  const int n = a.n_draft;
  const bool draft = row > n;
  const int i = draft ? row - (n + 1) : row;            // window index of the row
  const float* src = (draft ? a.draft : a.target) + static_cast<size_t>(i) * a.vocab;
  const int lo = blockIdx.x * kSChunk;
  const int hi = min(a.vocab, lo + kSChunk);
  float v[kSPer];
#pragma unroll
  for (int u = 0; u < kSPer; ++u) {
    const int k = lo + tid + u * kVThreads;
    v[u] = k < hi ? src[k] : 0.f;
  }
  const bool pen = a.penalty != 1.0f;
  if (pen) {
    const int head = ring_head(a), count = ring_count(a);
    for (int w = tid; w < kSChunk / 32; w += kVThreads) bits[w] = 0u;
    __syncthreads();
    const int total = count + i;
    const int start = total > a.window ? total - a.window : 0;
    for (int t = start + tid; t < total; t += kVThreads) {
      const int tok = window_token(a.ring, head, count, a.window, a.drafts, t);
      if (tok >= lo && tok < hi) atomicOr(&bits[(tok - lo) >> 5], 1u << ((tok - lo) & 31));
    }
    __syncthreads();
  }
  float* y = fs.y + static_cast<size_t>(row) * a.vocab;
  float m = -INFINITY;
#pragma unroll
  for (int u = 0; u < kSPer; ++u) {
    const int t = tid + u * kVThreads;
    const int k = lo + t;
    if (k < hi) {
      float x = v[u];
      if (pen && ((bits[t >> 5] >> (t & 31)) & 1u)) x = penalise(x, a.penalty);
      const float yy = x / a.temperature;
      y[k] = yy;
      m = fmaxf(m, yy);
    }
  }
  m = wave_max(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    float r = red[0];
    for (int w = 1; w < kVThreads / 64; ++w) r = fmaxf(r, red[w]);
    fs.cmax[static_cast<size_t>(row) * nb + blockIdx.x] = r;
  }
}

__device__ __forceinline__ unsigned long long shfl_down_u64(unsigned long long v, int o) {
  const uint32_t lo = __shfl_down(static_cast<uint32_t>(v), o, 64);
  const uint32_t hi = __shfl_down(static_cast<uint32_t>(v >> 32), o, 64);
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// Radix select over the row's keys at or above `floor`: the largest key T with
// (sum over keys >= T of c(key)) >= need, c = 1 (MASS false) or the integer
// mass (MASS true).  Eight-bit digits from the top; counts stop early once the
// chosen bin is exactly used up.
template <bool MASS>
__device__ unsigned long long row_select(const float* y, int vocab, float ymax, unsigned long long floor,
                                         double need, unsigned long long* hist, unsigned long long* sh) {
  const int tid = threadIdx.x, lane = tid & 63;
  unsigned long long prefix = 0ull, mask = 0ull;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int b = tid; b < 256; b += kFThreads) hist[b] = 0ull;
    __syncthreads();
    for (int j = tid; j < vocab; j += kFThreads) {
      const float yy = y[j];
      const unsigned long long key = argmax_key(yy, static_cast<uint32_t>(j));
      if (key >= floor && (key & mask) == prefix)
        atomicAdd(&hist[(key >> shift) & 255], MASS ? mass_fx(yy, ymax) : 1ull);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns bins 4l..4l+3; inclusive suffix sums over lanes (bins from the top)
      const unsigned long long b0 = hist[4 * lane], b1 = hist[4 * lane + 1], b2 = hist[4 * lane + 2],
                               b3 = hist[4 * lane + 3];
      unsigned long long suf = b0 + b1 + b2 + b3;
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long v = shfl_down_u64(suf, o);
        if (lane + o < 64) suf += v;
      }
      const unsigned long long above = suf - (b0 + b1 + b2 + b3);
      const bool last = lane == 0;   // lane 0 takes the remainder if rounding leaves need unmet
      if ((static_cast<double>(above) < need && static_cast<double>(suf) >= need) ||
          (last && static_cast<double>(suf) < need)) {
        const unsigned long long bins[4] = {b0, b1, b2, b3};
        unsigned long long acc = above;
        int d = 4 * lane;
        for (int q = 3; q >= 0; --q) {
          d = 4 * lane + q;
          if (static_cast<double>(acc + bins[q]) >= need) break;
          if (q == 0) break;
          acc += bins[q];
        }
        sh[0] = static_cast<unsigned long long>(d);
        sh[1] = acc;                                   // content of the bins above the chosen one
        sh[2] = bins[d - 4 * lane];                    // content of the chosen bin
      }
    }
    __syncthreads();
    const int d = static_cast<int>(sh[0]);
    need -= static_cast<double>(sh[1]);
    prefix |= static_cast<unsigned long long>(d) << shift;
    mask |= 255ull << shift;
    const bool done = !MASS && static_cast<double>(sh[2]) == need;
    __syncthreads();
    if (done) return prefix;
  }
  return prefix;
}

__device__ double block_sum_f64(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < kFThreads / 64; ++w) t += red[w];
  return t;
}

__global__ __launch_bounds__(kFThreads) void k_full_select(VerifyArgs a, FullScratch fs, int nb) {
  if (a.batch > 1) {
    a = at_session(a);
    fs = full_scratch(a.scratch, a.n_draft, a.vocab);
  }
  __shared__ unsigned long long hist[256];
  __shared__ unsigned long long sh[4];
  __shared__ double red[kFThreads / 64];
  __shared__ float fred[kFThreads / 64];
  __shared__ unsigned long long ured[kFThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x;
  const int V = a.vocab;
  const float* y = fs.y + static_cast<size_t>(row) * V;
  // y_max over the chunk maxima
  float m = -INFINITY;
  for (int c = tid; c < nb; c += kFThreads) m = fmaxf(m, fs.cmax[static_cast<size_t>(row) * nb + c]);
  m = wave_max(m);
  if (lane == 0) fred[wave] = m;
  __syncthreads();
  float ymax = fred[0];
  for (int w = 1; w < kFThreads / 64; ++w) ymax = fmaxf(ymax, fred[w]);
  __syncthreads();
  // top-k cut
  const int kk = (a.top_k > 0 && a.top_k < V) ? a.top_k : V;
  const unsigned long long tk = kk < V ? row_select<false>(y, V, ymax, 0ull, static_cast<double>(kk), hist, sh) : 0ull;
  // top-p cut within the top-k set
  unsigned long long tp = 0ull;
  if (a.top_p < 1.0f) {
    unsigned long long zk = 0ull;
    for (int j = tid; j < V; j += kFThreads) {
      const float yy = y[j];
      if (argmax_key(yy, static_cast<uint32_t>(j)) >= tk) zk += mass_fx(yy, ymax);
    }
    for (int o = 32; o > 0; o >>= 1) zk += __shfl_xor(zk, o, 64);
    __syncthreads();
    if (lane == 0) ured[wave] = zk;
    __syncthreads();
    unsigned long long tot = 0ull;
    for (int w = 0; w < kFThreads / 64; ++w) tot += ured[w];
    __syncthreads();
    tp = row_select<true>(y, V, ymax, tk, static_cast<double>(a.top_p) * static_cast<double>(tot), hist, sh);
  }
  // min-p cut: every value >= the smallest one with y - y_max >= ln(min_p)
  unsigned long long tm = 0ull;
  if (a.min_p > 0.0f) {
    float lo = INFINITY;
    for (int j = tid; j < V; j += kFThreads) {
      const float yy = y[j];
      if ((yy - ymax) >= a.ln_min_p) lo = fminf(lo, yy);
    }
    for (int o = 32; o > 0; o >>= 1) lo = fminf(lo, __shfl_xor(lo, o, 64));
    __syncthreads();
    if (lane == 0) fred[wave] = lo;
    __syncthreads();
    float v = fred[0];
    for (int w = 1; w < kFThreads / 64; ++w) v = fminf(v, fred[w]);
    tm = static_cast<unsigned long long>(ord_key(v)) << 32;
  }
  const unsigned long long cut = max(tk, max(tp, tm));
  // normaliser over the kept keys (fp64; per-thread then fixed-order block sum)
  double z = 0.0;
  for (int j = tid; j < V; j += kFThreads) {
    const float yy = y[j];
    if (argmax_key(yy, static_cast<uint32_t>(j)) >= cut) z += static_cast<double>(__expf(yy - ymax));
  }
  z = block_sum_f64(z, red);
  if (tid == 0) {
    fs.ymax[row] = ymax;
    fs.z[row] = z;
    fs.cut[row] = cut;
  }
}

__device__ __forceinline__ double full_prob(const VerifyArgs& a, const FullScratch& fs, int row, int tok) {
  if (tok < 0 || tok >= a.vocab) return 0.0;             // a draft id outside the vocabulary has no mass
  const float yy = fs.y[static_cast<size_t>(row) * a.vocab + tok];
  if (argmax_key(yy, static_cast<uint32_t>(tok)) < fs.cut[row]) return 0.0;
  return static_cast<double>(__expf(yy - fs.ymax[row])) / fs.z[row];
}

// Inverse CDF over ids ascending with weight max(0, p_a - p_b) (rb < 0: p_a):
// the first id whose running sum exceeds u * total, else the last positive-
// weight id; -1 if the total is 0.  Every thread of the block calls it.
// Thread i sums the ids of its contiguous range; the range offsets are
// sequential sums (within each wave, then over the waves), so they never
// decrease and exactly one thread's [offset, next offset) holds u * total.
struct DrawShared {
  double sum[kFThreads];     // per-thread weight sums, then exclusive offsets
  double wbase[kFThreads / 64 + 1];
  int res[2];                // claimed id, last positive-weight id
};

__device__ int full_draw(const VerifyArgs& a, const FullScratch& fs, int ra, int rb, float u, DrawShared& ds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int kW = kFThreads / 64;
  const int V = a.vocab;
  const int per = (V + kFThreads - 1) / kFThreads;
  const int j0 = min(V, tid * per), j1 = min(V, j0 + per);
  auto weight = [&](int x) {
    const double pa = full_prob(a, fs, ra, x);
    const double pb = rb >= 0 ? full_prob(a, fs, rb, x) : 0.0;
    return fmax(pa - pb, 0.0);
  };
  double s = 0.0;
  int lastpos = -1;
  for (int x = j0; x < j1; ++x) {
    const double w = weight(x);
    s += w;
    if (w > 0.0) lastpos = x;
  }
  __syncthreads();                                     // ds is free (a previous draw may have used it)
  ds.sum[tid] = s;
  if (tid == 0) { ds.res[0] = -1; ds.res[1] = -1; }
  __syncthreads();
  if (lane == 0) {                                     // wave-local exclusive offsets, in order
    double c = 0.0;
    for (int l = 0; l < 64; ++l) {
      const double v = ds.sum[wave * 64 + l];
      ds.sum[wave * 64 + l] = c;
      c += v;
    }
    ds.wbase[wave + 1] = c;                            // the wave's total, for now
  }
  __syncthreads();
  if (tid == 0) {
    double c = 0.0;
    for (int w = 0; w < kW; ++w) {
      const double t = ds.wbase[w + 1];
      ds.wbase[w] = c;
      c += t;
    }
    ds.wbase[kW] = c;                                  // the total
  }
  __syncthreads();
  const double total = ds.wbase[kW];
  const double off = ds.wbase[wave] + ds.sum[tid];
  const double next = lane < 63 ? ds.wbase[wave] + ds.sum[tid + 1] : ds.wbase[wave + 1];
  if (lastpos >= 0) atomicMax(&ds.res[1], lastpos);
  __syncthreads();
  if (!(total > 0.0)) return -1;                       // the same in every thread
  const double t = static_cast<double>(u) * total;
  if (off <= t && t < next) {                          // at most one thread
    const double tau = t - off;
    double r = 0.0;
    int pick = lastpos;
    for (int x = j0; x < j1; ++x) {
      r += weight(x);
      if (tau < r) { pick = x; break; }
    }
    ds.res[0] = pick;
  }
  __syncthreads();
  return ds.res[0] >= 0 ? ds.res[0] : ds.res[1];
}

__global__ __launch_bounds__(kFThreads) void k_full_decide(VerifyArgs a, FullScratch fs) {
  if (a.batch > 1) {
    a = at_session(a);
    fs = full_scratch(a.scratch, a.n_draft, a.vocab);
  }
  __shared__ DrawShared ds;
  __shared__ int s_k;
  const int n = a.n_draft;
  const KvWords w = threadIdx.x == 0 ? load_kv_words(a) : KvWords{0, 0, 0, 0};
  if (threadIdx.x == 0) {
    int k = n;
    for (int i = 0; i < n; ++i) {
      const int d = a.drafts[i];
      const double p = full_prob(a, fs, i, d);
      const double q = full_prob(a, fs, n + 1 + i, d);
      if (static_cast<double>(a.uniforms[i]) * q < p) continue;
      k = i;
      break;
    }
    s_k = k;
  }
  __syncthreads();
  const int k = s_k;
  int tok;
  if (k < n) {
    tok = full_draw(a, fs, k, n + 1 + k, a.uniforms[n], ds);
    if (tok < 0) tok = full_draw(a, fs, k, -1, a.uniforms[n], ds);
  } else {
    tok = full_draw(a, fs, n, -1, a.uniforms[n], ds);
  }
  if (threadIdx.x != 0) return;
  commit_round(a, a.drafts, k, tok, w);
}

// the per-chunk candidate path holds the top_k keys of every chunk
static bool radix_path(int top_k, int vocab) {
  const int nb = (vocab + kSChunk - 1) / kSChunk;
  return top_k >= 1 && top_k <= kSMaxTopK && static_cast<long>(nb) * (top_k < kSChunk ? top_k : kSChunk) <= kSMaxCand;
}

bool verify_sampled_supported(int top_k, int vocab) { return top_k >= 0 && vocab >= 1; }

hipError_t launch_verify_sampled(const VerifyArgs& a, hipStream_t s) {
  if (!verify_sampled_supported(a.top_k, a.vocab)) return hipErrorNotSupported;
  const int rows = 2 * a.n_draft + 1;
  const int nb = (a.vocab + kSChunk - 1) / kSChunk;
  const unsigned bz = a.batch > 1 ? a.batch : 1;
  if (!radix_path(a.top_k, a.vocab)) {
    const FullScratch fs = full_scratch(a.scratch, a.n_draft, a.vocab);
    (void)hipGetLastError();
    int slot = -1;
    time_mark(TIME_VERIFY, true, s, &slot);
    hipLaunchKernelGGL(k_full_transform, dim3(nb, rows, bz), dim3(kVThreads), 0, s, a, fs, nb);
    time_mark(TIME_VERIFY, false, s, &slot);
    hipLaunchKernelGGL(k_full_select, dim3(rows, 1, bz), dim3(kFThreads), 0, s, a, fs, nb);
    hipLaunchKernelGGL(k_full_decide, dim3(1, 1, bz), dim3(kFThreads), 0, s, a, fs);
    return hipGetLastError();
  }
  const int kk = a.top_k < kSChunk ? a.top_k : kSChunk;
  const SampledScratch sc = sampled_scratch(a.scratch, a.n_draft, a.vocab);
  (void)hipGetLastError();
  int slot = -1;
  time_mark(TIME_VERIFY, true, s, &slot);
  hipLaunchKernelGGL(k_sample_chunk, dim3(nb, rows, bz), dim3(kVThreads), 0, s, a, sc, nb, kk);
  time_mark(TIME_VERIFY, false, s, &slot);
  hipLaunchKernelGGL(k_sample_row, dim3(rows, 1, bz), dim3(kVThreads), 0, s, a, sc, nb, kk, a.top_k);
  hipLaunchKernelGGL(k_sample_decide, dim3(1, 1, bz), dim3(64), 0, s, a, sc);
  return hipGetLastError();
}

}  // namespace mtp
