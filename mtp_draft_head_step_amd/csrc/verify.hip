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

__device__ __forceinline__ float penalise(float v, float pen) { return v > 0.f ? v / pen : v * pen; }

__global__ __launch_bounds__(kVThreads) void k_verify_greedy(VerifyArgs a) {
  __shared__ uint32_t bits[kVMaxChunk / 32];
  __shared__ unsigned long long s_best[kVThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = blockIdx.y;
  const int lo = blockIdx.x * a.chunk;
  const int hi = min(a.vocab, lo + a.chunk);
  const bool pen = a.penalty != 1.0f;
  const int head = a.ring_state[0];
  const int count = a.ring_state[1];
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
  const float* row = a.target + static_cast<size_t>(i) * a.vocab;
  unsigned long long best = 0ull;
  for (int k = lo + tid; k < hi; k += kVThreads) {
    float v = row[k];
    if (pen && ((bits[(k - lo) >> 5] >> ((k - lo) & 31)) & 1u)) v = penalise(v, a.penalty);
    const unsigned long long key = argmax_key(v, static_cast<uint32_t>(k));
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

__global__ __launch_bounds__(kVThreads) void k_verify_greedy_finish(VerifyArgs a, int nb) {
  __shared__ int am[MTP_MAX_DRAFT_DEV + 1];
  const int n = a.n_draft;
  for (int r = 0; r <= n; ++r) {
    const unsigned long long b = block_max_u64(a.parts + static_cast<size_t>(r) * nb, nb);
    if (threadIdx.x == 0) am[r] = argmax_index(b);
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  int k = n;
  for (int r = 0; r < n; ++r) {
    if (a.drafts[r] != am[r]) { k = r; break; }
  }
  int h = a.ring_state[0], c = a.ring_state[1];
  for (int r = 0; r <= k; ++r) {
    const int t = r < k ? a.drafts[r] : am[k];
    a.out_tokens[r] = t;
    a.ring[h] = t;
    h = (h + 1) % a.window;
    c = c + 1 < a.window ? c + 1 : a.window;
  }
  a.out_counts[0] = k;
  a.out_counts[1] = k + 1;
  a.ring_state[0] = h;
  a.ring_state[1] = c;
}

hipError_t launch_verify_greedy(const VerifyArgs& a, hipStream_t s) {
  const int nb = (a.vocab + a.chunk - 1) / a.chunk;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_verify_greedy, dim3(nb, a.n_draft + 1), dim3(kVThreads), 0, s, a);
  hipLaunchKernelGGL(k_verify_greedy_finish, dim3(1), dim3(kVThreads), 0, s, a, nb);
  return hipGetLastError();
}

size_t verify_sampled_scratch_bytes(int n_draft, int vocab, int chunk) {
  (void)n_draft; (void)vocab; (void)chunk;
  return 0;
}

hipError_t launch_verify_sampled(const VerifyArgs& a, hipStream_t s) {
  (void)a; (void)s;
  return hipErrorNotSupported;
}

}  // namespace mtp
