// Draft-KV rollback (O(1): only the device length word moves) and the
// workspace fill kernel (used instead of a memset so callers may capture it).
#include "common.h"
#include "kernels.h"

namespace mtp {

// Thread b rolls back session b (state words st + 4 b; its accepted count, when
// given, n_acc[b * acc_stride]).
__global__ void k_rollback(int32_t* st0, int to_len, const int32_t* n_acc0, int n_draft, int batch,
                           int acc_stride) {
  const int b = threadIdx.x;
  if (blockIdx.x != 0 || b >= batch) return;
  int32_t* st = st0 + 4 * b;
  const int32_t* n_acc = n_acc0 ? n_acc0 + b * acc_stride : nullptr;
  // every load first (one memory round trip)
  const int err0 = st[3], len0 = st[0], base0 = st[1];
  const int k0 = n_acc ? *n_acc : 0;
  if (err0 != 0) return;
  const int to = rollback_length(to_len, len0, base0, k0, n_acc != nullptr, n_draft);
  if (to < 0) {
    st[3] = 2;
    return;
  }
  st[0] = to;
}

hipError_t launch_rollback(int32_t* state, int to_len, const int32_t* n_acc, int n_draft,
                           int capacity, hipStream_t s, int batch, int acc_stride) {
  (void)capacity;
  if (batch < 1 || batch > 64) return hipErrorInvalidValue;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_rollback, dim3(1), dim3(64), 0, s, state, to_len, n_acc, n_draft, batch, acc_stride);
  return hipGetLastError();
}

// Policy-B re-pairing: with k = out_counts[0] (brought into [0, n_draft]) and
// j0 = min(k, n_draft - 1), pending pair j = 0..k - j0 is (out_tokens[j0 + j],
// hidden row j0 + j); the count k + 1 - j0 goes to *pend_count.  Rows are
// copied in 16-bit units (elems16 per row).
// Workgroup b re-pairs session b (its rows of every array, n_draft + 1 rows each).
__global__ void k_repair(const int32_t* out_tokens, const int32_t* out_counts, const uint16_t* hid, int elems16,
                         int n_draft, int32_t* pend_tokens, uint16_t* pend_hid, int32_t* pend_count) {
  const size_t b = blockIdx.x, rows = n_draft + 1;
  out_tokens += b * rows;
  out_counts += 2 * b;
  hid += b * rows * elems16;
  pend_tokens += b * rows;
  pend_hid += b * rows * elems16;
  pend_count += b;
  int k = out_counts[0];
  k = k < 0 ? 0 : (k > n_draft ? n_draft : k);
  const int j0 = n_draft > 0 ? (k < n_draft - 1 ? k : n_draft - 1) : 0;
  const int cnt = k + 1 - j0;
  for (int j = 0; j < cnt; ++j) {
    const uint16_t* src = hid + static_cast<size_t>(j0 + j) * elems16;
    uint16_t* dst = pend_hid + static_cast<size_t>(j) * elems16;
    for (int e = threadIdx.x; e < elems16; e += blockDim.x) dst[e] = src[e];
  }
  if (threadIdx.x < cnt) pend_tokens[threadIdx.x] = out_tokens[j0 + threadIdx.x];
  if (threadIdx.x == 0) *pend_count = cnt;
}

hipError_t launch_repair(const int32_t* out_tokens, const int32_t* out_counts, const void* hid, int elems16,
                         int n_draft, int32_t* pend_tokens, void* pend_hid, int32_t* pend_count, hipStream_t s,
                         int batch) {
  if (batch < 1) return hipErrorInvalidValue;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_repair, dim3(batch), dim3(256), 0, s, out_tokens, out_counts, static_cast<const uint16_t*>(hid),
                     elems16, n_draft, pend_tokens, static_cast<uint16_t*>(pend_hid), pend_count);
  return hipGetLastError();
}

__global__ void k_fill_zero(uint4* p, size_t n16, unsigned char* tail, size_t ntail) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  const size_t ntail = bytes - n16 * 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) blocks = 1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_fill_zero, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<uint4*>(p), n16, static_cast<unsigned char*>(p) + n16 * 16, ntail);
  return hipGetLastError();
}

}  // namespace mtp
