// Draft-KV rollback (O(1): only the device length word moves) and the
// workspace fill kernel (used instead of a memset so callers may capture it).
#include "common.h"
#include "kernels.h"

namespace mtp {

__global__ void k_rollback(int32_t* st, int to_len, const int32_t* n_acc, int n_draft) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  if (st[3] != 0) return;
  int to = to_len;
  if (to_len < 0) {
    to = st[1];
    if (n_acc) {
      const int keep_max = n_draft > 0 ? n_draft - 1 : 0;
      int k = *n_acc;
      k = k < 0 ? 0 : k;
      to += k < keep_max ? k : keep_max;
    }
  }
  if (to < 0 || to > st[0]) {
    st[3] = 2;
    return;
  }
  st[0] = to;
}

hipError_t launch_rollback(int32_t* state, int to_len, const int32_t* n_acc, int n_draft,
                           int capacity, hipStream_t s) {
  (void)capacity;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_rollback, dim3(1), dim3(64), 0, s, state, to_len, n_acc, n_draft);
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
