// Instantiations of the weight-streaming GEMV launches: fp32 weights, 1..16 activation rows.
#include "gemv_impl.h"

namespace mtp {
template hipError_t launch_r<W_F32, 1>(const GemvArgs&, hipStream_t, int*);
template hipError_t launch_r<W_F32, 2>(const GemvArgs&, hipStream_t, int*);
template hipError_t launch_r<W_F32, 3>(const GemvArgs&, hipStream_t, int*);
template hipError_t launch_r<W_F32, 4>(const GemvArgs&, hipStream_t, int*);
template hipError_t launch_r<W_F32, 8>(const GemvArgs&, hipStream_t, int*);
template hipError_t launch_r<W_F32, 16>(const GemvArgs&, hipStream_t, int*);
}  // namespace mtp
