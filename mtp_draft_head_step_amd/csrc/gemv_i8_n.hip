// Instantiations of the weight-streaming GEMV launches: int8-g128 weights (the
// unembedding of several sessions), 2..16 activation rows.
#include "gemv_impl.h"

namespace mtp {
template hipError_t launch_r<W_I8, 2>(const GemvArgs&, hipStream_t, int*);
template hipError_t launch_r<W_I8, 3>(const GemvArgs&, hipStream_t, int*);
template hipError_t launch_r<W_I8, 4>(const GemvArgs&, hipStream_t, int*);
template hipError_t launch_r<W_I8, 8>(const GemvArgs&, hipStream_t, int*);
template hipError_t launch_r<W_I8, 16>(const GemvArgs&, hipStream_t, int*);
}  // namespace mtp
