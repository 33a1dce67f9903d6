// Instantiations of the weight-streaming GEMV launches: bf16 weights, two and three activation rows.
#include "gemv_impl.h"

namespace mtp {
template hipError_t launch_r<W_BF16, 2>(const GemvArgs&, hipStream_t, int*);
template hipError_t launch_r<W_BF16, 3>(const GemvArgs&, hipStream_t, int*);
}  // namespace mtp
