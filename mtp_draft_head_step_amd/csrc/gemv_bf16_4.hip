// Instantiations of the weight-streaming GEMV launches: bf16 weights, four to sixteen activation rows.
#include "gemv_impl.h"

namespace mtp {
template hipError_t launch_r<W_BF16, 4>(const GemvArgs&, hipStream_t, int*);
template hipError_t launch_r<W_BF16, 8>(const GemvArgs&, hipStream_t, int*);
template hipError_t launch_r<W_BF16, 16>(const GemvArgs&, hipStream_t, int*);
}  // namespace mtp
