// Instantiations of the weight-streaming GEMV launches: bf16 weights, one activation row.
#include "gemv_impl.h"

namespace mtp {
template hipError_t launch_r<W_BF16, 1>(const GemvArgs&, hipStream_t, int*);
}  // namespace mtp
