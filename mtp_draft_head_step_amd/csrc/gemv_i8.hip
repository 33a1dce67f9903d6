// Instantiations of the weight-streaming GEMV launches: int8-g128 weights (the unembedding), one activation row.
#include "gemv_impl.h"

namespace mtp {
template hipError_t launch_r<W_I8, 1>(const GemvArgs&, hipStream_t, int*);
}  // namespace mtp
