// dQ kernels for head dimension 128 (see dq_impl.hpp).
#include "dq_impl.hpp"

namespace rga {
template hipError_t launch_dq_d<128>(const AttnArgs&, int, bool, int, hipStream_t);
}  // namespace rga
