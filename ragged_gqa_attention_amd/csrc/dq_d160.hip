// dQ kernels for head dimension 160 (see dq_impl.hpp).
#include "dq_impl.hpp"

namespace rga {
template hipError_t launch_dq_d<160>(const AttnArgs&, int, bool, int, hipStream_t);
}  // namespace rga
