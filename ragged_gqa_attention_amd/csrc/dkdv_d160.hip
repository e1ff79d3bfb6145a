// dK / dV kernels for head dimension 160 (see dkdv_impl.hpp).
#include "dkdv_impl.hpp"

namespace rga {
template hipError_t launch_dkdv_d<160>(const AttnArgs&, int, bool, int, hipStream_t);
}  // namespace rga
