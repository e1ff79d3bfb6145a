// Forward kernels for head dimension 160 (see fwd_impl.hpp).
#include "fwd_impl.hpp"

namespace rga {
template hipError_t launch_fwd_d<160>(const AttnArgs&, const PlanArgs&, int, bool, bool,
                                     hipStream_t);
}  // namespace rga
