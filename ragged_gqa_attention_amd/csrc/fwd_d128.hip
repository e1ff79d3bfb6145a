// Forward kernels for head dimension 128 (see fwd_impl.hpp).
#include "fwd_impl.hpp"

namespace rga {
template hipError_t launch_fwd_d<128>(const AttnArgs&, const PlanArgs&, int, bool, bool,
                                     hipStream_t);
}  // namespace rga
