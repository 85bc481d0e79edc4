// Route kernel instances of one score variant (kVarSoftmax); see route_kernel.hpp.
#include "route_kernel.hpp"

namespace moe {
template hipError_t launch_route_variant<kVarSoftmax>(const RouteParams&, int, int, bool, int,
                                                hipStream_t);
}  // namespace moe
