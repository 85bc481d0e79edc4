// Route kernel instances of one score variant (kVarSigmoid); see route_kernel.hpp.
#include "route_kernel.hpp"

namespace moe {
template hipError_t launch_route_variant<kVarSigmoid>(const RouteParams&, int, int, bool, int,
                                                hipStream_t);
}  // namespace moe
