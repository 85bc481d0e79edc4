// gfx950 kernels for the fused decode front end (RMSNorm -> router projection
// -> top-k on raw logits -> activation); see rmsnorm_gate_route in moe_route.h.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"
