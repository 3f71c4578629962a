#include "moe_internal.h"
namespace moe {
hipError_t launch_prefill_experts(const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }
}
