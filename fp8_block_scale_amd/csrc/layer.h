// Steps 1-5 in one call (moe_fp8_layer): the plan's one-workgroup launch
// also clears what the gate/up stage would otherwise clear in a launch of
// its own -- the route map (to -1) and the split-K arrival counters (to 0).
#pragma once

#include "internal.h"

namespace moe {

struct ClearJob {
    uint32_t *rpos;     // [nr] set to 0xffffffff
    size_t nr;
    uint32_t *cnt;      // [nc] set to 0
    size_t nc;
};

// launch_plan_quant's one-workgroup form (no plan workspace, or fewer routes
// than the several-workgroup build takes) with the clearing of c done by
// extra workgroups of the same launch.
hipError_t launch_plan_quant_clear(const void *ids, bool ids_i64, int64_t R, int E, int block_m,
                                   int32_t *sorted, int32_t *expert_ids, int32_t *ntp,
                                   const QuantJob &q, bool ue8m0, const ClearJob &c, hipStream_t st);

}  // namespace moe
