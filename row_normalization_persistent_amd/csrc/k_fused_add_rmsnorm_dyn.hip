// Run-time-hidden fused_add_rmsnorm kernels (every access width, lane count and per-lane
// access count) and their launch table.
#include "kernels_fwd_dyn.hpp"

namespace rownorm {

const std::vector<DynFwdEntry>& fused_add_rmsnorm_dyn_table() {
    static const std::vector<DynFwdEntry> table = build_dyn_fwd_table<OpFusedDyn>();
    return table;
}

}  // namespace rownorm
