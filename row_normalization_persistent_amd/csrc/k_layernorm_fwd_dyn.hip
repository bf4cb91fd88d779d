// Run-time-hidden layernorm_fwd kernels (every access width, lane count and per-lane
// access count) and their launch table.
#include "kernels_fwd_dyn.hpp"

namespace rownorm {

const std::vector<DynFwdEntry>& layernorm_fwd_dyn_table() {
    static const std::vector<DynFwdEntry> table = build_dyn_fwd_table<OpLnFwdDyn>();
    return table;
}

}  // namespace rownorm
