// Run-time-hidden rmsnorm_fwd kernels (every access width, lane count and per-lane
// access count) and their launch table.
#include "kernels_fwd_dyn.hpp"

namespace rownorm {

const std::vector<DynFwdEntry>& rmsnorm_fwd_dyn_table() {
    static const std::vector<DynFwdEntry> table = build_dyn_fwd_table<OpRmsDyn>();
    return table;
}

}  // namespace rownorm
