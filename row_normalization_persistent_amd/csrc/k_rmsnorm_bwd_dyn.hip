// Run-time-hidden RMSNorm backward row kernels (with and without the fused
// residual-add's residual gradient) and their launch table.
#include "kernels_bwd_dyn.hpp"

namespace rownorm {

const std::vector<DynBwdEntry>& rmsnorm_bwd_dyn_table() {
    static const std::vector<DynBwdEntry> table = build_dyn_bwd_table<false>();
    return table;
}

}  // namespace rownorm
