// Compiled shapes of fused residual-add + RMSNorm forward.
#include "kernels_fwd.hpp"

namespace rownorm {
const std::vector<FwdEntry>& fused_add_rmsnorm_table() {
    static const std::vector<FwdEntry> table = build_fwd_table<OpFused>();
    return table;
}
}  // namespace rownorm
