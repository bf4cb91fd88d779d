// Compiled shapes of RMSNorm forward.
#include "kernels_fwd.hpp"

namespace rownorm {
const std::vector<FwdEntry>& rmsnorm_fwd_table() {
    static const std::vector<FwdEntry> table = build_fwd_table<OpRms>();
    return table;
}
}  // namespace rownorm
