// Compiled shapes of LayerNorm forward.
#include "kernels_fwd.hpp"

namespace rownorm {
const std::vector<FwdEntry>& layernorm_fwd_table() {
    static const std::vector<FwdEntry> table = build_fwd_table<OpLnFwd>();
    return table;
}
}  // namespace rownorm
