// Run-time-hidden LayerNorm backward row kernels and their launch table.
#include "kernels_bwd_dyn.hpp"

namespace rownorm {

const std::vector<DynBwdEntry>& layernorm_bwd_dyn_table() {
    static const std::vector<DynBwdEntry> table = build_dyn_bwd_table<true>();
    return table;
}

}  // namespace rownorm
