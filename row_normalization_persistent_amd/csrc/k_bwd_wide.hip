// Backward kernels for rows wider than the register-resident layout holds
// (LayerNorm, RMSNorm, fused residual-add + RMSNorm; 3 to 8 16-byte accesses a
// lane at 1024 lanes) and their launch tables.
#include "kernels_bwd_wide.hpp"

namespace rownorm {

namespace {
template <bool LN, int... Vs>
std::vector<WideBwdEntry> wide_table(std::integer_sequence<int, Vs...>) {
    return {WideBwdEntry{Vs, &launch_bwd_wide<Vs, LN>}...};
}
}  // namespace

const std::vector<WideBwdEntry>& layernorm_bwd_wide_table() {
    static const std::vector<WideBwdEntry> t = wide_table<true>(WideVecsLn{});
    return t;
}

const std::vector<WideBwdEntry>& rmsnorm_bwd_wide_table() {
    static const std::vector<WideBwdEntry> t = wide_table<false>(WideVecsRms{});
    return t;
}

}  // namespace rownorm
