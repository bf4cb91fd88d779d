// Backward kernels for rows wider than the register-resident layout holds
// (LayerNorm, RMSNorm, fused residual-add + RMSNorm; 5 to 8 16-byte accesses a
// lane at 512 lanes): the bf16 launch tables and the fp32 launcher.
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

template <bool LN>
hipError_t wide_f32_by_vecs(const DynBwdArgs& a, hipStream_t stream) {
    switch (wide_vecs_f32(a.hidden)) {
        case 5: return launch_bwd_wide<5, LN, float>(a, stream);
        case 6: return launch_bwd_wide<6, LN, float>(a, stream);
        case 7: return launch_bwd_wide<7, LN, float>(a, stream);
        case 8: return launch_bwd_wide<8, LN, float>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bwd_wide_f32(bool ln, const DynBwdArgs& a, hipStream_t stream) {
    return ln ? wide_f32_by_vecs<true>(a, stream) : wide_f32_by_vecs<false>(a, stream);
}

}  // namespace rownorm
