// Row-split forward kernels (fused residual-add + RMSNorm, RMSNorm,
// LayerNorm; 1 to 8 16-byte accesses per lane) and their launch table.
#include <utility>

#include "kernels_split.hpp"

namespace rownorm {

namespace {
template <int OP, int... Vs>
void add_split(std::vector<SplitEntry>& v, std::integer_sequence<int, Vs...>) {
    (v.push_back({OP, Vs, &launch_split<Vs, OP>}), ...);
}
}  // namespace

const std::vector<SplitEntry>& split_table() {
    static const std::vector<SplitEntry> table = [] {
        std::vector<SplitEntry> v;
        using Vecs = std::integer_sequence<int, 1, 2, 3, 4, 5, 6, 7, 8>;
        add_split<kSplitFused>(v, Vecs{});
        add_split<kSplitRms>(v, Vecs{});
        add_split<kSplitLn>(v, Vecs{});
        return v;
    }();
    return table;
}

}  // namespace rownorm
