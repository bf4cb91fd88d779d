// Streamed rows (kernels_stream.hpp): the forward of each operation and the
// backward's two kernels, ahead of the shared column reduce.
#include "kernels_stream.hpp"

namespace rownorm {

// Rows of the tile kernel's ring: the deepest that compiles without register
// spills on gfx950 at 512 lanes (256 VGPRs a lane) for 4 accesses a lane.
template <bool LN, bool DRES>
constexpr int tile_depth() { return DRES ? 2 : 3; }

hipError_t launch_stream_fwd(int op, const DynFwdArgs& a, hipStream_t stream) {
    switch (op) {
        case kSplitFused: return launch_stream_fwd_op<kSplitFused>(a, stream);
        case kSplitRms: return launch_stream_fwd_op<kSplitRms>(a, stream);
        case kSplitLn: return launch_stream_fwd_op<kSplitLn>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <bool LN, bool DRES>
hipError_t launch_tiles(const DynBwdArgs& a, const float* stats, int32_t tiles, int32_t walkers,
                        hipStream_t stream) {
    hipLaunchKernelGGL((stream_bwd_tile_kernel<kStreamTileVecs, LN, DRES, tile_depth<LN, DRES>()>),
                       dim3((unsigned)(walkers * tiles)), dim3(kStreamTileLanes), 0, stream, a,
                       stats, (int)tiles);
    return hipGetLastError();
}

hipError_t launch_stream_bwd(bool ln, const DynBwdArgs& a, int32_t tiles, int32_t walkers,
                             hipStream_t stream) {
    const int outs = ln ? 2 : 1;
    const int32_t padded = (int32_t)((a.hidden + 63) / 64 * 64);
    if (a.rows > 0) {
        float* stats = a.workspace + (int64_t)walkers * outs * padded;
        const int64_t grid = a.rows < kStreamMaxGrid ? a.rows : kStreamMaxGrid;
        if (ln)
            hipLaunchKernelGGL((stream_bwd_stats_kernel<true>), dim3((unsigned)grid),
                               dim3(kStreamFwdLanes), 0, stream, a, stats);
        else
            hipLaunchKernelGGL((stream_bwd_stats_kernel<false>), dim3((unsigned)grid),
                               dim3(kStreamFwdLanes), 0, stream, a, stats);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (ln) e = launch_tiles<true, false>(a, stats, tiles, walkers, stream);
        else if (a.dres) e = launch_tiles<false, true>(a, stats, tiles, walkers, stream);
        else e = launch_tiles<false, false>(a, stats, tiles, walkers, stream);
        if (e != hipSuccess) return e;
    }
    return launch_norm_colreduce(a.workspace, a.rows > 0 ? walkers : 0, a.hidden, padded, outs,
                                 a.dweight, a.dbias, stream);
}

}  // namespace rownorm
