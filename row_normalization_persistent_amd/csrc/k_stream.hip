// Streamed rows (kernels_stream.hpp): the forward of each operation and the
// backward's two kernels, ahead of the shared column reduce, for bf16 and
// fp32 activations.
#include <type_traits>

#include <algorithm>

#include "kernels_stream.hpp"
#include "stream_select.hpp"

namespace rownorm {

// Rows of the tile kernel's ring: the deepest that compiles without register
// spills on gfx950 at 512 lanes (256 VGPRs a lane) for 4 accesses a lane.
template <bool LN, bool DRES>
constexpr int tile_depth() { return DRES ? 2 : 3; }

// Only the shapes stream_fwd_shape picks are instantiated.
template <int OP>
hipError_t fwd_f32_rms(const StreamFwdShape& sh, const DynFwdArgs& a, hipStream_t stream) {
    switch (sh.lanes * 100 + sh.unroll) {
        case 6404: return launch_stream_fwd_op<float, OP, 64, 4>(a, stream);
        case 12804: return launch_stream_fwd_op<float, OP, 128, 4>(a, stream);
        case 25604: return launch_stream_fwd_op<float, OP, 256, 4>(a, stream);
        case 51204: return launch_stream_fwd_op<float, OP, 512, 4>(a, stream);
        case 102404: return launch_stream_fwd_op<float, OP, 1024, 4>(a, stream);
        default: return launch_stream_fwd_op<float, OP, 1024, 8>(a, stream);
    }
}

hipError_t fwd_f32_ln(const StreamFwdShape& sh, const DynFwdArgs& a, hipStream_t stream) {
    switch (sh.lanes * 100 + sh.unroll) {
        case 6404: return launch_stream_fwd_op<float, kSplitLn, 64, 4>(a, stream);
        case 6408: return launch_stream_fwd_op<float, kSplitLn, 64, 8>(a, stream);
        case 12808: return launch_stream_fwd_op<float, kSplitLn, 128, 8>(a, stream);
        case 25608: return launch_stream_fwd_op<float, kSplitLn, 256, 8>(a, stream);
        case 51208: return launch_stream_fwd_op<float, kSplitLn, 512, 8>(a, stream);
        default: return launch_stream_fwd_op<float, kSplitLn, 1024, 4>(a, stream);
    }
}

// fp32 rows of up to 1024 values: G lanes a row, U accesses a lane, 256 / G
// rows a workgroup (group_fwd_kernel).  Measured on MI355X with one row per
// 64-lane workgroup instead: RMSNorm 262144 x 64 1.39 TB/s, 131072 x 128 2.43,
// 65536 x 256 3.93, 32768 x 512 5.13, 16384 x 1024 5.35; with the group
// kernel 5.74-5.77 up to 512 columns and 5.44 at 1024 (fused 5.62).
template <int OP>
hipError_t group_fwd_f32(int64_t hidden, const DynFwdArgs& a, hipStream_t stream) {
    if (hidden <= 32) return launch_group_fwd<OP, 8, 1>(a, stream);
    if (hidden <= 64) return launch_group_fwd<OP, 8, 2>(a, stream);
    if (hidden <= 128) return launch_group_fwd<OP, 8, 4>(a, stream);
    if (hidden <= 256) return launch_group_fwd<OP, 16, 4>(a, stream);
    if (hidden <= 512) return launch_group_fwd<OP, 32, 4>(a, stream);
    return launch_group_fwd<OP, 32, 8>(a, stream);
}
// (a whole wave a row, 8 accesses a lane, ran 4-9 % slower at 1536-2048
// columns than the one-row streamed launch)
constexpr int64_t kGroupFwdMaxHidden = 1024;

template <typename E, int OP>
hipError_t launch_stage_op(const DynFwdArgs& a, hipStream_t stream) {
    constexpr StageShape sh = stage_fwd_shape(OP, std::is_same_v<E, float>);
    return launch_stage_fwd<E, OP, sh.u, sh.l>(a, stream);
}

template <typename E>
hipError_t launch_stage_by_op(int op, const DynFwdArgs& a, hipStream_t stream) {
    switch (op) {
        case kSplitFused: return launch_stage_op<E, kSplitFused>(a, stream);
        case kSplitRms: return launch_stage_op<E, kSplitRms>(a, stream);
        default: return hipErrorInvalidValue;  // LayerNorm streams
    }
}

hipError_t launch_stream_fwd(int op, bool f32, const DynFwdArgs& a, hipStream_t stream) {
    if (f32 && a.hidden <= kGroupFwdMaxHidden) {
        switch (op) {
            case kSplitFused: return group_fwd_f32<kSplitFused>(a.hidden, a, stream);
            case kSplitRms: return group_fwd_f32<kSplitRms>(a.hidden, a, stream);
            case kSplitLn: return group_fwd_f32<kSplitLn>(a.hidden, a, stream);
            default: return hipErrorInvalidValue;
        }
    }
    if (stage_fwd_holds(op, f32, a.hidden))
        return f32 ? launch_stage_by_op<float>(op, a, stream)
                   : launch_stage_by_op<uint16_t>(op, a, stream);
    const StreamFwdShape sh = stream_fwd_shape(f32, op == kSplitLn, op == kSplitRms, a.hidden);
    switch (op) {
        case kSplitFused:
            if (f32) return fwd_f32_rms<kSplitFused>(sh, a, stream);
            return sh.unroll == 6
                       ? launch_stream_fwd_op<uint16_t, kSplitFused, kStreamFwdLanes, 6>(a, stream)
                       : launch_stream_fwd_op<uint16_t, kSplitFused, kStreamFwdLanes, 4>(a, stream);
        case kSplitRms:
            if (f32) return fwd_f32_rms<kSplitRms>(sh, a, stream);
            return sh.unroll == 8
                       ? launch_stream_fwd_op<uint16_t, kSplitRms, kStreamFwdLanes, 8>(a, stream)
                       : launch_stream_fwd_op<uint16_t, kSplitRms, kStreamFwdLanes, 4>(a, stream);
        case kSplitLn:
            return f32 ? fwd_f32_ln(sh, a, stream)
                       : launch_stream_fwd_op<uint16_t, kSplitLn, kStreamFwdLanes, 4>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename E, bool LN, bool DRES>
hipError_t launch_tiles(const DynBwdArgs& a, const float* stats, int32_t tiles, int32_t walkers,
                        hipStream_t stream) {
    hipLaunchKernelGGL(
        (stream_bwd_tile_kernel<E, kStreamTileVecs, LN, DRES, tile_depth<LN, DRES>()>),
        dim3((unsigned)(walkers * tiles)), dim3(kStreamTileLanes), 0, stream, a, stats,
        (int)tiles, (uint64_t*)nullptr, 0u);
    return hipGetLastError();
}

// The tiles of each row exchange their partial sums (no statistics kernel):
// the exchange area is zero-filled first.
template <typename E, bool LN, bool DRES>
hipError_t launch_tiles_xch(const DynBwdArgs& a, uint64_t* xch, int32_t tiles, int32_t walkers,
                            hipStream_t stream) {
    if (tiles < 2 || tiles > kXchMaxTiles) return hipErrorInvalidValue;  // the LDS slots
    if (a.rows > INT32_MAX) return hipErrorInvalidValue;  // the walk counts rows in 32 bits
    const int64_t words = xch_bytes(walkers, tiles) / 16;
    const int64_t zgrid = std::min<int64_t>((words + 255) / 256, 1024);
    hipLaunchKernelGGL(stream_zero_kernel, dim3((unsigned)zgrid), dim3(256), 0, stream,
                       (u32x4*)xch, words);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr bool kF32 = std::is_same_v<E, float>;
    constexpr int V = kF32 ? kStreamTileVecs : kXchVecsBf16;
    // fp32: two rings of 2 (LayerNorm, RMSNorm) or of 1 (fused); bf16: 2 accesses
    // a lane, two rings of kXchDepthBf16
    constexpr int D =
        kF32 ? (kXchAheadF32 && !DRES ? 2 : kXchAheadF32Dres ? 1 : tile_depth<LN, DRES>())
             : kXchDepthBf16;
    hipLaunchKernelGGL(
        (stream_bwd_tile_kernel<E, V, LN, DRES, D, false, true>),
        dim3((unsigned)(walkers * tiles)), dim3(kF32 ? kXchLanesF32 : kXchLanesBf16), 0,
        stream, a, (const float*)nullptr, (int)tiles, xch, stream_bwd_spin_limit());
    return hipGetLastError();
}

// One tile holds the whole fp32 row (hidden <= 8192): V accesses a lane, the
// row reduced in the tile kernel, each row read once.  Ring depth: the
// deepest without spills, fewer rows for wider tiles and with dres.
template <int V, bool DRES>
constexpr int inrow_depth() { return V == 4 ? (DRES ? 2 : 3) : V == 2 ? (DRES ? 3 : 4) : (DRES ? 6 : 8); }

template <int V, bool LN, bool DRES>
hipError_t launch_inrow(const DynBwdArgs& a, int32_t walkers, hipStream_t stream) {
    hipLaunchKernelGGL(
        (stream_bwd_tile_kernel<float, V, LN, DRES, inrow_depth<V, DRES>(), true>),
        dim3((unsigned)walkers), dim3(kStreamTileLanes), 0, stream, a, nullptr, 1,
        (uint64_t*)nullptr, 0u);
    return hipGetLastError();
}

template <bool LN, bool DRES>
hipError_t inrow_by_vecs(const DynBwdArgs& a, int32_t walkers, hipStream_t stream) {
    switch (stream_inrow_vecs_f32(a.hidden)) {
        case 1: return launch_inrow<1, LN, DRES>(a, walkers, stream);
        case 2: return launch_inrow<2, LN, DRES>(a, walkers, stream);
        default: return launch_inrow<4, LN, DRES>(a, walkers, stream);
    }
}

template <typename E>
hipError_t stream_bwd_typed(bool ln, const DynBwdArgs& a, int32_t tiles, int32_t walkers,
                            hipStream_t stream) {
    const int outs = ln ? 2 : 1;
    const int32_t padded = (int32_t)((a.hidden + 63) / 64 * 64);
    if (a.rows > 0 && std::is_same_v<E, float> && tiles == 1) {
        hipError_t e = ln              ? inrow_by_vecs<true, false>(a, walkers, stream)
                       : a.dres        ? inrow_by_vecs<false, true>(a, walkers, stream)
                                       : inrow_by_vecs<false, false>(a, walkers, stream);
        if (e != hipSuccess) return e;
    } else if (a.rows > 0 && stream_bwd_xch(a.hidden)) {
        uint64_t* xch = (uint64_t*)(a.workspace + (int64_t)walkers * outs * padded);
        hipError_t e = ln       ? launch_tiles_xch<E, true, false>(a, xch, tiles, walkers, stream)
                       : a.dres ? launch_tiles_xch<E, false, true>(a, xch, tiles, walkers, stream)
                                : launch_tiles_xch<E, false, false>(a, xch, tiles, walkers, stream);
        if (e != hipSuccess) return e;
    } else if (a.rows > 0) {
        float* stats = a.workspace + (int64_t)walkers * outs * padded;
        const int64_t grid = a.rows < kStreamMaxGrid ? a.rows : kStreamMaxGrid;
        if (ln)
            hipLaunchKernelGGL((stream_bwd_stats_kernel<E, true>), dim3((unsigned)grid),
                               dim3(kStreamFwdLanes), 0, stream, a, stats);
        else
            hipLaunchKernelGGL((stream_bwd_stats_kernel<E, false>), dim3((unsigned)grid),
                               dim3(kStreamFwdLanes), 0, stream, a, stats);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (ln) e = launch_tiles<E, true, false>(a, stats, tiles, walkers, stream);
        else if (a.dres) e = launch_tiles<E, false, true>(a, stats, tiles, walkers, stream);
        else e = launch_tiles<E, false, false>(a, stats, tiles, walkers, stream);
        if (e != hipSuccess) return e;
    }
    return launch_norm_colreduce(a.workspace, a.rows > 0 ? walkers : 0, a.hidden, padded, outs,
                                 a.dweight, a.dbias, stream);
}

hipError_t launch_stream_bwd(bool ln, bool f32, const DynBwdArgs& a, int32_t tiles,
                             int32_t walkers, hipStream_t stream) {
    return f32 ? stream_bwd_typed<float>(ln, a, tiles, walkers, stream)
               : stream_bwd_typed<uint16_t>(ln, a, tiles, walkers, stream);
}

}  // namespace rownorm
