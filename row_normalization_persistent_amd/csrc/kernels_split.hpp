// Row-split forward kernels: the grid-parallel inner normalization of "Llu/ln
// bwd" (author note: the inner reduction split over several workgroups, which
// the pages list as missing), for batches too small to fill the chip with one
// workgroup per row.  One workgroup of kSplitLanes lanes streams a row at
// about 50 GB/s (a lone 64K-element fused row takes ~10 us), so with few rows
// each row is cut into k contiguous chunks of kSplitLanes * V * 8 columns, one
// workgroup per chunk, and the chunks' partial sums meet in a workspace.
//
// Per workgroup (row i, chunk j of k):
//   1. load the chunk (16-byte accesses, the dyn_common.hpp layout with the
//      chunk's first column as origin; columns past hidden load zeros);
//      fused op: s = x + r, residual <- bf16(s) at once;
//   2. reduce over the workgroup: sum s^2 (RMSNorm, fused) or, for LayerNorm,
//      the chunk's sum S_j and its centered sum of squares M2_j around its
//      own mean (two passes over the registers);
//   3. lane 0 publishes the partials in the row's slot j of the workspace,
//      each as one device-coherent 64-bit word carrying its own ready flag;
//      lanes 0 .. k-1 of wave 0 poll the row's k slots at once until all are
//      there; every lane then adds the k partials in chunk order, so the
//      result is the same in every workgroup of the row and from run to run.
//      LayerNorm combines the chunks' (S_j, M2_j) exactly (pairwise update of
//      a sum of squared deviations):
//        mean = sum_j S_j / H,  M2 = sum_j M2_j + n_j (S_j / n_j - mean)^2;
//   4. normalize the chunk from registers and store it;
//   5. count the workgroup out of the row (acquire-release); the row's last
//      one zeroes the row's words, so the workspace is zero-filled again for
//      the next call.
//
// Every workgroup of a launch must be resident at once (the waits); the host
// keeps rows * k at or below the CU count, one workgroup per CU.  A wait polls
// at most SplitArgs::spin_limit times (kSplitSpinLimit, about a second, unless
// the host set another limit; 0: give up without polling).  A workgroup that
// gives up sets bit 0 of the workspace's first word and takes NaN for every
// partial it has not seen, so its chunk's outputs (and, for chunk 0, the
// row's mean and rstd) are NaN rather than wrong finite values; it still
// departs the row, so the workspace's row words end zero-filled.  Giving up
// can only happen when other work keeps this launch's workgroups off the CUs
// (or the host asked for it).
#pragma once

#include "dyn_common.hpp"
#include "launch.hpp"

namespace rownorm {

// Step 3 for wave 0 of the workgroup.  A partial is published as one 64-bit
// word (value bits << 32 | 1): its nonzero low half says it is there, so the
// data and its ready flag arrive together and no fence is needed on this
// path.  Lane i < k polls chunk i's word(s) (one round trip per poll for the
// whole row), at most `limit` times, and puts the values in q0[i], q1[i]
// (LDS); a lane that runs out of polls records the give-up in *err and
// writes NaN there instead.
__device__ __forceinline__ void split_publish_and_gather(uint64_t* slot, uint32_t* err, int j,
                                                         int k, bool two, float p0, float p1,
                                                         float* q0, float* q1, int lane,
                                                         uint32_t limit) {
    if (lane == 0) {
        __hip_atomic_store(&slot[kSplitP0 + j], ((uint64_t)__float_as_uint(p0) << 32) | 1u,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (two)
            __hip_atomic_store(&slot[kSplitP1 + j], ((uint64_t)__float_as_uint(p1) << 32) | 1u,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (lane < k) {
        uint64_t a = 0, b = two ? 0 : 1;
        bool seen = false;
        for (uint32_t polls = 0; polls < limit; ++polls) {
            if (!(a & 1u))
                a = __hip_atomic_load(&slot[kSplitP0 + lane], __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
            if (!(b & 1u))
                b = __hip_atomic_load(&slot[kSplitP1 + lane], __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
            if ((a & b & 1u) != 0) {
                seen = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (!seen) {
            __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            a = (uint64_t)__float_as_uint(__builtin_nanf("")) << 32;
            b = a;
        }
        q0[lane] = __uint_as_float((uint32_t)(a >> 32));
        q1[lane] = __uint_as_float((uint32_t)(b >> 32));
    }
}

// Step 4, after the workgroup is done with the partials (off the critical
// path): the row's last workgroup to get here zeroes the row's words.  The
// acquire-release count orders every workgroup's reads of the partials
// before the zeroing.  Wave 0 only.
__device__ __forceinline__ void split_depart(uint64_t* slot, int k, bool two, int lane) {
    uint32_t last = 0;
    if (lane == 0)
        last = __hip_atomic_fetch_add(reinterpret_cast<uint32_t*>(&slot[kSplitDepart]), 1u,
                                      __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
               (uint32_t)(k - 1);
    last = __shfl(last, 0);
    if (last && lane < k) {
        __hip_atomic_store(&slot[kSplitP0 + lane], (uint64_t)0, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        if (two)
            __hip_atomic_store(&slot[kSplitP1 + lane], (uint64_t)0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        if (lane == 0)
            __hip_atomic_store(&slot[kSplitDepart], (uint64_t)0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int V, int OP>
__global__ __launch_bounds__(kSplitLanes) void split_norm_kernel(SplitArgs a) {
    constexpr int kChunk = kSplitLanes * V * 8;  // columns per workgroup
    constexpr int kWaves = kSplitLanes / kWave;
    __shared__ float red[2 * kWaves];
    __shared__ float q0[kSplitMax], q1[kSplitMax];
    const int k = a.split;
    const int64_t row = blockIdx.x / k;
    const int j = (int)(blockIdx.x - row * k);
    const int lane = threadIdx.x;
    const int h = a.hidden;
    const int col0 = j * kChunk;
    const int n_j = min(h - col0, kChunk);  // > 0: the host leaves no chunk empty

    const rsrc_t rx = row_rsrc_ld(a.x, row, a.rows, a.ld_x * 2, h * 2);
    const rsrc_t ro = row_rsrc_ld(a.out, row, a.rows, a.ld_out * 2, h * 2);
    const rsrc_t rw = row_rsrc_ld(a.weight, 0, 1, 0, h * 2);
    rsrc_t rr = rx, rb = rx;
    if constexpr (OP == kSplitFused) rr = row_rsrc_ld(a.residual, row, a.rows, a.ld_res * 2, h * 2);
    if constexpr (OP == kSplitLn) rb = row_rsrc_ld(a.bias, 0, 1, 0, h * 2);

    u32x4 xv[V], rv[OP == kSplitFused ? V : 1], wv[V], bv[OP == kSplitLn ? V : 1];
#pragma unroll
    for (int b = 0; b < V; ++b) {
        const int off = (col0 + (b * kSplitLanes + lane) * 8) * 2;
        xv[b] = aload<8, kCachePolicyNT>(rx, off);
        if constexpr (OP == kSplitFused) rv[b] = aload<8, kCachePolicyNT>(rr, off);
    }
#pragma unroll
    for (int b = 0; b < V; ++b) {
        const int off = (col0 + (b * kSplitLanes + lane) * 8) * 2;
        wv[b] = aload<8, 0>(rw, off);
        if constexpr (OP == kSplitLn) bv[b] = aload<8, 0>(rb, off);
    }
    issue_fence();

    // step 1-2: the chunk's partial sums
    float s[V][8];
    float p0 = 0.0f, p1 = 0.0f;
    if constexpr (OP == kSplitLn) {
        float acc = 0.0f;
#pragma unroll
        for (int b = 0; b < V; ++b) {
            unpack8(xv[b], s[b]);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc += s[b][e];
        }
        p0 = row_sum<kSplitLanes>(acc, red, lane);
        const float mu_j = p0 / (float)n_j;
        float acc2 = 0.0f;
#pragma unroll
        for (int b = 0; b < V; ++b) {
            // accesses past the row's end hold zeros; (0 - mu_j)^2 must not count
            const bool in_row = col0 + (b * kSplitLanes + lane) * 8 < h;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float d = in_row ? s[b][e] - mu_j : 0.0f;
                acc2 += d * d;
            }
        }
        p1 = row_sum<kSplitLanes>(acc2, red + kWaves, lane);
    } else {
        float acc = 0.0f;
#pragma unroll
        for (int b = 0; b < V; ++b) {
            float xf[8];
            unpack8(xv[b], xf);
            if constexpr (OP == kSplitFused) {
                float rf[8];
                unpack8(rv[b], rf);
#pragma unroll
                for (int e = 0; e < 8; ++e) s[b][e] = xf[e] + rf[e];
                astore<8, kCachePolicyNT>(rr, (col0 + (b * kSplitLanes + lane) * 8) * 2,
                                          pack8(s[b]));
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) s[b][e] = xf[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) acc += s[b][e] * s[b][e];  // past the end: 0
        }
        p0 = row_sum<kSplitLanes>(acc, red, lane);
    }

    // step 3: meet the row's other chunks
    uint64_t* slot = reinterpret_cast<uint64_t*>(a.ws + kSplitHeaderWords) + row * kSplitRowQwords;
    if (lane < kWave)
        split_publish_and_gather(slot, a.ws, j, k, OP == kSplitLn, p0, p1, q0, q1, lane,
                                 a.spin_limit);
    __syncthreads();

    const float inv_h = 1.0f / (float)h;
    float mu = 0.0f, rstd;
    if constexpr (OP == kSplitLn) {
        float tot = 0.0f;
        for (int i = 0; i < k; ++i) tot += q0[i];
        mu = tot * inv_h;
        float m2 = 0.0f;
        for (int i = 0; i < k; ++i) {
            const float n_i = (float)min(h - i * kChunk, kChunk);
            const float d = q0[i] / n_i - mu;
            m2 += q1[i] + n_i * d * d;
        }
        rstd = fast_rsqrt(m2 * inv_h + a.eps);
        if (j == 0 && lane == 0 && a.mean != nullptr) {
            a.mean[row] = mu;
            a.rstd[row] = rstd;
        }
    } else {
        float tot = 0.0f;
        for (int i = 0; i < k; ++i) tot += q0[i];
        rstd = fast_rsqrt(tot * inv_h + a.eps);
    }

    // step 5: normalize from registers
#pragma unroll
    for (int b = 0; b < V; ++b) {
        float wf[8], o[8];
        unpack8(wv[b], wf);
        if constexpr (OP == kSplitLn) {
            float bf[8];
            unpack8(bv[b], bf);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = (s[b][e] - mu) * rstd * wf[e] + bf[e];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = s[b][e] * rstd * wf[e];
        }
        astore<8, kCachePolicyNT>(ro, (col0 + (b * kSplitLanes + lane) * 8) * 2, pack8(o));
    }
    // step 4
    if (lane < kWave) split_depart(slot, k, OP == kSplitLn, lane);
}

template <int V, int OP>
hipError_t launch_split(const SplitArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.rows * a.split)), block(kSplitLanes);
    hipLaunchKernelGGL((split_norm_kernel<V, OP>), grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace rownorm
