// Device helpers shared by the row-normalization kernels (gfx950, wave64).
//
// Data layout of a row held in registers ("persistent buffer"): a row of H
// bf16 values is H/8 16-byte vectors.  With T lanes per row, lane t holds the
// vectors b*T + t for b = 0 .. H/(8T)-1, so at every b the T lanes read T
// consecutive 16-byte chunks (fully coalesced 128-bit loads), and the same
// lane always owns the same columns of every row.  This is the
// [serial, lanes, vector] split of the reduction axis that "optimize inner
// persistent scheduler for static fusion" (reviewer guide, split logic) uses
// with a static lane count; here the serial factor is a compile-time constant
// so the per-lane buffer is a fixed register array.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rownorm {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 8 bf16 values
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 pattern.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ void unpack8(const u32x4& v, float (&f)[8]) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// Two fp32 -> packed bf16x2, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
    u32x4 r;
    r.x = pack2(f[0], f[1]);
    r.y = pack2(f[2], f[3]);
    r.z = pack2(f[4], f[5]);
    r.w = pack2(f[6], f[7]);
    return r;
}

// Streamed row accesses (every byte of x / residual / out is touched once per
// call) carry the non-temporal hint: the fastest choice in steady-state
// measurements on MI355X.  The forward kernels use plain global loads and
// stores (measured 4-5% faster there than buffer instructions); the
// software-pipelined LayerNorm backward loop uses the buffer-descriptor
// helpers below with the same hint.
__device__ __forceinline__ u32x4 load_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_stream(u32x4* p, const u32x4& v) { __builtin_nontemporal_store(v, p); }
constexpr int kCachePolicyNT = 2;  // aux bits of buffer instructions: bit 1 = nt

// ---------------------------------------------------------------------------
// Row access through buffer resource descriptors.  A descriptor covers one
// row (base = that row's first byte, size = the row's bytes); for a row index
// past the end of the matrix the size is 0, so its loads return zeros and its
// stores are dropped by the hardware range check without touching memory.
// Rows beyond the end can then go through exactly the same instructions as
// real rows: no branch around any load or store, which keeps the compiler's
// memory-counter waits precise in software-pipelined loops.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9-family raw buffer, 32-bit data format

__device__ __forceinline__ rsrc_t row_rsrc(const void* base, int64_t row, int64_t rows,
                                           int row_bytes) {
    const char* p = static_cast<const char*>(base) + row * (int64_t)row_bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0,
                                             row < rows ? row_bytes : 0, kRsrcWord3);
}

__device__ __forceinline__ u32x4 rload_stream(rsrc_t r, int byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kCachePolicyNT);
}
__device__ __forceinline__ void rstore_stream(rsrc_t r, int byte_off, const u32x4& v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, kCachePolicyNT);
}
__device__ __forceinline__ float rload_f32(rsrc_t r, int byte_off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

// Keeps the scheduler from moving any instruction across this point.  Used
// right after a row's loads are issued so that all of them are in flight
// before the first arithmetic waits on one (the compiler otherwise sinks
// loads toward their uses to save registers, which serializes HBM latency).
__device__ __forceinline__ void issue_fence() { __builtin_amdgcn_sched_barrier(0); }

// DPP lane permutations (GFX9 encodings), full row/bank masks, all lanes active.
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                kCtrl, 0xF, 0xF, true));
}
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;  // rotate right by 4 inside each 16-lane row
constexpr int kDppRowRor8 = 0x128;  // rotate right by 8 inside each 16-lane row

__device__ __forceinline__ float readlane(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over the 64 lanes of the wave; every lane gets the same value (the
// final combine runs on lane-uniform operands in a fixed order).  Must be
// called with all 64 lanes active.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<kDppQuadXor1>(v);
    v += dpp<kDppQuadXor2>(v);
    v += dpp<kDppRowRor4>(v);
    v += dpp<kDppRowRor8>(v);
    // each lane now holds the sum of its 16-lane row; combine the 4 rows
    return (readlane(v, 0) + readlane(v, 16)) + (readlane(v, 32) + readlane(v, 48));
}

// Sum over the T lanes of one row.  T == 64: a wave reduction, no LDS.
// T > 64: each wave's total goes to LDS, one barrier, then every lane adds the
// T/64 totals in wave order.  `slot` is the row's LDS area (T/64 floats); the
// caller gives each consecutive reduction whose results may still be read a
// different slot so one barrier per reduction suffices.  Must be reached by
// every lane of the workgroup (uniform control flow).
template <int T>
__device__ __forceinline__ float row_sum(float v, float* slot, int lane_in_row) {
    v = wave_sum(v);
    if constexpr (T == kWave) {
        return v;
    } else {
        constexpr int kWaves = T / kWave;
        const int w = lane_in_row / kWave;
        if ((lane_in_row & (kWave - 1)) == 0) slot[w] = v;
        __syncthreads();
        float s = slot[0];
#pragma unroll
        for (int i = 1; i < kWaves; ++i) s += slot[i];
        return s;
    }
}

// Two sums at once (one barrier for both).
template <int T>
__device__ __forceinline__ void row_sum2(float& a, float& b, float* slot, int lane_in_row) {
    a = wave_sum(a);
    b = wave_sum(b);
    if constexpr (T != kWave) {
        constexpr int kWaves = T / kWave;
        const int w = lane_in_row / kWave;
        if ((lane_in_row & (kWave - 1)) == 0) {
            slot[2 * w] = a;
            slot[2 * w + 1] = b;
        }
        __syncthreads();
        float sa = slot[0], sb = slot[1];
#pragma unroll
        for (int i = 1; i < kWaves; ++i) {
            sa += slot[2 * i];
            sb += slot[2 * i + 1];
        }
        a = sa;
        b = sb;
    }
}

__device__ __forceinline__ float fast_rsqrt(float v) { return __builtin_amdgcn_rsqf(v); }

// Compile-time shape of one instantiation.
template <int H, int T, int R>
struct Shape {
    static constexpr int kHidden = H;
    static constexpr int kLanes = T;                  // lanes per row
    static constexpr int kRows = R;                   // rows per workgroup
    static constexpr int kBlock = T * R;              // workgroup size
    static constexpr int kVecs = H / (8 * T);         // 16-byte vectors per lane
    static constexpr int kRowVecs = H / 8;            // 16-byte vectors per row
    static constexpr int kWaves = T / kWave;          // waves per row
    static_assert(T % kWave == 0, "lanes per row must be whole waves");
    static_assert(H % (8 * T) == 0, "hidden must split evenly over the row's lanes");
    static_assert(kBlock <= 1024, "workgroup too large");
};

}  // namespace rownorm
