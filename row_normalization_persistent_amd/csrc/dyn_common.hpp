// Device helpers of the run-time-hidden kernels: the fallback for hidden
// sizes outside the compiled set, hidden sizes that are not a multiple of 8,
// and rows with a leading dimension (row stride) larger than the row.  This is
// the non-static path of "optimize inner persistent scheduler for static
// fusion" (reviewer guide, split logic: without a static extent the reduction
// axis is split by a run-time factor) and the dynamic block dimensions of
// "TMA inner persistent scheduler" (description summary).
//
// Layout in registers is the compiled kernels' [serial, lanes, vector] split
// with a run-time extent: a row of `hidden` bf16 values is cut into accesses of
// W elements (W = 8, 4, 2 or 1: 16, 8, 4 or 2 bytes, the widest that hidden,
// every row stride and every pointer allow), lane t of the row's T lanes holds
// the accesses b*T + t for b < V, and V*T*W >= hidden.  Accesses past the
// row's end go through a buffer descriptor sized to the row, so they load
// zeros from no memory and their stores are dropped.  Rows narrower than a
// wave (T = 8, 16, 32) share a wave and reduce within their lane group.
#pragma once

#include "device_common.hpp"

namespace rownorm {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---- accesses of W bf16 elements ------------------------------------------------
template <int W> struct Access;
template <> struct Access<8> { using raw = u32x4; };
template <> struct Access<4> { using raw = u32x2; };
template <> struct Access<2> { using raw = uint32_t; };
template <> struct Access<1> { using raw = uint16_t; };
template <int W> using raw_t = typename Access<W>::raw;

// Aux is the buffer instruction's cache-policy field (kCachePolicyNT or 0).
template <int W, int Aux>
__device__ __forceinline__ raw_t<W> aload(rsrc_t r, int byte_off) {
    if constexpr (W == 8) return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, Aux);
    else if constexpr (W == 4) return __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, Aux);
    else if constexpr (W == 2) return __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, Aux);
    else return __builtin_amdgcn_raw_buffer_load_b16(r, byte_off, 0, Aux);
}

template <int W, int Aux>
__device__ __forceinline__ void astore(rsrc_t r, int byte_off, const raw_t<W>& v) {
    if constexpr (W == 8) __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, Aux);
    else if constexpr (W == 4) __builtin_amdgcn_raw_buffer_store_b64(v, r, byte_off, 0, Aux);
    else if constexpr (W == 2) __builtin_amdgcn_raw_buffer_store_b32(v, r, byte_off, 0, Aux);
    else __builtin_amdgcn_raw_buffer_store_b16(v, r, byte_off, 0, Aux);
}

template <int W>
__device__ __forceinline__ void aunpack(const raw_t<W>& v, float (&f)[W]) {
    if constexpr (W == 8) {
        unpack8(v, f);
    } else if constexpr (W == 4) {
        f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
        f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    } else if constexpr (W == 2) {
        f[0] = bf16_lo(v); f[1] = bf16_hi(v);
    } else {
        f[0] = bf16_lo((uint32_t)v);
    }
}

template <int W>
__device__ __forceinline__ raw_t<W> apack(const float (&f)[W]) {
    if constexpr (W == 8) {
        return pack8(f);
    } else if constexpr (W == 4) {
        u32x2 r;
        r.x = pack2(f[0], f[1]);
        r.y = pack2(f[2], f[3]);
        return r;
    } else if constexpr (W == 2) {
        return pack2(f[0], f[1]);
    } else {
        return (uint16_t)(pack2(f[0], 0.0f) & 0xffffu);
    }
}

// Descriptor of row `row` of a matrix whose rows start `ld_bytes` apart and
// hold `row_bytes` bytes of data; a row index past the end gets size 0.
__device__ __forceinline__ rsrc_t row_rsrc_ld(const void* base, int64_t row, int64_t rows,
                                              int64_t ld_bytes, int row_bytes) {
    const char* p = static_cast<const char*>(base) + row * ld_bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0,
                                             row < rows ? row_bytes : 0, kRsrcWord3);
}

// ---- addressing a set of rows -------------------------------------------------------
// Buffer descriptors are scalar: every lane of a wave must use the same one, or
// the compiler serializes the access over the distinct values.  A row of at
// least 64 lanes is uniform over its waves, so it gets a descriptor of its own
// (sized to the row: accesses past its end are range-checked to zero).  Rows
// narrower than a wave share one descriptor per set of consecutive rows (the
// rows of a workgroup, or of one backward ring step), and each lane adds its
// row's offset; an access past its row's end gets an offset beyond the range.
// The host keeps such a set's extent below 2^31 bytes.
constexpr int kOutOfRange = 0x7ffffff0;

template <int T>
__device__ __forceinline__ int uniform_group(int g) {
    if constexpr (T >= kWave) return __builtin_amdgcn_readfirstlane(g);
    else return g;
}

// Descriptor of rows [first, first + span) of a matrix (rows past `rows` are
// left out; an empty set gets size 0).  For T >= 64 the set is one row.
template <int T>
__device__ __forceinline__ rsrc_t rows_rsrc(const void* base, int64_t first, int64_t span,
                                            int64_t rows, int64_t ld, int hidden, int elem) {
    const char* p = static_cast<const char*>(base) + first * ld * elem;
    int bytes;
    if constexpr (T >= kWave) {
        bytes = first < rows ? hidden * elem : 0;
    } else {
        const int64_t n = rows - first < span ? rows - first : span;
        bytes = n > 0 ? (int)(((n - 1) * ld + hidden) * elem) : 0;
    }
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0, bytes, kRsrcWord3);
}

// An optimization barrier for a wave-uniform row index: the compiler may not
// precompute values derived from it for several loop iterations at once
// (which, for every matrix and ring slot, would hold scalar registers for
// the whole loop).  Emits no instruction.
__device__ __forceinline__ int64_t opaque_row(int64_t r) {
    asm volatile("" : "+s"(r));
    return r;
}

// Byte offset of a lane's access at column `col` of row `local` of a set
// (T >= 64: the set's only row, masked by the descriptor's size).
template <int T>
__device__ __forceinline__ int set_off(int local, int col, int64_t ld, int hidden, int elem) {
    if constexpr (T >= kWave) return col * elem;
    else return col < hidden ? (int)((local * ld + col) * elem) : kOutOfRange;
}

// ---- workgroup shape ---------------------------------------------------------------
// Rows narrower than 256 lanes are packed 256 / T to a workgroup (four waves),
// wider rows take a workgroup each.
template <int T>
constexpr int dyn_block() { return T < 256 ? 256 : T; }

// ---- reductions over a row's T lanes ------------------------------------------------
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7 - i inside each 8-lane half row

// Sum over an aligned group of T lanes (T = 8, 16, 32) of one wave; every lane
// of the group gets the same value (each step adds a value to its partner's
// in commutative pairs).  All 64 lanes must be active.
template <int T>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(T == 8 || T == 16 || T == 32, "sub-wave groups only");
    v += dpp<kDppQuadXor1>(v);
    v += dpp<kDppQuadXor2>(v);
    v += dpp<kDppHalfMirror>(v);                   // lanes 0-3 + lanes 4-7
    if constexpr (T >= 16) v += dpp<kDppRowRor8>(v);  // the two 8-lane halves of a 16-lane row
    if constexpr (T >= 32) v += __shfl_xor(v, 16);    // the two 16-lane rows of a 32-lane half
    return v;
}

// Sum over the T lanes of one row for any T of the run-time path.  `slot` is
// the row's LDS area (T/64 floats) when T > 64; uniform control flow required.
template <int T>
__device__ __forceinline__ float dyn_row_sum(float v, float* slot, int lane_in_row) {
    if constexpr (T < kWave) return group_sum<T>(v);
    else return row_sum<T>(v, slot, lane_in_row);
}

template <int T>
__device__ __forceinline__ void dyn_row_sum2(float& a, float& b, float* slot, int lane_in_row) {
    if constexpr (T < kWave) {
        a = group_sum<T>(a);
        b = group_sum<T>(b);
    } else {
        row_sum2<T>(a, b, slot, lane_in_row);
    }
}

// LDS floats one reduction of a workgroup needs (per row: T/64 wave totals).
template <int T>
constexpr int dyn_red_floats() { return T > kWave ? (dyn_block<T>() / T) * (T / kWave) : 1; }

// ---- elements of a 16-byte access ------------------------------------------------
template <typename E> struct Elems;
template <> struct Elems<uint16_t> { static constexpr int kPer = 8; };  // bf16 patterns
template <> struct Elems<float> { static constexpr int kPer = 4; };

template <typename E>
__device__ __forceinline__ void unpack16(const u32x4& v, float (&f)[Elems<E>::kPer]) {
    if constexpr (Elems<E>::kPer == 8) {
        unpack8(v, f);
    } else {
        f[0] = __uint_as_float(v.x);
        f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z);
        f[3] = __uint_as_float(v.w);
    }
}

// bf16: round to nearest even; fp32: the values themselves
template <typename E>
__device__ __forceinline__ u32x4 pack16(const float (&f)[Elems<E>::kPer]) {
    if constexpr (Elems<E>::kPer == 8) {
        return pack8(f);
    } else {
        u32x4 v;
        v.x = __float_as_uint(f[0]);
        v.y = __float_as_uint(f[1]);
        v.z = __float_as_uint(f[2]);
        v.w = __float_as_uint(f[3]);
        return v;
    }
}


}  // namespace rownorm
