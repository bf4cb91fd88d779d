// Device helpers of the LDS-staged kernels: rows (or the part of a row that
// registers cannot hold) go from HBM straight into LDS by buffer loads with
// the LDS bit (gfx950), the CDNA counterpart of the bulk copies into shared
// memory of "TMA inner persistent scheduler" (description summary), and come
// back to registers by 16-byte LDS reads.  The loads are issued from asm, so
// the kernels order them with explicit counter waits.
#pragma once

#include "dyn_common.hpp"

namespace rownorm {

// Waits written as volatile asm with a memory clobber, so that the compiler
// moves no LDS access across them: every counter to zero (the row's
// buffer-to-LDS loads have landed), and the LDS / scalar counter alone (this
// wave's LDS reads of a slot are done before a load may overwrite it).
__device__ __forceinline__ void wait_all_counters() {
    asm volatile("s_waitcnt vmcnt(0) expcnt(0) lgkmcnt(0)" ::: "memory");
}
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// At most N vector-memory operations of this wave still outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// At most n vector-memory operations outstanding, n a constant once the
// caller's loop is unrolled (one wait instruction); counts above 63, the
// counter's range, wait for 63.
template <int N = 63>
__device__ __forceinline__ void wait_vm_at_most(int n) {
    if constexpr (N == 0) {
        wait_vm<0>();
    } else {
        if (n >= N) wait_vm<N>();
        else wait_vm_at_most<N - 1>(n);
    }
}

// p[i] through the scalar data cache (a wave-uniform index into a read-only
// input of the kernel, so the load is a scalar one and no vector-memory wait
// ever waits for it), or 0 for i >= n.
__device__ __forceinline__ float uniform_load_f32(const float* p, int64_t i, int64_t n) {
    const __attribute__((address_space(4))) float* q =
        (const __attribute__((address_space(4))) float*)p;
    return i < n ? q[i] : 0.0f;
}

// A row's buffer descriptor as four scalar words: base address (48 bits, no
// stride), size in bytes (0 past the matrix's last row), format word.
typedef uint32_t desc4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ desc4 row_desc(const void* base, int64_t row, int64_t rows,
                                          int64_t ld_bytes, int row_bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(static_cast<const char*>(base) + row * ld_bytes);
    desc4 d;
    d.x = (uint32_t)p;
    d.y = (uint32_t)(p >> 32) & 0xffffu;
    d.z = row < rows ? (uint32_t)row_bytes : 0u;
    d.w = (uint32_t)kRsrcWord3;
    return d;
}

// One 16-byte-per-lane buffer load straight into LDS (non-temporal): lane i
// of the wave writes bytes [16 i, 16 i + 16) past LDS address `lds` (wave
// uniform) with the 16 bytes at byte `voff` of the descriptor's range (zeros,
// from no memory, past its end).  Issued from asm so that the compiler does
// not track it: it would otherwise make every later LDS read of the wave wait
// for it, the reads of other slots included.  The caller orders it: LDS reads
// of the slots before it (wait_lds), and its landing before any read of them
// (wait_all_counters).
// M0 (which the load takes its LDS address from) is saved and restored inside
// the asm, since the compiler does not allocate M0 and may not expect an asm
// statement to change it.
__device__ __forceinline__ void lds_load16(desc4 d, int voff, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen nt lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(d), "s"(lds)
        : "memory");
}

// The value of v, opaque to the optimizer (emits no instruction).
__device__ __forceinline__ int opaque_lane(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

}  // namespace rownorm
