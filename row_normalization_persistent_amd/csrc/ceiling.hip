// Measurement kernel for the benchmark only (not part of the normalization
// library or its C ABI): the fused residual-add + RMSNorm forward's exact
// memory traffic at hidden 4096 without its arithmetic.  Each row's x and
// residual vectors are read with the same lane layout, launch shape and
// non-temporal hints as fused_add_rmsnorm_kernel<4096, T, R>, and two outputs
// are written (x to `residual`, the old residual to `out`); no reduction, no
// barrier.  Its time is a same-traffic ceiling for the fused kernel on the
// part it runs on.  Built into libnormceiling.so, loaded by bench.py.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace {

using rownorm::u32x4;

template <int H, int T, int R>
__global__ __launch_bounds__(T * R) void same_traffic_copy_kernel(u32x4* out, u32x4* residual,
                                                                  const u32x4* x, int64_t rows) {
    constexpr int V = H / (8 * T);
    constexpr int kRowVecs = H / 8;
    const int lane = threadIdx.x % T;
    const int64_t row = (int64_t)blockIdx.x * R + threadIdx.x / T;
    if (row >= rows) return;
    const int64_t base = row * kRowVecs + lane;
    u32x4 xv[V], rv[V];
#pragma unroll
    for (int b = 0; b < V; ++b) {
        xv[b] = rownorm::load_stream(x + base + b * T);
        rv[b] = rownorm::load_stream(residual + base + b * T);
    }
    rownorm::issue_fence();
#pragma unroll
    for (int b = 0; b < V; ++b) rownorm::store_stream(residual + base + b * T, xv[b]);
#pragma unroll
    for (int b = 0; b < V; ++b) rownorm::store_stream(out + base + b * T, rv[b]);
}

template <int T, int R>
hipError_t launch(void* out, void* residual, const void* x, int64_t rows, hipStream_t stream) {
    const int64_t grid = (rows + R - 1) / R;
    hipLaunchKernelGGL((same_traffic_copy_kernel<4096, T, R>), dim3((unsigned)grid), dim3(T * R),
                       0, stream, (u32x4*)out, (u32x4*)residual, (const u32x4*)x, rows);
    return hipGetLastError();
}

}  // namespace

// Returns 0 on success, 1 for invalid arguments (null or misaligned pointers,
// rows outside [0, 2^31)) or a shape that is not compiled, 2 when the launch
// fails.  x, residual and out are contiguous [rows, 4096] bf16 device
// matrices; residual and out are overwritten.  Shapes (threads_per_row,
// rows_per_block): (64, 4), (128, 2), (256, 1), (512, 1).
extern "C" __attribute__((visibility("default"))) int normceil_same_traffic_h4096(
    void* out, void* residual, const void* x, int64_t rows, int32_t threads_per_row,
    int32_t rows_per_block, hipStream_t stream) {
    if (rows < 0 || rows >= (int64_t(1) << 31)) return 1;
    if (rows == 0) return 0;
    auto misaligned = [](const void* p) { return !p || reinterpret_cast<uintptr_t>(p) % 16 != 0; };
    if (misaligned(out) || misaligned(residual) || misaligned(x)) return 1;
    hipError_t e;
    if (threads_per_row == 64 && rows_per_block == 4)
        e = launch<64, 4>(out, residual, x, rows, stream);
    else if (threads_per_row == 128 && rows_per_block == 2)
        e = launch<128, 2>(out, residual, x, rows, stream);
    else if (threads_per_row == 256 && rows_per_block == 1)
        e = launch<256, 1>(out, residual, x, rows, stream);
    else if (threads_per_row == 512 && rows_per_block == 1)
        e = launch<512, 1>(out, residual, x, rows, stream);
    else
        return 1;
    return e == hipSuccess ? 0 : 2;
}
