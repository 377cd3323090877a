// moe_probe.hip - measurement helper: a plain streaming read of a device
// buffer, the HBM ceiling the layer's weight streams are compared with.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kProbeThreads = 512;
constexpr int kProbeLoads = 8;   // 16-byte loads in flight per thread and round

// Thread g of the grid reads chunks g, g + n, g + 2n, ... (n = grid threads),
// kProbeLoads at a time, all issued before any is used; the XOR of the data
// is stored only if it equals a value no run produces, which keeps the loads
// alive without writing anything.
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4* __restrict__ src,
                                                                   int64_t n_chunks,
                                                                   u32x4* __restrict__ sink) {
    const int64_t n = (int64_t)gridDim.x * kProbeThreads;
    const int64_t g = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t base = g; base < n_chunks; base += n * kProbeLoads) {
        u32x4 v[kProbeLoads];
#pragma unroll
        for (int i = 0; i < kProbeLoads; ++i) {
            const int64_t c = min(base + n * i, n_chunks - 1);
            v[i] = __builtin_nontemporal_load(src + c);
        }
#pragma unroll
        for (int i = 0; i < kProbeLoads; ++i) acc ^= v[i];
    }
    if (acc.x == 0x9E3779B9u && acc.y == 0x7F4A7C15u && acc.z == 0x94D049BBu && acc.w == 0x2545F491u)
        sink[g & 255] = acc;
}

hipError_t launch_probe_read(const void* src, size_t bytes, int grid, void* sink, hipStream_t s) {
    MOE_LAUNCH(probe_read_kernel, dim3(grid), dim3(kProbeThreads), 0, s, (const u32x4*)src,
               (int64_t)(bytes / 16), (u32x4*)sink);
    return hipGetLastError();
}

}  // namespace moe
