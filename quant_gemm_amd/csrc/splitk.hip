// Split-K support for the prefill GEMMs: how many K ranges a launch is cut
// into, and the pass that sums the partial results in a fixed order.
//
// A GEMM whose tile count is small against the workgroups the chip holds at
// once (2 per CU for both GEMM kernels) leaves CUs idle or ends on a partial
// wave of tiles. Cutting K into S ranges multiplies the workgroups by S; each
// range writes f32 partial sums to its own [M][N] plane of the caller's
// workspace, and splitk_reduce adds the S planes in order s = 0..S-1, so the
// result does not depend on scheduling.
#include <atomic>
#include <cmath>
#include <cstdint>

#include "mq_device.h"
#include "mq_launch.h"

namespace mq {
namespace {

__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ part, int nsplit,
                                                            int64_t n, float *__restrict__ out)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        float v = part[i];
        for (int s = 1; s < nsplit; ++s)
            v += part[(int64_t)s * n + i];
        out[i] = v;
    }
}

// n4 float4 groups; out 16-byte aligned
__global__ __launch_bounds__(256) void splitk_reduce4_kernel(const v4f *__restrict__ part, int nsplit,
                                                             int64_t n4, v4f *__restrict__ out)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        v4f v = part[i];
        for (int s = 1; s < nsplit; ++s)
            v += part[(int64_t)s * n4 + i];
        out[i] = v;
    }
}

} // namespace

int device_cu_count()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0)
        return v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
        v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

int gemm_splits(int tiles, int tile_elems, int pairs, int64_t M, int64_t N, int K, double slot_ops)
{
    // Time of the tiles over all of K at two workgroups per CU. A
    // last, partial wave of at most one workgroup per CU runs about 1.6x as
    // fast (its workgroups do not share a CU), so it counts 0.6.
    const int ncu = device_cu_count();
    const int slots = 2 * ncu;
    const double t_tile = 2.0 * tile_elems * K / slot_ops;  // seconds, one tile over all of K
    const double bw = 4.0e12;                                // bytes/s of the reduction pass
    auto waves = [&](int64_t n) {
        const int64_t full = n / slots, rem = n % slots;
        return (double)full + (rem == 0 ? 0.0 : rem <= ncu ? 0.6 : 1.0);
    };
    double best_t = waves(tiles) * t_tile;
    int best = 1;
    for (int s : {2, 3, 4, 6, 8, 12, 16}) {
        if (s > pairs)
            break;
        const double t = waves((int64_t)tiles * s) * t_tile / s +
                         (double)(s + 1) * (double)M * (double)N * 4.0 / bw + 3e-6;
        if (t < 0.97 * best_t) {
            best_t = t;
            best = s;
        }
    }
    return best;
}

hipError_t splitk_reduce(const float *part, int nsplit, int64_t n, float *out, hipStream_t st)
{
    const int64_t cap = 8 * (int64_t)device_cu_count();
    if (n % 4 == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0 &&
        (reinterpret_cast<uintptr_t>(part) & 15) == 0) {
        const int64_t n4 = n / 4;
        const int64_t grid = std::max<int64_t>(1, std::min<int64_t>((n4 + 255) / 256, cap));
        splitk_reduce4_kernel<<<dim3((unsigned)grid), dim3(256), 0, st>>>(
            reinterpret_cast<const v4f *>(part), nsplit, n4, reinterpret_cast<v4f *>(out));
    } else {
        const int64_t grid = std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, cap));
        splitk_reduce_kernel<<<dim3((unsigned)grid), dim3(256), 0, st>>>(part, nsplit, n, out);
    }
    return hipGetLastError();
}

} // namespace mq
