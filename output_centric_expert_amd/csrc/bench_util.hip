// Measurement kernels: a contiguous streaming read (the peak-bandwidth
// reference the warp-decode post measures its kernels against -- section
// "Hardware efficiency": peak taken with a copy kernel over contiguous reads)
// and a plain copy of known size, used to calibrate HBM byte counters.
#include "launch.h"
#include "mx_device.h"

namespace moed {

// Each wavefront reads kReadU x 16 bytes per lane, all loads issued before
// use; the XOR of the data is written to sink only if it equals a sentinel,
// which keeps the loads alive without a data-dependent store stream.
constexpr int kReadU = 2;

__global__ void __launch_bounds__(256)
moe_bench_read_kernel(const u32x4* __restrict__ src, long n16, uint32_t* sink)
{
    const int lane = threadIdx.x & (kWave - 1);
    const long wave = (long)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const long base = wave * (long)kWave * kReadU;
    u32x4 v[kReadU];
#pragma unroll
    for (int m = 0; m < kReadU; ++m) {
        const long c = base + lane + (long)kWave * m;
        v[m] = c < n16 ? __builtin_nontemporal_load(src + c) : u32x4{0, 0, 0, 0};
    }
    uint32_t x = 0;
#pragma unroll
    for (int m = 0; m < kReadU; ++m)
        x ^= v[m].x ^ v[m].y ^ v[m].z ^ v[m].w;
    if (x == 0x9E3779B9u)
        sink[wave & 1023] = x;
}

// The read probe with a chosen launch shape: each wavefront reads chunks of
// 64*U 16-byte units (all U loads in flight together) at a stride of the whole
// grid's wavefronts, so a grid that covers the bytes reads each chunk once in
// a single pass and a smaller (persistent) grid loops.
template <int U>
__global__ void __launch_bounds__(1024)
moe_bench_read_cfg_kernel(const u32x4* __restrict__ src, long n16, uint32_t* sink)
{
    const int lane = threadIdx.x & (kWave - 1);
    const long nw = (long)gridDim.x * (blockDim.x / kWave);
    const long wave = (long)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const long nchunk = (n16 + (long)kWave * U - 1) / ((long)kWave * U);
    uint32_t x = 0;
    for (long ch = wave; ch < nchunk; ch += nw) {
        u32x4 v[U];
#pragma unroll
        for (int m = 0; m < U; ++m) {
            const long c = ch * (long)kWave * U + lane + (long)kWave * m;
            v[m] = c < n16 ? __builtin_nontemporal_load(src + c) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int m = 0; m < U; ++m)
            x ^= v[m].x ^ v[m].y ^ v[m].z ^ v[m].w;
    }
    if (x == 0x9E3779B9u)
        sink[wave & 1023] = x;
}

__global__ void __launch_bounds__(256)
moe_bench_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, long n16)
{
    const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < n16)
        dst[t] = src[t];
}

hipError_t launch_bench_read(const void* src, size_t bytes, void* sink, hipStream_t s)
{
    const long n16 = (long)(bytes / 16);
    if (n16 == 0)
        return hipSuccess;
    const long waves = (n16 + (long)kWave * kReadU - 1) / ((long)kWave * kReadU);
    hipLaunchKernelGGL(moe_bench_read_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s,
                       static_cast<const u32x4*>(src), n16, static_cast<uint32_t*>(sink));
    return hipGetLastError();
}

hipError_t launch_bench_read_cfg(const void* src, size_t bytes, void* sink, int unroll, int waves_per_group,
                                 int groups, hipStream_t s)
{
    const long n16 = (long)(bytes / 16);
    if (n16 == 0)
        return hipSuccess;
    const long per_group = (long)kWave * unroll * waves_per_group;
    const long grid = groups > 0 ? groups : (n16 + per_group - 1) / per_group;
    const dim3 g((unsigned)grid), b((unsigned)(waves_per_group * kWave));
    const u32x4* p = static_cast<const u32x4*>(src);
    uint32_t* k = static_cast<uint32_t*>(sink);
    switch (unroll) {
    case 1: hipLaunchKernelGGL(moe_bench_read_cfg_kernel<1>, g, b, 0, s, p, n16, k); break;
    case 2: hipLaunchKernelGGL(moe_bench_read_cfg_kernel<2>, g, b, 0, s, p, n16, k); break;
    case 4: hipLaunchKernelGGL(moe_bench_read_cfg_kernel<4>, g, b, 0, s, p, n16, k); break;
    case 8: hipLaunchKernelGGL(moe_bench_read_cfg_kernel<8>, g, b, 0, s, p, n16, k); break;
    case 16: hipLaunchKernelGGL(moe_bench_read_cfg_kernel<16>, g, b, 0, s, p, n16, k); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_bench_copy(const void* src, void* dst, size_t bytes, hipStream_t s)
{
    const long n16 = (long)(bytes / 16);
    if (n16 == 0)
        return hipSuccess;
    hipLaunchKernelGGL(moe_bench_copy_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
    return hipGetLastError();
}

}  // namespace moed
