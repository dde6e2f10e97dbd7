// Opt-in input check (environment variable MOED_CHECK=1): the preconditions
// the layer does not check on its hot path -- every routed expert id in
// [0, E), and no NaN code (E4M3 S.1111.111) or NaN scale (UE8M0 0xFF) in the
// rows of the experts that are routed to. E2M1 has no NaN code; its scales
// are checked. It also flags block scales of routed experts outside the range
// the large-batch kernels decode exactly (they fold the scale into the BF16
// conversion), separately for the gate/up and the down matrices, so that the
// caller can reject only the calls that take those kernels. The result is a
// flag word (kCheck* bits) in a file-scope device array: no allocation.
#include <mutex>

#include "launch.h"
#include "mx_device.h"

namespace moed {

namespace {
__device__ __align__(256) uint32_t check_flag_word[64];
}

// Per-device facts are kept in fixed tables (no heap allocation, so that the
// entry point for callers that cannot allocate may use them too).
hipError_t check_flag(uint32_t** flag)
{
    static std::mutex mu;
    static uint32_t* addr[kMaxDevices] = {};      // per device: the array's address on it
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return err;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(check_flag_word));
        if (err != hipSuccess)
            return err;
        addr[dev] = static_cast<uint32_t*>(p);
    }
    *flag = addr[dev];
    return hipSuccess;
}

hipError_t set_max_dynamic_lds(const void* func, int bytes)
{
    struct Entry {
        int dev;
        const void* func;
        int bytes;
    };
    constexpr int kSlots = 256;                   // (device, kernel) pairs: a handful of kernels per device
    static std::mutex mu;
    static Entry done[kSlots];
    static int used = 0;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return err;
    std::lock_guard<std::mutex> lock(mu);
    int slot = -1;
    for (int i = 0; i < used; ++i) {
        if (done[i].dev == dev && done[i].func == func) {
            if (done[i].bytes >= bytes)
                return hipSuccess;
            slot = i;
        }
    }
    err = hipFuncSetAttribute(func, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (err != hipSuccess)
        return err;
    if (slot < 0 && used < kSlots)
        slot = used++;
    if (slot >= 0)
        done[slot] = Entry{dev, func, bytes};
    return hipSuccess;
}

__global__ void moe_check_clear_kernel(uint32_t* flag)
{
    if (threadIdx.x == 0)
        flag[0] = 0u;
}

// Grid (E, parts): block (e, part) scans rows part, part + parts, ... of
// expert e's three matrices if some slot is routed to e; block (0, 0) also
// checks the ids.
__global__ void __launch_bounds__(256)
moe_check_kernel(const int32_t* ids, int nslots, int E, const uint8_t* wg_q, const uint8_t* wg_s,
                 const uint8_t* wu_q, const uint8_t* wu_s, const uint8_t* wd_q, const uint8_t* wd_s, int H,
                 int I, int fp4, uint32_t* flag)
{
    __shared__ int routed;
    const int e = blockIdx.x;
    const int part = blockIdx.y;
    const int parts = gridDim.y;
    if (threadIdx.x == 0)
        routed = 0;
    __syncthreads();
    bool bad_id = false;
    for (int t = threadIdx.x; t < nslots; t += blockDim.x) {
        const int v = ids[t];
        if (v == e)
            routed = 1;                               // benign race: every writer stores 1
        bad_id |= (unsigned)v >= (unsigned)E;
    }
    if (bad_id && e == 0 && part == 0)
        atomicOr(flag, kCheckBadId);
    __syncthreads();
    if (!routed)
        return;                                       // whole block
    bool bad = false;
    bool range_gu = false, range_dn = false;
    const uint32_t lo = fp4 ? kExactScaleLoFP4 : kExactScaleLoFP8;
    const uint32_t hi = fp4 ? kExactScaleHiFP4 : kExactScaleHiFP8;
    // codes: rows of K bytes (K/2 for E2M1, which has no NaN code)
    auto scan_codes = [&](const uint8_t* q, int rows, int K) {
        if (fp4 || !q)
            return;
        const size_t base = (size_t)e * (size_t)rows * (size_t)K;
        for (int r = part; r < rows; r += parts)
            for (int c = threadIdx.x; c < K; c += blockDim.x)
                bad |= (q[base + (size_t)r * K + c] & 0x7Fu) == 0x7Fu;
    };
    auto scan_scales = [&](const uint8_t* s, int rows, int K, bool& range) {
        if (!s)
            return;
        const size_t base = (size_t)e * (size_t)rows * (size_t)(K / 32);
        for (int r = part; r < rows; r += parts)
            for (int c = threadIdx.x; c < K / 32; c += blockDim.x) {
                const uint32_t v = s[base + (size_t)r * (K / 32) + c];
                bad |= v == 0xFFu;
                range |= v != 0xFFu && (v < lo || v > hi);
            }
    };
    scan_codes(wg_q, I, H);
    scan_codes(wu_q, I, H);
    scan_codes(wd_q, H, I);
    scan_scales(wg_s, I, H, range_gu);
    scan_scales(wu_s, I, H, range_gu);
    scan_scales(wd_s, H, I, range_dn);
    if (bad)
        atomicOr(flag, kCheckNaN);
    if (range_gu)
        atomicOr(flag, kCheckScaleGateUp);
    if (range_dn)
        atomicOr(flag, kCheckScaleDown);
}

hipError_t launch_check(const CheckArgs& c, uint32_t* flag, hipStream_t s)
{
    hipLaunchKernelGGL(moe_check_clear_kernel, dim3(1), dim3(64), 0, s, flag);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    const dim3 grid((unsigned)c.E, 64u), block(256);
    hipLaunchKernelGGL(moe_check_kernel, grid, block, 0, s, c.ids, c.B * c.k, c.E, c.wg_q, c.wg_s, c.wu_q, c.wu_s,
                       c.wd_q, c.wd_s, c.H, c.I, c.wfmt == kMXFP4 ? 1 : 0, flag);
    return hipGetLastError();
}

}  // namespace moed
