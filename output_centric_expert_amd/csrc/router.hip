// Router front-end: softmax -> top-k -> renormalise on the GPU, plus the
// shared-expert slots, writing the topk_ids / topk_w rows the layer kernels
// read (the routing recipe the warp-decode layer consumes; shared experts as
// in the GC-MoE summary's fused epilogue, onedev.kr/papers/1690, "How to
// use").
//
// One wavefront per token. Experts are ordered by 64-bit keys: an
// order-preserving map of the float32 logit in the high word and
// (2^32 - 1 - id) in the low word, so a larger key is a larger logit and,
// among equal logits, a lower expert id. +0 and -0 map to the same key; a NaN
// logit maps to key 0 and is never selected. Softmax is strictly increasing,
// so the k largest keys are the top-k routing probabilities, in descending
// order. Round j takes the wave-wide maximum key over the experts not yet
// taken (DPP / ds_swizzle exchanges, no LDS memory); its owner lane marks it
// taken and lane j keeps it. The routed weights are exp(l_j - m) / sum_j' exp(l_j' - m)
// (m = the largest selected logit) times routed_scale; shared slot s gets id
// E + s and weight 1. If fewer than k experts can be selected (NaN logits),
// the missing slots get id -1 (an id the layer turns into NaN outputs) and a
// NaN weight.
#include "launch.h"
#include "mx_device.h"

namespace moed {

namespace {

__device__ __forceinline__ uint64_t route_key(float v, int e)
{
    if (v != v)
        return 0ull;                              // NaN: never selected
    uint32_t u = v == 0.0f ? 0u : __float_as_uint(v);
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ float key_value(uint64_t key)
{
    const uint32_t ord = (uint32_t)(key >> 32);
    const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
    return __uint_as_float(u);
}

__device__ __forceinline__ int key_id(uint64_t key)
{
    return (int)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull));
}

// One exchange step of the 64-bit maximum: both halves moved by the same DPP
// pattern, then the larger key kept.
template <int CTRL>
__device__ __forceinline__ uint64_t max_dpp(uint64_t v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, true);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    return o > v ? o : v;
}

// Maximum of a 64-bit key over the 64 lanes (every lane gets it), with the
// exchange pattern of wave_sum: DPP quad_perm xor 1 and xor 2, row_half_mirror
// and row_mirror inside each 16-lane row, a ds_swizzle (lane ^ 16) between row
// pairs, and the two 32-lane halves through readlane. All lanes must be active.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
    v = max_dpp<0xB1>(v);                         // quad_perm [1,0,3,2]
    v = max_dpp<0x4E>(v);                         // quad_perm [2,3,0,1]
    v = max_dpp<0x141>(v);                        // row_half_mirror
    v = max_dpp<0x140>(v);                        // row_mirror
    {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_swizzle((int)(uint32_t)v, (0x10 << 10) | 0x1F);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_swizzle((int)(uint32_t)(v >> 32), (0x10 << 10) | 0x1F);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    const uint64_t a = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 0) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 0);
    const uint64_t c = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 32) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 32);
    return a > c ? a : c;
}

}  // namespace

template <int NPL>                                // logits held per lane (E <= 64 * NPL)
__global__ void __launch_bounds__(256)
moe_route_kernel(const float* logits, int B, int E, int k, int n_shared, float routed_scale, int32_t* ids,
                 float* w)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int b = (int)(blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave);
    if (b >= B)
        return;                                   // whole wavefront
    const float* l = logits + (size_t)b * E;
    uint64_t key[NPL];
#pragma unroll
    for (int t = 0; t < NPL; ++t) {
        const int e = lane + kWave * t;
        key[t] = e < E ? route_key(l[e], e) : 0ull;
    }
    uint32_t taken = 0;                           // bit t: expert lane + 64t selected
    uint64_t mine = 0;                            // lane j: the key of round j
    uint64_t first = 0;
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int t = 0; t < NPL; ++t)
            if (!((taken >> t) & 1u) && key[t] > best)
                best = key[t];
        best = wave_max_u64(best);
        if (best != 0ull) {
            const int e = key_id(best);
            if ((e & (kWave - 1)) == lane)
                taken |= 1u << (e / kWave);
        }
        if (lane == j)
            mine = best;
        if (j == 0)
            first = best;
    }
    const int kt = k + n_shared;
    const float m = key_value(first);
    const bool ok = lane < k && mine != 0ull;
    const float ex = ok ? expf(key_value(mine) - m) : 0.0f;
    const float sum = wave_sum(ex);
    if (lane < k) {
        ids[(size_t)b * kt + lane] = ok ? key_id(mine) : -1;
        w[(size_t)b * kt + lane] = ok ? ex / sum * routed_scale : __builtin_nanf("");
    }
    for (int s = lane; s < n_shared; s += kWave) {
        ids[(size_t)b * kt + k + s] = E + s;
        w[(size_t)b * kt + k + s] = 1.0f;
    }
}

hipError_t launch_route(const float* logits, int B, int E, int k, int n_shared, float routed_scale, int32_t* ids,
                        float* w, hipStream_t s)
{
    if (B == 0)
        return hipSuccess;
    const int per_lane = (E + kWave - 1) / kWave;
    constexpr int wpb = 4;
    const dim3 grid((unsigned)((B + wpb - 1) / wpb)), block(wpb * kWave);
#define MOED_RT(N) \
    hipLaunchKernelGGL((moe_route_kernel<N>), grid, block, 0, s, logits, B, E, k, n_shared, routed_scale, ids, w)
    if (per_lane <= 1) MOED_RT(1);
    else if (per_lane <= 2) MOED_RT(2);
    else if (per_lane <= 4) MOED_RT(4);
    else if (per_lane <= 8) MOED_RT(8);
    else if (per_lane <= 16) MOED_RT(16);
    else if (per_lane <= 32) MOED_RT(32);
    else return hipErrorInvalidValue;
#undef MOED_RT
    return hipGetLastError();
}

}  // namespace moed
