// Gate/up kernel of the two-launch layer: one wavefront per intermediate
// neuron of one (token, routed slot) pair -- the first of the two warp-decode
// kernels (warp-decode post, "How the two kernels work", first two
// paragraphs), laid out for 64-lane CDNA4 wavefronts. The per-wave work is
// gate_up_wave(); after it the 64 partials are reduced with DPP/ds_swizzle and
// one value SiLU(g)*u is stored at its place in the chunk-interleaved
// intermediate layout (inter_index).
#include "gate_up_body.h"

namespace moed {

template <int U, bool DOT_BF16, bool A_BF16, bool NT, bool FP4, int NPW>
__global__ void __launch_bounds__(256)
moe_gate_up_kernel(GateUpArgs p)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wpb = blockDim.x / kWave;
    const int wave = __builtin_amdgcn_readfirstlane(blockIdx.x * wpb + (int)(threadIdx.x / kWave));
    const int n_out = p.B * p.k * p.I;
    const int n0 = wave * NPW;                    // first of the wave's NPW neurons
    if (n0 >= n_out)
        return;                                   // whole wavefront leaves together
    float g[NPW], u[NPW];
    bool bad_id;
    gate_up_wave<U, DOT_BF16, NT, FP4, NPW>(p, n0, lane, g, u, bad_id);
#pragma unroll
    for (int n = 0; n < NPW; ++n) {
        g[n] = wave_sum(g[n]);
        u[n] = wave_sum(u[n]);
    }
    if (lane == 0) {
#pragma unroll
        for (int n = 0; n < NPW; ++n) {
            const float v = bad_id ? __builtin_nanf("") : swiglu(g[n], u[n]);
            const size_t a_idx = inter_index<A_BF16>((n0 + n) / p.I, (n0 + n) % p.I, p.I);
            if constexpr (A_BF16)
                static_cast<uint16_t*>(p.a)[a_idx] = f32_to_bf16_rne(v);
            else
                static_cast<float*>(p.a)[a_idx] = v;
        }
    }
}

template <bool DOT_BF16, bool A_BF16, bool NT, bool FP4>
static hipError_t dispatch_u(int U, int npw, const GateUpArgs& p, dim3 grid, dim3 block, hipStream_t s)
{
    if (npw == 2) {                               // two neurons per wave: U <= 4
        switch (U) {
#define MOED_GU2_CASE(N) \
        case N: hipLaunchKernelGGL((moe_gate_up_kernel<N, DOT_BF16, A_BF16, NT, FP4, 2>), grid, block, 0, s, p); break;
            MOED_GU2_CASE(1) MOED_GU2_CASE(2) MOED_GU2_CASE(3) MOED_GU2_CASE(4)
#undef MOED_GU2_CASE
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    switch (U) {
#define MOED_GU_CASE(N) \
    case N: hipLaunchKernelGGL((moe_gate_up_kernel<N, DOT_BF16, A_BF16, NT, FP4, 1>), grid, block, 0, s, p); break;
        MOED_GU_CASE(1) MOED_GU_CASE(2) MOED_GU_CASE(3) MOED_GU_CASE(4)
        MOED_GU_CASE(5) MOED_GU_CASE(6) MOED_GU_CASE(7) MOED_GU_CASE(8)
#undef MOED_GU_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gate_up(const GateUpArgs& p, bool a_bf16, const Tuning& t, hipStream_t s)
{
    const long n_out = (long)p.B * p.k * p.I;
    if (n_out == 0)
        return hipSuccess;
    const bool fp4 = p.wfmt == kMXFP4;
    const int nch = fp4 ? p.H / 32 : p.H / 16;    // 16-byte chunks per row
    // neurons per wavefront: 2 shares each x load between two rows (decode route 1 only)
    const int npw = (t.gu_npw == 2 && (t.gu_dot != 0 || fp4)) ? 2 : 1;
    int U = (nch + kWave - 1) / kWave;
    const int umax = npw == 2 ? (t.gu_umax < 4 ? t.gu_umax : 4) : t.gu_umax;
    if (U > umax)
        U = umax;
    if (U < 1)
        U = 1;
    const int wpb = t.gu_wpb;
    const long n_waves = (n_out + npw - 1) / npw;
    const dim3 block(wpb * kWave);
    const dim3 grid((unsigned)((n_waves + wpb - 1) / wpb));
    const bool dot = t.gu_dot != 0, nt = t.nt != 0;
    if (fp4) {                                    // one decode route (BF16 dot2)
        if (a_bf16) return nt ? dispatch_u<true, true, true, true>(U, npw, p, grid, block, s)
                              : dispatch_u<true, true, false, true>(U, npw, p, grid, block, s);
        return nt ? dispatch_u<true, false, true, true>(U, npw, p, grid, block, s)
                  : dispatch_u<true, false, false, true>(U, npw, p, grid, block, s);
    }
    if (dot) {
        if (a_bf16) return nt ? dispatch_u<true, true, true, false>(U, npw, p, grid, block, s)
                              : dispatch_u<true, true, false, false>(U, npw, p, grid, block, s);
        return nt ? dispatch_u<true, false, true, false>(U, npw, p, grid, block, s)
                  : dispatch_u<true, false, false, false>(U, npw, p, grid, block, s);
    }
    if (a_bf16) return nt ? dispatch_u<false, true, true, false>(U, 1, p, grid, block, s)
                          : dispatch_u<false, true, false, false>(U, 1, p, grid, block, s);
    return nt ? dispatch_u<false, false, true, false>(U, 1, p, grid, block, s)
              : dispatch_u<false, false, false, false>(U, 1, p, grid, block, s);
}

}  // namespace moed
