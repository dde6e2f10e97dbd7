// Gate/up kernel: one wavefront per intermediate neuron of one (token, routed
// slot) pair -- the first of the two warp-decode kernels (warp-decode post,
// "How the two kernels work", first two paragraphs), laid out for 64-lane
// CDNA4 wavefronts.
//
// Wave w owns (b, j, i) with w = (b*k + j)*I + i. It first issues the loads
// of its 16 bf16 activations per chunk, x[b][16c..16c+15] (used by both
// projections), then reads e = ids[b][j] with a scalar load and streams the
// gate row Wg[e][i][:] and the up row Wu[e][i][:] in 16-byte chunks: chunk c
// (16 codes) goes to lane c % 64, so each wave-wide load instruction covers
// 1 KiB of one row contiguously. Every load of a pass is issued before the
// first FMA, without branches around them.
// Each lane keeps two FP32 accumulators (gate, up); after the row the 64
// partials are reduced with DPP/ds_swizzle and one value SiLU(g)*u is stored,
// at its place in the chunk-interleaved intermediate layout (inter_index).
#include "launch.h"
#include "mx_device.h"

namespace moed {

template <int U, bool DOT_BF16, bool A_BF16, bool NT>
__global__ void __launch_bounds__(256)
moe_gate_up_kernel(GateUpArgs p)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wpb = blockDim.x / kWave;
    const int wave = __builtin_amdgcn_readfirstlane(blockIdx.x * wpb + (int)(threadIdx.x / kWave));
    const int n_out = p.B * p.k * p.I;
    if (wave >= n_out)
        return;                                   // whole wavefront leaves together
    const int i = wave % p.I;
    const int bj = wave / p.I;
    const int b = bj / p.k;
    const int H = p.H;
    const int nch = H / 16;                       // 16-code chunks per row
    const u32x4* xq = reinterpret_cast<const u32x4*>(p.x + (size_t)b * (size_t)H);

    float g = 0.0f, u = 0.0f;
    bool bad_id = false;
    for (int base = 0; base < nch; base += kWave * U) {
        // x first: its address does not depend on the routed id, so these loads
        // overlap the id's scalar load. Every load is unconditional from a
        // clamped, in-bounds address; chunks past the row end get scale 0.
        u32x4 xa[U], xb[U];
#pragma unroll
        for (int m = 0; m < U; ++m) {
            const int c = base + lane + kWave * m;
            const int cc = c < nch ? c : nch - 1;
            xa[m] = xq[2 * cc];
            xb[m] = xq[2 * cc + 1];
        }
        __builtin_amdgcn_sched_barrier(0);
        const int e_raw = p.ids[bj];
        bad_id = (unsigned)e_raw >= (unsigned)p.E;   // invalid routing: expert 0's rows are read, result NaN
        const int e = bad_id ? 0 : e_raw;
        const size_t row = (size_t)e * (size_t)p.I + (size_t)i;
        const u32x4* gq = reinterpret_cast<const u32x4*>(p.wg_q + row * (size_t)H);
        const u32x4* uq = reinterpret_cast<const u32x4*>(p.wu_q + row * (size_t)H);
        const uint8_t* gs = p.wg_s + row * (size_t)(H / 32);
        const uint8_t* us = p.wu_s + row * (size_t)(H / 32);
        u32x4 wg[U], wu[U];
        uint32_t sg[U], su[U];
        float live[U];
#pragma unroll
        for (int m = 0; m < U; ++m) {
            const int c = base + lane + kWave * m;
            const int cc = c < nch ? c : nch - 1;
            wg[m] = ld<NT>(gq + cc);
            wu[m] = ld<NT>(uq + cc);
            sg[m] = gs[cc >> 1];
            su[m] = us[cc >> 1];
            live[m] = c < nch ? 1.0f : 0.0f;
        }
#pragma unroll
        for (int m = 0; m < U; ++m) {
            float pg = 0.0f, pu = 0.0f;
            if constexpr (DOT_BF16) {
                pg = dot4_bf16(wg[m].x, xa[m].x, xa[m].y, pg);
                pu = dot4_bf16(wu[m].x, xa[m].x, xa[m].y, pu);
                pg = dot4_bf16(wg[m].y, xa[m].z, xa[m].w, pg);
                pu = dot4_bf16(wu[m].y, xa[m].z, xa[m].w, pu);
                pg = dot4_bf16(wg[m].z, xb[m].x, xb[m].y, pg);
                pu = dot4_bf16(wu[m].z, xb[m].x, xb[m].y, pu);
                pg = dot4_bf16(wg[m].w, xb[m].z, xb[m].w, pg);
                pu = dot4_bf16(wu[m].w, xb[m].z, xb[m].w, pu);
            } else {
                pg = dot4_f32(wg[m].x, xa[m].x, xa[m].y, pg);
                pu = dot4_f32(wu[m].x, xa[m].x, xa[m].y, pu);
                pg = dot4_f32(wg[m].y, xa[m].z, xa[m].w, pg);
                pu = dot4_f32(wu[m].y, xa[m].z, xa[m].w, pu);
                pg = dot4_f32(wg[m].z, xb[m].x, xb[m].y, pg);
                pu = dot4_f32(wu[m].z, xb[m].x, xb[m].y, pu);
                pg = dot4_f32(wg[m].w, xb[m].z, xb[m].w, pg);
                pu = dot4_f32(wu[m].w, xb[m].z, xb[m].w, pu);
            }
            g = __builtin_fmaf(pg, ue8m0_to_f32(sg[m]) * live[m], g);
            u = __builtin_fmaf(pu, ue8m0_to_f32(su[m]) * live[m], u);
        }
    }
    g = wave_sum(g);
    u = wave_sum(u);
    if (lane == 0) {
        const float v = bad_id ? __builtin_nanf("") : swiglu(g, u);
        const size_t a_idx = inter_index<A_BF16>(bj, i, p.I);
        if constexpr (A_BF16)
            static_cast<uint16_t*>(p.a)[a_idx] = f32_to_bf16_rne(v);
        else
            static_cast<float*>(p.a)[a_idx] = v;
    }
}

template <bool DOT_BF16, bool A_BF16, bool NT>
static hipError_t dispatch_u(int U, const GateUpArgs& p, dim3 grid, dim3 block, hipStream_t s)
{
    switch (U) {
#define MOED_GU_CASE(N) \
    case N: hipLaunchKernelGGL((moe_gate_up_kernel<N, DOT_BF16, A_BF16, NT>), grid, block, 0, s, p); break;
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
    const int nch = p.H / 16;
    int U = (nch + kWave - 1) / kWave;
    if (U > t.gu_umax)
        U = t.gu_umax;
    if (U < 1)
        U = 1;
    const int wpb = t.gu_wpb;
    const dim3 block(wpb * kWave);
    const dim3 grid((unsigned)((n_out + wpb - 1) / wpb));
    const bool dot = t.gu_dot != 0, nt = t.nt != 0;
    if (dot) {
        if (a_bf16) return nt ? dispatch_u<true, true, true>(U, p, grid, block, s)
                              : dispatch_u<true, true, false>(U, p, grid, block, s);
        return nt ? dispatch_u<true, false, true>(U, p, grid, block, s)
                  : dispatch_u<true, false, false>(U, p, grid, block, s);
    }
    if (a_bf16) return nt ? dispatch_u<false, true, true>(U, p, grid, block, s)
                          : dispatch_u<false, true, false>(U, p, grid, block, s);
    return nt ? dispatch_u<false, false, true>(U, p, grid, block, s)
              : dispatch_u<false, false, false>(U, p, grid, block, s);
}

}  // namespace moed
