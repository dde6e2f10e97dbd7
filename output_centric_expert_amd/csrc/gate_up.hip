// Gate/up kernel of the two-launch layer: one wavefront per intermediate
// neuron of one (token, routed slot) pair -- the first of the two warp-decode
// kernels (warp-decode post, "How the two kernels work", first two
// paragraphs), laid out for 64-lane CDNA4 wavefronts. The per-wave work is
// gate_up_wave(); after it the 64 partials are reduced with DPP/ds_swizzle and
// one value SiLU(g)*u is stored at its place in the chunk-interleaved
// intermediate layout (inter_index).
#include "gate_up_body.h"

namespace moed {

template <int U, bool A_BF16, bool FP4>
__global__ void __launch_bounds__(256)
moe_gate_up_kernel(GateUpArgs p)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wpb = blockDim.x / kWave;
    const int n0 = __builtin_amdgcn_readfirstlane(blockIdx.x * wpb + (int)(threadIdx.x / kWave));
    if (n0 >= p.B * p.k * p.I)
        return;                                   // whole wavefront leaves together
    float g, u;
    bool bad_id;
    gate_up_wave<U, FP4>(p, n0, lane, g, u, bad_id);
    g = wave_sum(g);
    u = wave_sum(u);
    if (lane == 0) {
        const float v = bad_id ? __builtin_nanf("") : swiglu(g, u);
        const size_t a_idx = inter_index<A_BF16>(n0 / p.I, n0 % p.I, p.I);
        if constexpr (A_BF16)
            static_cast<uint16_t*>(p.a)[a_idx] = f32_to_bf16_rne(v);
        else
            static_cast<float*>(p.a)[a_idx] = v;
    }
}

// Exact-fit form for rows of exactly 64*U chunks (MXFP8: H a multiple of
// 1024; MXFP4: of 2048): every lane holds U whole chunks, so there is no clamping or lane
// factor, and the routed id is requested ahead of the activations so that its
// round trip overlaps theirs. The per-lane products, the order of the FMAs
// and the reduction are those of moe_gate_up_kernel (whose lane factor is 1
// here), so the values are the same floats.
//
// ORD 0: slot-major order (wavefront n takes slot n / I, neuron n % I).
// ORD 1, neuron-block order (for B > 1): wavefront n takes neuron block
// n / (16*S) (S = B*k slots), slot (n % (16*S)) / 16 and neuron n % 16 of the
// block, and each XCD runs a contiguous range of workgroups; the slots that
// share an expert then read the same rows on one XCD at about the same time,
// so the second read is served by that XCD's L2. ORD 2 (single token): slot-
// major with streaming (non-temporal) loads of the scale bytes as well; a
// single token reads every routed row once, and each further cached load per
// lane lengthens a launch whose loads are all in flight together (B = 1
// layer 10.56 -> 10.37 us MXFP8, 8.50 -> 8.26 us MXFP4; at B = 8, where
// tokens share rows, streaming scale loads measured 2-4% slower). Only the
// order of the work and the cache policy change, never the values.
template <int U, bool A_BF16, bool FP4, int ORD>
__global__ void __launch_bounds__(256)
moe_gate_up_exact_kernel(GateUpArgs p)
{
    constexpr bool NB = ORD == 1;
    constexpr bool NTS = ORD == 2;
    constexpr int NX = FP4 ? 4 : 2;               // 16-byte pieces of x per chunk
    const int lane = threadIdx.x & (kWave - 1);
    const int wpb = blockDim.x / kWave;
    const int n_out = p.B * p.k * p.I;
    const int wgi = NB ? xcd_contiguous((int)blockIdx.x, (int)gridDim.x) : (int)blockIdx.x;
    const int n_raw = __builtin_amdgcn_readfirstlane(wgi * wpb + (int)(threadIdx.x / kWave));
    const int n0 = n_raw < n_out ? n_raw : n_out - 1;   // no early exit; the extra waves store nothing
    int i0, bj;
    if constexpr (NB) {
        const int per_blk = 16 * p.B * p.k;
        const int r = n0 % per_blk;
        i0 = (n0 / per_blk) * 16 + r % 16;
        bj = r / 16;
    } else {
        i0 = n0 % p.I;
        bj = n0 / p.I;
    }
    const int b = bj / p.k;
    const int H = p.H;
    const size_t row_bytes = FP4 ? (size_t)(H / 2) : (size_t)H;
    const int e_raw = p.ids[bj];
    const u32x4* xq = reinterpret_cast<const u32x4*>(p.x + (size_t)b * (size_t)H);
    u32x4 xv[U][NX];
#pragma unroll
    for (int m = 0; m < U; ++m) {
#pragma unroll
        for (int t = 0; t < NX; ++t)
            xv[m][t] = xq[NX * (lane + kWave * m) + t];
    }
    __builtin_amdgcn_sched_barrier(0);
    const bool bad_id = (unsigned)e_raw >= (unsigned)p.E;   // expert 0's rows are read, result NaN
    const int e = bad_id ? 0 : e_raw;
    const size_t row = (size_t)e * (size_t)p.I + (size_t)i0;
    const u32x4* gq = reinterpret_cast<const u32x4*>(p.wg_q + row * row_bytes);
    const u32x4* uq = reinterpret_cast<const u32x4*>(p.wu_q + row * row_bytes);
    const uint8_t* gs = p.wg_s + row * (size_t)(H / 32);
    const uint8_t* us = p.wu_s + row * (size_t)(H / 32);
    u32x4 wg[U], wu[U];
    uint32_t sg[U], su[U];
#pragma unroll
    for (int m = 0; m < U; ++m) {
        const int c = lane + kWave * m;
        wg[m] = __builtin_nontemporal_load(gq + c);
        wu[m] = __builtin_nontemporal_load(uq + c);
        sg[m] = ld<NTS>(gs + (FP4 ? c : c >> 1));
        su[m] = ld<NTS>(us + (FP4 ? c : c >> 1));
    }
    float g = 0.0f, u = 0.0f;
#pragma unroll
    for (int m = 0; m < U; ++m) {
        const float pg = gu_chunk_dot<FP4, NX>(wg[m], xv[m]);
        const float pu = gu_chunk_dot<FP4, NX>(wu[m], xv[m]);
        g = __builtin_fmaf(pg, ue8m0_to_f32(sg[m]), g);
        u = __builtin_fmaf(pu, ue8m0_to_f32(su[m]), u);
    }
    g = wave_sum(g);
    u = wave_sum(u);
    if (lane == 0 && n_raw < n_out) {
        const float v = bad_id ? __builtin_nanf("") : swiglu(g, u);
        const size_t a_idx = inter_index<A_BF16>(bj, i0, p.I);
        if constexpr (A_BF16)
            static_cast<uint16_t*>(p.a)[a_idx] = f32_to_bf16_rne(v);
        else
            static_cast<float*>(p.a)[a_idx] = v;
    }
}

// Exact-fit form with two neighbouring neurons i0, i0+1 of one slot per
// wavefront (x loaded once for both; four row loads per lane chunk), for
// MXFP4 rows at B > 1: an MXFP4 row is half as long, so one neuron per
// wavefront keeps only two 16-byte loads per lane in flight (B = 8 gate/up
// 18.6 vs 20.0 us; at B = 1 the same, and slower for MXFP8, whose rows
// already give four loads per lane). Per neuron the products, the FMA order
// and the reduction are those of moe_gate_up_exact_kernel: the same floats.
template <int U, bool A_BF16, bool FP4>
__global__ void __launch_bounds__(256)
moe_gate_up_exact_pair_kernel(GateUpArgs p)
{
    constexpr int NX = FP4 ? 4 : 2;               // 16-byte pieces of x per chunk
    const int lane = threadIdx.x & (kWave - 1);
    const int wpb = blockDim.x / kWave;
    const int n_pairs = p.B * p.k * (p.I / 2);
    const int n_raw = __builtin_amdgcn_readfirstlane((int)blockIdx.x * wpb + (int)(threadIdx.x / kWave));
    const int n0 = n_raw < n_pairs ? n_raw : n_pairs - 1;   // no early exit; the extra waves store nothing
    const int i0 = 2 * (n0 % (p.I / 2));
    const int bj = n0 / (p.I / 2);
    const int b = bj / p.k;
    const int H = p.H;
    const size_t row_bytes = FP4 ? (size_t)(H / 2) : (size_t)H;
    const int e_raw = p.ids[bj];
    const u32x4* xq = reinterpret_cast<const u32x4*>(p.x + (size_t)b * (size_t)H);
    u32x4 xv[U][NX];
#pragma unroll
    for (int m = 0; m < U; ++m) {
#pragma unroll
        for (int t = 0; t < NX; ++t)
            xv[m][t] = xq[NX * (lane + kWave * m) + t];
    }
    __builtin_amdgcn_sched_barrier(0);
    const bool bad_id = (unsigned)e_raw >= (unsigned)p.E;   // expert 0's rows are read, result NaN
    const int e = bad_id ? 0 : e_raw;
    u32x4 wg[2][U], wu[2][U];
    uint32_t sg[2][U], su[2][U];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const size_t row = (size_t)e * (size_t)p.I + (size_t)(i0 + n);
        const u32x4* gq = reinterpret_cast<const u32x4*>(p.wg_q + row * row_bytes);
        const u32x4* uq = reinterpret_cast<const u32x4*>(p.wu_q + row * row_bytes);
        const uint8_t* gs = p.wg_s + row * (size_t)(H / 32);
        const uint8_t* us = p.wu_s + row * (size_t)(H / 32);
#pragma unroll
        for (int m = 0; m < U; ++m) {
            const int c = lane + kWave * m;
            wg[n][m] = __builtin_nontemporal_load(gq + c);
            wu[n][m] = __builtin_nontemporal_load(uq + c);
            sg[n][m] = gs[FP4 ? c : c >> 1];
            su[n][m] = us[FP4 ? c : c >> 1];
        }
    }
    float g[2], u[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        g[n] = 0.0f;
        u[n] = 0.0f;
#pragma unroll
        for (int m = 0; m < U; ++m) {
            const float pg = gu_chunk_dot<FP4, NX>(wg[n][m], xv[m]);
            const float pu = gu_chunk_dot<FP4, NX>(wu[n][m], xv[m]);
            g[n] = __builtin_fmaf(pg, ue8m0_to_f32(sg[n][m]), g[n]);
            u[n] = __builtin_fmaf(pu, ue8m0_to_f32(su[n][m]), u[n]);
        }
        g[n] = wave_sum(g[n]);
        u[n] = wave_sum(u[n]);
    }
    if (lane == 0 && n_raw < n_pairs) {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const float v = bad_id ? __builtin_nanf("") : swiglu(g[n], u[n]);
            const size_t a_idx = inter_index<A_BF16>(bj, i0 + n, p.I);
            if constexpr (A_BF16)
                static_cast<uint16_t*>(p.a)[a_idx] = f32_to_bf16_rne(v);
            else
                static_cast<float*>(p.a)[a_idx] = v;
        }
    }
}

template <bool A_BF16>
static hipError_t dispatch_pair(int U, const GateUpArgs& p, dim3 grid, dim3 block, hipStream_t s)
{
    switch (U) {
#define MOED_GUP_CASE(N) \
    case N: hipLaunchKernelGGL((moe_gate_up_exact_pair_kernel<N, A_BF16, true>), grid, block, 0, s, p); break;
        MOED_GUP_CASE(1) MOED_GUP_CASE(2) MOED_GUP_CASE(3) MOED_GUP_CASE(4)
#undef MOED_GUP_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool A_BF16, bool FP4>
static hipError_t dispatch_exact(int U, int ord, const GateUpArgs& p, dim3 grid, dim3 block, hipStream_t s)
{
    switch (U) {
#define MOED_GUX_CASE(N)                                                                              \
    case N:                                                                                            \
        if (ord == 1)                                                                                  \
            hipLaunchKernelGGL((moe_gate_up_exact_kernel<N, A_BF16, FP4, 1>), grid, block, 0, s, p);   \
        else if (ord == 2)                                                                             \
            hipLaunchKernelGGL((moe_gate_up_exact_kernel<N, A_BF16, FP4, 2>), grid, block, 0, s, p);   \
        else                                                                                           \
            hipLaunchKernelGGL((moe_gate_up_exact_kernel<N, A_BF16, FP4, 0>), grid, block, 0, s, p);   \
        break;
        MOED_GUX_CASE(1) MOED_GUX_CASE(2) MOED_GUX_CASE(3) MOED_GUX_CASE(4)
        MOED_GUX_CASE(5) MOED_GUX_CASE(6) MOED_GUX_CASE(7) MOED_GUX_CASE(8)
#undef MOED_GUX_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool A_BF16, bool FP4>
static hipError_t dispatch_u(int U, const GateUpArgs& p, dim3 grid, dim3 block, hipStream_t s)
{
    switch (U) {
#define MOED_GU_CASE(N) \
    case N: hipLaunchKernelGGL((moe_gate_up_kernel<N, A_BF16, FP4>), grid, block, 0, s, p); break;
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
    int U = (nch + kWave - 1) / kWave;
    if (U > t.gu_umax)
        U = t.gu_umax;
    if (U < 1)
        U = 1;
    const int wpb = t.gu_wpb;
    const dim3 block(wpb * kWave);
    const dim3 grid((unsigned)((n_out + wpb - 1) / wpb));
    // rows of exactly 64*U chunks, U <= gu_umax: the exact-fit kernel
    if (t.gu_exact != 0 && nch == kWave * U) {
        // neuron-block order where slots may share experts (B > 1); by default for
        // MXFP8 only (measured 3-4% faster at B = 8-16 there, 2% slower for MXFP4)
        const bool nb = (t.gu_order == 2 || (t.gu_order == 1 && !fp4)) && p.B > 1 && p.I % 16 == 0;
        // MXFP4 at B > 1 (unless neuron-block order is asked for): two neurons per wavefront
        if (fp4 && !nb && t.gu_pair != 0 && p.B > 1 && p.I % 2 == 0 && U <= 4) {
            const dim3 g2((unsigned)((n_out / 2 + wpb - 1) / wpb));
            return a_bf16 ? dispatch_pair<true>(U, p, g2, block, s) : dispatch_pair<false>(U, p, g2, block, s);
        }
        const int ord = nb ? 1 : (p.B == 1 ? 2 : 0);
        if (fp4)
            return a_bf16 ? dispatch_exact<true, true>(U, ord, p, grid, block, s)
                          : dispatch_exact<false, true>(U, ord, p, grid, block, s);
        return a_bf16 ? dispatch_exact<true, false>(U, ord, p, grid, block, s)
                      : dispatch_exact<false, false>(U, ord, p, grid, block, s);
    }
    if (fp4)
        return a_bf16 ? dispatch_u<true, true>(U, p, grid, block, s) : dispatch_u<false, true>(U, p, grid, block, s);
    return a_bf16 ? dispatch_u<true, false>(U, p, grid, block, s) : dispatch_u<false, false>(U, p, grid, block, s);
}

}  // namespace moed
