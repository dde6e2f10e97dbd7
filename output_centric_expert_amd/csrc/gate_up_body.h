// Per-wave body of the general per-slot gate/up kernel (one wavefront per
// intermediate neuron of one (token, routed slot) pair; warp-decode post, "How
// the two kernels work", first two paragraphs); the exact-fit kernel uses the
// same chunk dot.
//
// Wave w owns (b, j, i) with w = (b*k + j)*I + i. It first issues the loads
// of its 16 bf16 activations per chunk, x[b][16c..16c+15] (used by both
// projections), then reads e = ids[b][j] with a scalar load and streams the
// gate row Wg[e][i][:] and the up row Wu[e][i][:] in 16-byte chunks: chunk c
// (16 codes) goes to lane c % 64, so each wave-wide load instruction covers
// 1 KiB of one row contiguously (MXFP4: a chunk is 32 codes, one MX block).
// Every load of a pass is issued before the
// first FMA, without branches around them. Each lane keeps two FP32
// accumulators (gate, up); the caller reduces them across the wavefront.
#pragma once

#include "launch.h"
#include "mx_device.h"

namespace moed {

// Partial dot (scale 1) of one 16-byte chunk of a gate or up row with its x
// pieces: 16 MXFP8 codes against 16 activations (x pieces 0, 1) or 32 MXFP4
// codes against 32 (pieces 0..3; dword d of the chunk = codes 8d..8d+7).
// Decode route: FP8/FP4 -> BF16 (exact) and BF16 dot2 with FP32 accumulation.
template <bool FP4, int NX>
__device__ __forceinline__ float gu_chunk_dot(const u32x4& w, const u32x4 (&x)[NX])
{
    float p = 0.0f;
    if constexpr (FP4) {
        p = dot8_fp4_bf16(w.x, x[0], p);
        p = dot8_fp4_bf16(w.y, x[1], p);
        p = dot8_fp4_bf16(w.z, x[2], p);
        p = dot8_fp4_bf16(w.w, x[3], p);
    } else {
        p = dot4_bf16(w.x, x[0].x, x[0].y, p);
        p = dot4_bf16(w.y, x[0].z, x[0].w, p);
        p = dot4_bf16(w.z, x[NX - 1].x, x[NX - 1].y, p);
        p = dot4_bf16(w.w, x[NX - 1].z, x[NX - 1].w, p);
    }
    return p;
}

// Lane partials of g = Wg[e][i]·x[b] and u = Wu[e][i]·x[b] for neuron
// i = n0 % I of slot bj = n0 / I; bad_id is set when ids[b][j] is outside
// [0, E) (the caller then stores NaN). FP4: MXFP4 weights -- a 16-byte chunk
// is 32 codes (one MX block, one scale byte) against 32 activations; MXFP8:
// 16 codes (half a block) against 16.
template <int U, bool FP4>
__device__ __forceinline__ void gate_up_wave(const GateUpArgs& p, int n0, int lane, float& g_out, float& u_out,
                                             bool& bad_out)
{
    constexpr int NX = FP4 ? 4 : 2;               // 16-byte pieces of x per chunk
    const int i0 = n0 % p.I;
    const int bj = n0 / p.I;
    const int b = bj / p.k;
    const int H = p.H;
    const int nch = FP4 ? H / 32 : H / 16;        // 16-byte chunks per row
    const size_t row_bytes = FP4 ? (size_t)(H / 2) : (size_t)H;
    const u32x4* xq = reinterpret_cast<const u32x4*>(p.x + (size_t)b * (size_t)H);

    float g = 0.0f, u = 0.0f;
    bool bad_id = false;
    for (int base = 0; base < nch; base += kWave * U) {
        // x first: its address does not depend on the routed id, so these loads
        // overlap the id's scalar load. Every load is unconditional from a
        // clamped, in-bounds address; chunks past the row end get scale 0.
        u32x4 xv[U][NX];
#pragma unroll
        for (int m = 0; m < U; ++m) {
            const int c = base + lane + kWave * m;
            const int cc = c < nch ? c : nch - 1;
#pragma unroll
            for (int t = 0; t < NX; ++t)
                xv[m][t] = xq[NX * cc + t];
        }
        __builtin_amdgcn_sched_barrier(0);
        const int e_raw = p.ids[bj];
        bad_id = (unsigned)e_raw >= (unsigned)p.E;   // invalid routing: expert 0's rows are read, result NaN
        const int e = bad_id ? 0 : e_raw;
        u32x4 wg[U], wu[U];
        uint32_t sg[U], su[U];
        float live[U];
        const size_t row = (size_t)e * (size_t)p.I + (size_t)i0;
        const u32x4* gq = reinterpret_cast<const u32x4*>(p.wg_q + row * row_bytes);
        const u32x4* uq = reinterpret_cast<const u32x4*>(p.wu_q + row * row_bytes);
        const uint8_t* gs = p.wg_s + row * (size_t)(H / 32);
        const uint8_t* us = p.wu_s + row * (size_t)(H / 32);
#pragma unroll
        for (int m = 0; m < U; ++m) {
            const int c = base + lane + kWave * m;
            const int cc = c < nch ? c : nch - 1;
            wg[m] = __builtin_nontemporal_load(gq + cc);   // each row is read once: streaming
            wu[m] = __builtin_nontemporal_load(uq + cc);
            sg[m] = gs[FP4 ? cc : cc >> 1];
            su[m] = us[FP4 ? cc : cc >> 1];
            live[m] = c < nch ? 1.0f : 0.0f;
        }
#pragma unroll
        for (int m = 0; m < U; ++m) {
            const float pg = gu_chunk_dot<FP4, NX>(wg[m], xv[m]);
            const float pu = gu_chunk_dot<FP4, NX>(wu[m], xv[m]);
            g = __builtin_fmaf(pg, ue8m0_to_f32(sg[m]) * live[m], g);
            u = __builtin_fmaf(pu, ue8m0_to_f32(su[m]) * live[m], u);
        }
    }
    g_out = g;
    u_out = u;
    bad_out = bad_id;
}

}  // namespace moed
