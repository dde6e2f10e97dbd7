// Slot-group helpers of the down step (one wavefront per output out[b][h];
// warp-decode post, "How the two kernels work", third and fourth
// paragraphs), shared by the LDS-staged down kernel and the single-launch
// layer kernel. a[b] sits in LDS in the chunk-interleaved order the gate/up
// step writes (inter_index), in 16-byte units.
#pragma once

#include "launch.h"
#include "mx_device.h"

namespace moed {

constexpr int kCopyRegs = 4;                  // a[b] units per thread loaded ahead of the weights

// One slot group (JB routed slots x CPL chunks per lane) of the staged down
// kernel: issue its weight and scale loads ... Every load is unconditional
// from a clamped, in-bounds address (a lane past the end of the row re-reads
// the row's last chunk, an invalid expert id reads expert 0's row); lanes that
// must not contribute get the scale factor 0 (or NaN for an invalid id, which
// makes the token's output NaN). Without branches around the loads all of them
// issue back to back.
template <int CPL, int JB, bool NT>
__device__ __forceinline__ void down_group_load(const DownArgs& p, const int* ids, const float* wts, int j0,
                                                int o0, int h, bool active, int lane, int cpr,
                                                u32x4 (&wq)[JB][CPL], uint32_t (&ws)[JB][CPL], float (&wt)[JB],
                                                float (&mask)[JB][CPL])
{
    const int k = p.k;
    const int I = p.I;
    int eid[JB];
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
        const int jc = j0 + jj < k ? j0 + jj : k - 1;
        eid[jj] = ids[jc];
        wt[jj] = wts[jc];
    }
    const int hc = active ? h : 0;
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
        const bool live = active && (j0 + jj) < k;
        const bool ok = (unsigned)eid[jj] < (unsigned)p.E;
        const size_t row = (size_t)(ok ? eid[jj] : 0) * (size_t)p.H + (size_t)hc;
        const u32x4* wrow = reinterpret_cast<const u32x4*>(p.wd_q + row * (size_t)I);
        const uint8_t* srow = p.wd_s + row * (size_t)(I / 32);
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            const int o = o0 + lane + kWave * cc;
            const int oc = o < cpr ? o : cpr - 1;
            wq[jj][cc] = ld<NT>(wrow + oc);
            ws[jj][cc] = srow[oc >> 1];
            mask[jj][cc] = (live && o < cpr) ? (ok ? 1.0f : __builtin_nanf("")) : 0.0f;
        }
    }
}

// ... and fold it into the accumulator, reading a from LDS.
template <int CPL, int JB, bool A_BF16>
__device__ __forceinline__ float down_group_dot(const u32x4* a_lds, int k, int j0, int o0, int lane, int cpr,
                                                const u32x4 (&wq)[JB][CPL], const uint32_t (&ws)[JB][CPL],
                                                const float (&wt)[JB], const float (&mask)[JB][CPL], float acc)
{
    constexpr int NA = A_BF16 ? 2 : 4;
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
        const int j = j0 + jj < k ? j0 + jj : k - 1;
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            const int o = o0 + lane + kWave * cc;
            u32x4 av[NA];
            const int base = (j * NA) * cpr + (o < cpr ? o : cpr - 1);
#pragma unroll
            for (int t = 0; t < NA; ++t)
                av[t] = a_lds[base + t * cpr];
            float part = 0.0f;
            if constexpr (A_BF16) {
                part = dot4_bf16(wq[jj][cc].x, av[0].x, av[0].y, part);
                part = dot4_bf16(wq[jj][cc].y, av[0].z, av[0].w, part);
                part = dot4_bf16(wq[jj][cc].z, av[1].x, av[1].y, part);
                part = dot4_bf16(wq[jj][cc].w, av[1].z, av[1].w, part);
            } else {
                part = dot4_f32a(wq[jj][cc].x, __builtin_bit_cast(f32x4, av[0]), part);
                part = dot4_f32a(wq[jj][cc].y, __builtin_bit_cast(f32x4, av[1]), part);
                part = dot4_f32a(wq[jj][cc].z, __builtin_bit_cast(f32x4, av[2]), part);
                part = dot4_f32a(wq[jj][cc].w, __builtin_bit_cast(f32x4, av[3]), part);
            }
            // fold the routing weight into the one accumulator
            acc = __builtin_fmaf(wt[jj] * mask[jj][cc], part * ue8m0_to_f32(ws[jj][cc]), acc);
        }
    }
    return acc;
}

}  // namespace moed
