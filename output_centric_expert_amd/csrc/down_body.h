// Slot-group helpers of the down step (one wavefront per output out[b][h];
// warp-decode post, "How the two kernels work", third and fourth
// paragraphs), shared by the down kernels. a sits in the chunk-interleaved
// order the gate/up step writes (inter_index), in 16-byte units: piece t of
// the 16-value group g of row bj is unit (bj*NA + t)*(I/16) + g, NA = 4 for
// float32 a, 2 for bfloat16 a.
//
// A weight chunk is 16 bytes of a row: 16 MXFP8 codes (half an MX block, the
// 16-value group g = o) or 32 MXFP4 codes (one MX block, the groups 2o and
// 2o+1).
#pragma once

#include "launch.h"
#include "mx_device.h"

namespace moed {

constexpr int kCopyRegs = 4;                  // a[b] units per thread loaded ahead of the weights

// 16-byte pieces of a one weight chunk is dotted with.
template <bool FP4, bool A_BF16>
struct APieces {
    static constexpr int NA = A_BF16 ? 2 : 4;             // per 16-value group
    static constexpr int N = FP4 ? 2 * NA : NA;
};

// Unit index of piece q of weight chunk o of row bj (cpr16 = I/16). MXFP4:
// q = g*NA + t covers group 2o + g.
template <bool FP4, bool A_BF16>
__device__ __forceinline__ int a_unit(int bj, int o, int q, int cpr16)
{
    constexpr int NA = APieces<FP4, A_BF16>::NA;
    if constexpr (FP4)
        return (bj * NA + q % NA) * cpr16 + 2 * o + q / NA;
    else
        return (bj * NA + q) * cpr16 + o;
}

// Partial dot of one weight chunk (scale 1) with its pieces of a.
template <bool FP4, bool A_BF16>
__device__ __forceinline__ float chunk_dot(const u32x4& w, const u32x4 (&av)[APieces<FP4, A_BF16>::N])
{
    float part = 0.0f;
    if constexpr (FP4) {
        // dword d = codes 8d..8d+7 = values 8(d%2).. of group d/2
        if constexpr (A_BF16) {                 // piece t of a group = values 8t..8t+7: piece d
            part = dot8_fp4_bf16(w.x, av[0], part);
            part = dot8_fp4_bf16(w.y, av[1], part);
            part = dot8_fp4_bf16(w.z, av[2], part);
            part = dot8_fp4_bf16(w.w, av[3], part);
        } else {                                // piece t = values 4t..4t+3: pieces 2d, 2d+1
            part = dot8_fp4_f32a(w.x, __builtin_bit_cast(f32x4, av[0]), __builtin_bit_cast(f32x4, av[1]), part);
            part = dot8_fp4_f32a(w.y, __builtin_bit_cast(f32x4, av[2]), __builtin_bit_cast(f32x4, av[3]), part);
            part = dot8_fp4_f32a(w.z, __builtin_bit_cast(f32x4, av[4]), __builtin_bit_cast(f32x4, av[5]), part);
            part = dot8_fp4_f32a(w.w, __builtin_bit_cast(f32x4, av[6]), __builtin_bit_cast(f32x4, av[7]), part);
        }
    } else if constexpr (A_BF16) {
        part = dot4_bf16(w.x, av[0].x, av[0].y, part);
        part = dot4_bf16(w.y, av[0].z, av[0].w, part);
        part = dot4_bf16(w.z, av[1].x, av[1].y, part);
        part = dot4_bf16(w.w, av[1].z, av[1].w, part);
    } else {
        part = dot4_f32a(w.x, __builtin_bit_cast(f32x4, av[0]), part);
        part = dot4_f32a(w.y, __builtin_bit_cast(f32x4, av[1]), part);
        part = dot4_f32a(w.z, __builtin_bit_cast(f32x4, av[2]), part);
        part = dot4_f32a(w.w, __builtin_bit_cast(f32x4, av[3]), part);
    }
    return part;
}

// Lane groups: with G > 1 (rows of at most 64/G chunks) the wavefront is cut
// into G groups of LW = 64/G lanes; group g takes the slots j = j0 + g + G*jj
// and lane c of a group the chunks o = o0 + c + LW*cc. With G = 1 every lane
// takes every slot and the slot (expert id, routing weight) is uniform across
// the wavefront.
template <int G>
struct LaneGroups {
    static constexpr int LW = kWave / G;
    __device__ static int group(int lane) { return G == 1 ? 0 : lane / LW; }
    __device__ static int chunk(int lane) { return G == 1 ? lane : lane % LW; }
};

// One slot group (JB routed slots x CPL chunks per lane) of the staged down
// kernel: issue its weight and scale loads (cpr = weight chunks per row).
// Every load is unconditional from a clamped, in-bounds address (a lane past
// the end of the row re-reads the row's last chunk, an invalid expert id reads
// expert 0's row); lanes that must not contribute get the scale factor 0 (or
// NaN for an invalid id, which makes the token's output NaN). Without branches
// around the loads all of them issue back to back.
template <int CPL, int JB, bool NT, bool FP4, int G = 1>
__device__ __forceinline__ void down_group_load(const DownArgs& p, const int* ids, const float* wts, int j0,
                                                int o0, int h, bool active, int lane, int cpr,
                                                u32x4 (&wq)[JB][CPL], uint32_t (&ws)[JB][CPL], float (&wt)[JB],
                                                float (&mask)[JB][CPL])
{
    using LG = LaneGroups<G>;
    const int k = p.k;
    const int I = p.I;
    const size_t row_bytes = FP4 ? (size_t)(I / 2) : (size_t)I;
    const int js = j0 + LG::group(lane);
    const int lc = LG::chunk(lane);
    int eid[JB];
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
        const int j = js + G * jj;
        const int jc = j < k ? j : k - 1;
        eid[jj] = ids[jc];
        wt[jj] = wts[jc];
    }
    const int hc = active ? h : 0;
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
        const bool live = active && (js + G * jj) < k;
        const bool ok = (unsigned)eid[jj] < (unsigned)p.E;
        const size_t row = (size_t)(ok ? eid[jj] : 0) * (size_t)p.H + (size_t)hc;
        const u32x4* wrow = reinterpret_cast<const u32x4*>(p.wd_q + row * row_bytes);
        const uint8_t* srow = p.wd_s + row * (size_t)(I / 32);
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            const int o = o0 + lc + LG::LW * cc;
            const int oc = o < cpr ? o : cpr - 1;
            wq[jj][cc] = ld<NT>(wrow + oc);
            ws[jj][cc] = srow[FP4 ? oc : oc >> 1];
            mask[jj][cc] = (live && o < cpr) ? (ok ? 1.0f : __builtin_nanf("")) : 0.0f;
        }
    }
}

// ... and fold it into the accumulator, reading a[b] from LDS (row j of the
// staged copy is bj = j).
template <int CPL, int JB, bool A_BF16, bool FP4, int G = 1>
__device__ __forceinline__ float down_group_dot(const u32x4* a_lds, int k, int j0, int o0, int lane, int cpr,
                                                int cpr16, const u32x4 (&wq)[JB][CPL],
                                                const uint32_t (&ws)[JB][CPL], const float (&wt)[JB],
                                                const float (&mask)[JB][CPL], float acc)
{
    using LG = LaneGroups<G>;
    constexpr int NP = APieces<FP4, A_BF16>::N;
    const int js = j0 + LG::group(lane);
    const int lc = LG::chunk(lane);
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
        const int j = js + G * jj < k ? js + G * jj : k - 1;
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            const int o = o0 + lc + LG::LW * cc;
            const int oc = o < cpr ? o : cpr - 1;
            u32x4 av[NP];
#pragma unroll
            for (int q = 0; q < NP; ++q)
                av[q] = a_lds[a_unit<FP4, A_BF16>(j, oc, q, cpr16)];
            const float part = chunk_dot<FP4, A_BF16>(wq[jj][cc], av);
            // fold the routing weight into the one accumulator
            acc = __builtin_fmaf(wt[jj] * mask[jj][cc], part * ue8m0_to_f32(ws[jj][cc]), acc);
        }
    }
    return acc;
}

// The same for R rows h .. h+R-1 of the lane's slots (one chunk per lane and
// row, lane groups as above): each piece of a read from LDS serves all R rows,
// and per row the FMAs, their operands and their order are those of
// down_group_dot with CPL = 1, so every output is the same float.
template <int JB, bool FP4, int G, int R>
__device__ __forceinline__ void down_group_dot_multi(const u32x4* a_lds, int k, int lane, int cpr, int cpr16,
                                                     const u32x4 (&wq)[R][JB], const uint32_t (&ws)[R][JB],
                                                     const float (&wt)[JB], const float (&mask)[JB], float (&acc)[R])
{
    using LG = LaneGroups<G>;
    constexpr int NP = APieces<FP4, false>::N;
    const int js = LG::group(lane);
    const int lc = LG::chunk(lane);
    const int oc = lc < cpr ? lc : cpr - 1;
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
        const int j = js + G * jj < k ? js + G * jj : k - 1;
        u32x4 av[NP];
#pragma unroll
        for (int q = 0; q < NP; ++q)
            av[q] = a_lds[a_unit<FP4, false>(j, oc, q, cpr16)];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float part = chunk_dot<FP4, false>(wq[r][jj], av);
            acc[r] = __builtin_fmaf(wt[jj] * mask[jj], part * ue8m0_to_f32(ws[r][jj]), acc[r]);
        }
    }
}

// Variants for a wavefront that owns R consecutive outputs h0 .. h0+R-1 of one
// token (rows Wd[e][h0+r] of the same experts): each piece of a read from LDS
// serves all R rows. Per row the loads, the order of the FMAs and their
// operands are those of down_group_load / down_group_dot, so every output is
// the same float as with one row per wavefront.
template <int CPL, int JB, bool FP4, int R>
__device__ __forceinline__ void down_group_load_rows(const DownArgs& p, const int* ids, const float* wts, int j0,
                                                     int o0, int h0, int lane, int cpr,
                                                     u32x4 (&wq)[R][JB][CPL], uint32_t (&ws)[R][JB][CPL],
                                                     float (&wt)[JB], float (&mask)[R][JB][CPL])
{
    const int k = p.k;
    const int I = p.I;
    const size_t row_bytes = FP4 ? (size_t)(I / 2) : (size_t)I;
    int eid[JB];
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
        const int jc = j0 + jj < k ? j0 + jj : k - 1;
        eid[jj] = ids[jc];
        wt[jj] = wts[jc];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool row_live = h0 + r < p.H;
        const int hc = row_live ? h0 + r : 0;
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
            const bool live = row_live && (j0 + jj) < k;
            const bool ok = (unsigned)eid[jj] < (unsigned)p.E;
            const size_t row = (size_t)(ok ? eid[jj] : 0) * (size_t)p.H + (size_t)hc;
            const u32x4* wrow = reinterpret_cast<const u32x4*>(p.wd_q + row * row_bytes);
            const uint8_t* srow = p.wd_s + row * (size_t)(I / 32);
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                const int o = o0 + lane + kWave * cc;
                const int oc = o < cpr ? o : cpr - 1;
                wq[r][jj][cc] = *(wrow + oc);
                ws[r][jj][cc] = srow[FP4 ? oc : oc >> 1];
                mask[r][jj][cc] = (live && o < cpr) ? (ok ? 1.0f : __builtin_nanf("")) : 0.0f;
            }
        }
    }
}

template <int CPL, int JB, bool A_BF16, bool FP4, int R>
__device__ __forceinline__ void down_group_dot_rows(const u32x4* a_lds, int k, int j0, int o0, int lane, int cpr,
                                                    int cpr16, const u32x4 (&wq)[R][JB][CPL],
                                                    const uint32_t (&ws)[R][JB][CPL], const float (&wt)[JB],
                                                    const float (&mask)[R][JB][CPL], float (&acc)[R])
{
    constexpr int NP = APieces<FP4, A_BF16>::N;
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
        const int j = j0 + jj < k ? j0 + jj : k - 1;
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            const int o = o0 + lane + kWave * cc;
            const int oc = o < cpr ? o : cpr - 1;
            u32x4 av[NP];
#pragma unroll
            for (int q = 0; q < NP; ++q)
                av[q] = a_lds[a_unit<FP4, A_BF16>(j, oc, q, cpr16)];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float part = chunk_dot<FP4, A_BF16>(wq[r][jj][cc], av);
                acc[r] = __builtin_fmaf(wt[jj] * mask[r][jj][cc], part * ue8m0_to_f32(ws[r][jj][cc]), acc[r]);
            }
        }
    }
}

}  // namespace moed
