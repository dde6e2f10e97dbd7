// Down kernel: one wavefront per output out[b][h] -- the second warp-decode
// kernel (warp-decode post, "How the two kernels work", third and fourth
// paragraphs), laid out for 64-lane CDNA4 wavefronts.
//
// Wave w owns (b, h) with w = b*H + h. It loops over the k routed slots of
// token b; the slot, its expert id e_j and routing weight w[b][j] are uniform
// across the wavefront (scalar loads into SGPRs), so each row's address is a
// scalar base plus a per-lane offset and no load waits on another load.
// The intermediate a is read in the chunk-interleaved order the gate/up
// kernel writes (inter_index), so each 16-byte load is contiguous across
// the wavefront.
// Row Wd[e_j][h][:] (I codes) is split into 16-code chunks, chunk o going to
// lane o % 64; JB slots x CPL chunks per lane are loaded (weights, the block
// scale byte and the 16 matching values of a[b][j][:]) before the first
// arithmetic. Each lane multiplies its chunk's partial dot by the block scale
// and the routing weight and adds it into a single FP32 accumulator; after
// all experts one DPP/ds_swizzle reduction and one scalar store (bf16
// round-to-nearest-even, or f32) finish the output.
#include "down_body.h"

namespace moed {

template <int CPL, int JB, bool A_BF16, bool OUT_BF16, bool NT, bool FP4>
__global__ void __launch_bounds__(256)
moe_down_kernel(DownArgs p)
{
    constexpr int NP = APieces<FP4, A_BF16>::N;   // 16-byte pieces of a per weight chunk
    const int lane = threadIdx.x & (kWave - 1);
    const int wpb = blockDim.x / kWave;
    const int blk = xcd_contiguous((int)blockIdx.x, (int)gridDim.x);
    const int wave = __builtin_amdgcn_readfirstlane(blk * wpb + (int)(threadIdx.x / kWave));
    const int n_out = p.B * p.H;
    if (wave >= n_out)
        return;
    // hidden-major (w = h*B + b): the tokens of one output h are neighbours
    const int b = wave % p.B;
    const int h = wave / p.B;
    const int k = p.k;
    const int I = p.I;
    const int cpr16 = I / 16;                     // 16-value groups per row of a
    const int cpr = FP4 ? I / 32 : cpr16;         // weight chunks per routed row
    const size_t row_bytes = FP4 ? (size_t)(I / 2) : (size_t)I;
    const int* ids = p.ids + (size_t)b * k;
    const float* wts = p.w + (size_t)b * k;
    const u32x4* a16 = static_cast<const u32x4*>(p.a);

    float acc = 0.0f;
    for (int j0 = 0; j0 < k; j0 += JB) {
        int e[JB];
        float wt[JB];
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
            const int j = j0 + jj;
            const int jc = j < k ? j : k - 1;     // in-bounds even if the load is speculated
            e[jj] = j < k ? ids[jc] : -1;
            wt[jj] = j < k ? wts[jc] : 0.0f;
        }
        for (int o0 = 0; o0 < cpr; o0 += kWave * CPL) {
            u32x4 wq[JB][CPL];
            uint32_t ws[JB][CPL];
            u32x4 av[JB][CPL][NP];
#pragma unroll
            for (int jj = 0; jj < JB; ++jj) {
                const int j = j0 + jj;
                const bool live = j < k;
                const bool ok = (unsigned)e[jj] < (unsigned)p.E;
                const size_t row = (size_t)(ok ? e[jj] : 0) * (size_t)p.H + (size_t)h;
                const uint8_t* wrow = p.wd_q + row * row_bytes;
                const uint8_t* srow = p.wd_s + row * (size_t)(I / 32);
                const int bj = b * k + (live ? j : 0);
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) {
                    const int o = o0 + lane + kWave * cc;
                    if (live && o < cpr) {
                        if (ok) {
                            wq[jj][cc] = ld<NT>(reinterpret_cast<const u32x4*>(wrow) + o);
                            ws[jj][cc] = srow[FP4 ? o : o >> 1];
                        } else {                  // invalid routing: NaN scale, no weight read
                            wq[jj][cc] = u32x4{0, 0, 0, 0};
                            ws[jj][cc] = 255u;
                        }
#pragma unroll
                        for (int q = 0; q < NP; ++q)
                            av[jj][cc][q] = a16[a_unit<FP4, A_BF16>(bj, o, q, cpr16)];
                    } else {
                        wq[jj][cc] = u32x4{0, 0, 0, 0};
                        ws[jj][cc] = 127u;
#pragma unroll
                        for (int q = 0; q < NP; ++q)
                            av[jj][cc][q] = u32x4{0, 0, 0, 0};
                    }
                }
            }
#pragma unroll
            for (int jj = 0; jj < JB; ++jj) {
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) {
                    const float part = chunk_dot<FP4, A_BF16>(wq[jj][cc], av[jj][cc]);
                    // fold the routing weight into the one accumulator
                    acc = __builtin_fmaf(wt[jj], part * ue8m0_to_f32(ws[jj][cc]), acc);
                }
            }
        }
    }
    acc = wave_sum(acc);
    if (lane == 0) {
        if constexpr (OUT_BF16)
            static_cast<uint16_t*>(p.out)[(size_t)b * p.H + h] = f32_to_bf16_rne(acc);
        else
            static_cast<float*>(p.out)[(size_t)b * p.H + h] = acc;
    }
}

// LDS-staged variant (used when a[b] fits in LDS): the waves of a workgroup
// all serve the same token b, so a[b][:][:] is copied once per workgroup
// into LDS and every wave reads its chunks from there instead of from L2.
// Still one wavefront per output. The first kCopyRegs units per thread of the
// copy are loaded, then the first slot group's weights; since loads retire in
// issue order, the LDS writes wait only for the copy, and each slot's FMAs
// start as soon as that slot's weights have arrived. The copy keeps the
// chunk-interleaved order, so the per-chunk LDS reads are contiguous across
// lanes (no bank conflicts).
template <int CPL, int JB, bool A_BF16, bool OUT_BF16, bool NT, bool FP4, int G>
__global__ void __launch_bounds__(512)
moe_down_staged_kernel(DownArgs p)
{
    extern __shared__ u32x4 a_lds[];
    constexpr int NA = A_BF16 ? 2 : 4;
    const int lane = threadIdx.x & (kWave - 1);
    const int wpb = blockDim.x / kWave;
    // workgroup hb*B + b (hidden-major, each XCD a contiguous range): the
    // workgroups of one hidden block -- the same weight rows -- are neighbours
    const int blk = xcd_contiguous((int)blockIdx.x, (int)gridDim.x);
    const int b = blk % p.B;
    const int h = (blk / p.B) * wpb + (int)(threadIdx.x / kWave);
    const bool active = h < p.H;                  // idle waves still help copy a[b]
    const int k = p.k;
    const int cpr16 = p.I / 16;                   // 16-value groups per row of a
    const int cpr = FP4 ? p.I / 32 : cpr16;       // weight chunks per routed row
    const int nunits = k * NA * cpr16;            // 16-byte units of a[b]
    const int* ids = p.ids + (size_t)b * k;
    const float* wts = p.w + (size_t)b * k;
    const u32x4* asrc = static_cast<const u32x4*>(p.a) + (size_t)b * (size_t)nunits;

    // 1) the first kCopyRegs units per thread of a[b], 2) the first group's
    // weights, 3) the LDS writes (which wait only for the copy), one barrier
    u32x4 cp[kCopyRegs];
#pragma unroll
    for (int q = 0; q < kCopyRegs; ++q) {
        const int u = (int)threadIdx.x + q * (int)blockDim.x;
        cp[q] = u < nunits ? asrc[u] : u32x4{0, 0, 0, 0};
    }
    __builtin_amdgcn_sched_barrier(0);
    u32x4 wq[JB][CPL];
    uint32_t ws[JB][CPL];
    float wt[JB];
    float mask[JB][CPL];
    down_group_load<CPL, JB, NT, FP4, G>(p, ids, wts, 0, 0, h, active, lane, cpr, wq, ws, wt, mask);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < kCopyRegs; ++q) {
        const int u = (int)threadIdx.x + q * (int)blockDim.x;
        if (u < nunits)
            a_lds[u] = cp[q];
    }
    for (int u = (int)threadIdx.x + kCopyRegs * (int)blockDim.x; u < nunits; u += blockDim.x)
        a_lds[u] = asrc[u];
    __syncthreads();
    if (!active)
        return;                                   // after the only barrier

    float acc = down_group_dot<CPL, JB, A_BF16, FP4, G>(a_lds, k, 0, 0, lane, cpr, cpr16, wq, ws, wt, mask, 0.0f);
    // remaining row passes and slot groups (none when one group covers the layer)
    constexpr int LW = LaneGroups<G>::LW;
    for (int j0 = 0; j0 < k; j0 += G * JB) {
        for (int o0 = (j0 == 0 ? LW * CPL : 0); o0 < cpr; o0 += LW * CPL) {
            down_group_load<CPL, JB, NT, FP4, G>(p, ids, wts, j0, o0, h, true, lane, cpr, wq, ws, wt, mask);
            acc = down_group_dot<CPL, JB, A_BF16, FP4, G>(a_lds, k, j0, o0, lane, cpr, cpr16, wq, ws, wt, mask,
                                                          acc);
        }
    }
    acc = wave_sum(acc);
    if (lane == 0) {
        if constexpr (OUT_BF16)
            static_cast<uint16_t*>(p.out)[(size_t)b * p.H + h] = f32_to_bf16_rne(acc);
        else
            static_cast<float*>(p.out)[(size_t)b * p.H + h] = acc;
    }
}

// LDS-staged variant with R consecutive outputs per wavefront (used once
// tokens share experts, B*k >= E, where the copy of a[b] and the LDS reads of
// it, not the weight stream, bound the kernel): each piece of a read from LDS
// serves R rows, and a workgroup of 8 wavefronts covers 8R outputs per copy of
// a[b]. The per-output arithmetic is that of the one-row kernel, bit for bit.
// Weights are loaded through the caches (rows are shared between tokens).
template <int CPL, int JB, bool A_BF16, bool OUT_BF16, bool FP4, int R>
__global__ void __launch_bounds__(512)
moe_down_rows_kernel(DownArgs p)
{
    extern __shared__ u32x4 a_lds[];
    constexpr int NA = A_BF16 ? 2 : 4;
    const int lane = threadIdx.x & (kWave - 1);
    const int wpb = blockDim.x / kWave;
    const int blk = xcd_contiguous((int)blockIdx.x, (int)gridDim.x);
    const int b = blk % p.B;
    const int h0 = ((blk / p.B) * wpb + (int)(threadIdx.x / kWave)) * R;
    const bool active = h0 < p.H;
    const int k = p.k;
    const int cpr16 = p.I / 16;
    const int cpr = FP4 ? p.I / 32 : cpr16;
    const int nunits = k * NA * cpr16;
    const int* ids = p.ids + (size_t)b * k;
    const float* wts = p.w + (size_t)b * k;
    const u32x4* asrc = static_cast<const u32x4*>(p.a) + (size_t)b * (size_t)nunits;

    u32x4 cp[kCopyRegs];
#pragma unroll
    for (int q = 0; q < kCopyRegs; ++q) {
        const int u = (int)threadIdx.x + q * (int)blockDim.x;
        cp[q] = u < nunits ? asrc[u] : u32x4{0, 0, 0, 0};
    }
    __builtin_amdgcn_sched_barrier(0);
    u32x4 wq[R][JB][CPL];
    uint32_t ws[R][JB][CPL];
    float wt[JB];
    float mask[R][JB][CPL];
    down_group_load_rows<CPL, JB, FP4, R>(p, ids, wts, 0, 0, active ? h0 : 0, lane, cpr, wq, ws, wt, mask);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < kCopyRegs; ++q) {
        const int u = (int)threadIdx.x + q * (int)blockDim.x;
        if (u < nunits)
            a_lds[u] = cp[q];
    }
    for (int u = (int)threadIdx.x + kCopyRegs * (int)blockDim.x; u < nunits; u += blockDim.x)
        a_lds[u] = asrc[u];
    __syncthreads();
    if (!active)
        return;                                   // after the only barrier

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        acc[r] = 0.0f;
    down_group_dot_rows<CPL, JB, A_BF16, FP4, R>(a_lds, k, 0, 0, lane, cpr, cpr16, wq, ws, wt, mask, acc);
    for (int j0 = 0; j0 < k; j0 += JB) {
        for (int o0 = (j0 == 0 ? kWave * CPL : 0); o0 < cpr; o0 += kWave * CPL) {
            down_group_load_rows<CPL, JB, FP4, R>(p, ids, wts, j0, o0, h0, lane, cpr, wq, ws, wt, mask);
            down_group_dot_rows<CPL, JB, A_BF16, FP4, R>(a_lds, k, j0, o0, lane, cpr, cpr16, wq, ws, wt, mask, acc);
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
        acc[r] = wave_sum(acc[r]);
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (h0 + r < p.H) {
                if constexpr (OUT_BF16)
                    static_cast<uint16_t*>(p.out)[(size_t)b * p.H + h0 + r] = f32_to_bf16_rne(acc[r]);
                else
                    static_cast<float*>(p.out)[(size_t)b * p.H + h0 + r] = acc[r];
            }
        }
    }
}

template <int CPL, int JB, int R>
static hipError_t dispatch_rows(bool fp4, bool a_bf16, bool out_bf16, const DownArgs& p, dim3 grid, dim3 block,
                                size_t lds, hipStream_t s)
{
#define MOED_DR(F, A, O) \
    if (fp4 == F && a_bf16 == A && out_bf16 == O) \
        hipLaunchKernelGGL((moe_down_rows_kernel<CPL, JB, A, O, F, R>), grid, block, lds, s, p);
    MOED_DR(false, false, false) MOED_DR(false, false, true) MOED_DR(false, true, false) MOED_DR(false, true, true)
    MOED_DR(true, false, false) MOED_DR(true, false, true) MOED_DR(true, true, false) MOED_DR(true, true, true)
#undef MOED_DR
    return hipGetLastError();
}

// R outputs per wavefront, rows covered in one pass (CPL * 64 >= chunks per
// row): CPL as for one row, JB cut so that R * CPL * JB <= 4 where it can be
// (in one pass the FMA order per lane does not depend on JB).
template <int R>
static hipError_t launch_rows(int cpl, bool fp4, bool a_bf16, bool out_bf16, const DownArgs& p, int wpb,
                              size_t lds, hipStream_t s)
{
    const dim3 grid((unsigned)((long)p.B * ((p.H + R * wpb - 1) / (R * wpb)))), block(wpb * kWave);
    int jb = 8 / cpl;
    while (jb > 1 && (R * cpl * jb > 4 || jb / 2 >= p.k))
        jb /= 2;
    switch (cpl * 16 + jb) {
    case 1 * 16 + 2: return dispatch_rows<1, 2, R>(fp4, a_bf16, out_bf16, p, grid, block, lds, s);
    case 1 * 16 + 1: return dispatch_rows<1, 1, R>(fp4, a_bf16, out_bf16, p, grid, block, lds, s);
    case 2 * 16 + 1: return dispatch_rows<2, 1, R>(fp4, a_bf16, out_bf16, p, grid, block, lds, s);
    case 4 * 16 + 1: return dispatch_rows<4, 1, R>(fp4, a_bf16, out_bf16, p, grid, block, lds, s);
    case 8 * 16 + 1: return dispatch_rows<8, 1, R>(fp4, a_bf16, out_bf16, p, grid, block, lds, s);
    default: return hipErrorInvalidValue;
    }
}

template <int CPL, int JB, bool FP4, int G = 1>
static hipError_t dispatch_v(bool staged, bool a_bf16, bool out_bf16, bool nt, const DownArgs& p, dim3 grid,
                             dim3 block, size_t lds, hipStream_t s)
{
#define MOED_DN(A, O, N) \
    if (a_bf16 == A && out_bf16 == O && nt == N) { \
        if (staged) \
            hipLaunchKernelGGL((moe_down_staged_kernel<CPL, JB, A, O, N, FP4, G>), grid, block, lds, s, p); \
        else if constexpr (G == 1) \
            hipLaunchKernelGGL((moe_down_kernel<CPL, JB, A, O, N, FP4>), grid, block, 0, s, p); \
    }
    MOED_DN(false, false, false) MOED_DN(false, false, true) MOED_DN(false, true, false) MOED_DN(false, true, true)
    MOED_DN(true, false, false) MOED_DN(true, false, true) MOED_DN(true, true, false) MOED_DN(true, true, true)
#undef MOED_DN
    return hipGetLastError();
}

template <int CPL, int JB>
static hipError_t dispatch_f(bool fp4, bool staged, bool a_bf16, bool out_bf16, bool nt, const DownArgs& p,
                             dim3 grid, dim3 block, size_t lds, hipStream_t s)
{
    return fp4 ? dispatch_v<CPL, JB, true>(staged, a_bf16, out_bf16, nt, p, grid, block, lds, s)
               : dispatch_v<CPL, JB, false>(staged, a_bf16, out_bf16, nt, p, grid, block, lds, s);
}

// staged kernel with G lane groups (one chunk per lane, JB slots per group)
template <int G>
static hipError_t dispatch_g(int jb, bool fp4, bool a_bf16, bool out_bf16, bool nt, const DownArgs& p, dim3 grid,
                             dim3 block, size_t lds, hipStream_t s)
{
    switch (jb * 2 + (fp4 ? 1 : 0)) {
    case 8 * 2 + 0: return dispatch_v<1, 8, false, G>(true, a_bf16, out_bf16, nt, p, grid, block, lds, s);
    case 8 * 2 + 1: return dispatch_v<1, 8, true, G>(true, a_bf16, out_bf16, nt, p, grid, block, lds, s);
    case 4 * 2 + 0: return dispatch_v<1, 4, false, G>(true, a_bf16, out_bf16, nt, p, grid, block, lds, s);
    case 4 * 2 + 1: return dispatch_v<1, 4, true, G>(true, a_bf16, out_bf16, nt, p, grid, block, lds, s);
    case 2 * 2 + 0: return dispatch_v<1, 2, false, G>(true, a_bf16, out_bf16, nt, p, grid, block, lds, s);
    case 2 * 2 + 1: return dispatch_v<1, 2, true, G>(true, a_bf16, out_bf16, nt, p, grid, block, lds, s);
    case 1 * 2 + 0: return dispatch_v<1, 1, false, G>(true, a_bf16, out_bf16, nt, p, grid, block, lds, s);
    case 1 * 2 + 1: return dispatch_v<1, 1, true, G>(true, a_bf16, out_bf16, nt, p, grid, block, lds, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_down(const DownArgs& p, bool a_bf16, bool out_bf16, const Tuning& t, hipStream_t s)
{
    const long n_out = (long)p.B * p.H;
    if (n_out == 0)
        return hipSuccess;
    // chunks per lane per row: the smallest of 1, 2, 4, 8 covering the row
    // (longer rows take several passes); slots per group so that CPL * JB <= 8
    const bool fp4 = p.wfmt == kMXFP4;
    const int cpr = fp4 ? p.I / 32 : p.I / 16;
    // a[b] staged in LDS when it fits in 64 KiB
    const size_t lds = (size_t)p.k * (size_t)p.I * (a_bf16 ? 2u : 4u);
    const bool staged = t.dn_stage != 0 && lds <= 65536;
    int cap = t.dn_umax < 1 ? 1 : t.dn_umax;
    // the unstaged kernel holds every piece of a for its chunks in registers:
    // 8 pieces per MXFP4 chunk (float32 a), so at most 2 chunks in flight
    if (fp4 && !staged && cap > 2)
        cap = 2;
    int cpl = 1;
    while (cpl < 8 && cpl * kWave < cpr)
        cpl *= 2;
    while (cpl > 1 && cpl > cap)
        cpl /= 2;
    const int wpb = t.dn_wpb > (staged ? 8 : 4) ? (staged ? 8 : 4) : t.dn_wpb;
    const dim3 block(wpb * kWave);
    const dim3 grid(staged ? (unsigned)((long)p.B * ((p.H + wpb - 1) / wpb)) : (unsigned)((n_out + wpb - 1) / wpb));
    // streaming weight loads unless tokens share rows (B*k >= E)
    const bool nt = (long)p.B * p.k < (long)p.E;
    const DownArgs& q = p;
    // lane groups (staged kernel): rows of at most 16 or 32 chunks share the
    // wavefront among 4 or 2 slots at a time (at most k groups)
    int groups = 1;
    if (staged && t.dn_lanegroups != 0) {
        while (groups < 4 && cpr <= kWave / (2 * groups) && 2 * groups <= p.k)
            groups *= 2;
    }
    // one-pass form: k is one slot group (G*JB with JB a power of two up to 8),
    // a row is one chunk per lane, float32 a, streaming loads, one output per
    // wavefront, 8 wavefronts per workgroup
    // (several outputs per wavefront once tokens share experts, with the same
    // arithmetic per output as one output per wavefront: 4 once B*k >= E, 2 for
    // smaller batches, 1 for a single token, where halving the workgroup count
    // would leave CUs idle -- measured; lane groups keep one output per
    // wavefront, and so does the one-pass kernel, which also replaces the
    // two-row default where it applies: B=4 down 12.7 -> 10.7 us, B=8 18.6 ->
    // 17.7 us at k=8, I=768; at B*k >= E four rows stay faster)
    const int rows = (long)p.B * p.k >= (long)p.E ? 4 : (p.B >= 2 ? 2 : 1);
    const int per_group = p.k / groups;
    // blocks form of the one-pass kernel where tokens share experts, below the
    // expert-major switch of moe_decode (E <= B*k < 2E; measured there), for the
    // one-pass shapes with H a multiple of 64; it replaces the four-row and
    // lane-group kernels with the same floats per output. Not for MXFP4 rows
    // of more than 32 chunks (eight slots per lane group: 210 registers, two
    // wavefronts per SIMD), where it measured slower (B = 16, H = 4096,
    // I = 1536: down 86.5 vs 81.9 us)
    const bool one_pass_shape = staged && t.dn_onepass != 0 && !a_bf16 && wpb == 8 && p.k == groups * per_group &&
                                (per_group & (per_group - 1)) == 0 && per_group <= 8 && cpr <= kWave / groups;
    if (one_pass_shape && !nt && (long)p.B * p.k < 2L * (long)p.E && p.H % (8 * kDownBlocks) == 0 &&
        !(fp4 && per_group == 8))
        return launch_down_blocks(q, per_group, groups, out_bf16, lds, s);
    if (staged && t.dn_onepass != 0 && !a_bf16 && nt && wpb == 8 && p.k == groups * per_group &&
        (per_group & (per_group - 1)) == 0 && per_group <= 8 && cpr <= kWave / groups &&
        (groups > 1 || rows <= 2)) {
        // MXFP4 at B > 1: two outputs per wavefront (an MXFP4 chunk is dotted with
        // 128 bytes of a from LDS, an MXFP8 one with 64: sharing each read between
        // two rows pays for MXFP4 only -- measured), with 4 wavefronts per
        // workgroup unless that leaves at least 2048 workgroups of 8
        int pair_wpb = 0;
        if (fp4 && t.dn_pair != 0 && p.B > 1 && p.H % 2 == 0)
            pair_wpb = (long)p.B * (p.H / 16) >= 2048 ? 8 : 4;
        return launch_down_onepass(q, per_group, groups, out_bf16, pair_wpb, grid, block, lds, s);
    }
    if (groups > 1) {
        const int per = (p.k + groups - 1) / groups;   // slots per group
        int jbg = 8;
        while (jbg > 1 && (jbg > cap || jbg / 2 >= per))
            jbg /= 2;
        if (groups == 2)
            return dispatch_g<2>(jbg, fp4, a_bf16, out_bf16, nt, q, grid, block, lds, s);
        return dispatch_g<4>(jbg, fp4, a_bf16, out_bf16, nt, q, grid, block, lds, s);
    }
    int jb = 8 / cpl;
    while (jb > 1 && (cpl * jb > cap || jb / 2 >= p.k))
        jb /= 2;
    if (staged && rows > 1 && cpl * kWave >= cpr) {
        if (rows == 4)
            return launch_rows<4>(cpl, fp4, a_bf16, out_bf16, q, wpb, lds, s);
        return launch_rows<2>(cpl, fp4, a_bf16, out_bf16, q, wpb, lds, s);
    }
    switch (cpl * 16 + jb) {
    case 1 * 16 + 8: return dispatch_f<1, 8>(fp4, staged, a_bf16, out_bf16, nt, q, grid, block, lds, s);
    case 1 * 16 + 4: return dispatch_f<1, 4>(fp4, staged, a_bf16, out_bf16, nt, q, grid, block, lds, s);
    case 1 * 16 + 2: return dispatch_f<1, 2>(fp4, staged, a_bf16, out_bf16, nt, q, grid, block, lds, s);
    case 1 * 16 + 1: return dispatch_f<1, 1>(fp4, staged, a_bf16, out_bf16, nt, q, grid, block, lds, s);
    case 2 * 16 + 4: return dispatch_f<2, 4>(fp4, staged, a_bf16, out_bf16, nt, q, grid, block, lds, s);
    case 2 * 16 + 2: return dispatch_f<2, 2>(fp4, staged, a_bf16, out_bf16, nt, q, grid, block, lds, s);
    case 2 * 16 + 1: return dispatch_f<2, 1>(fp4, staged, a_bf16, out_bf16, nt, q, grid, block, lds, s);
    case 4 * 16 + 2: return dispatch_f<4, 2>(fp4, staged, a_bf16, out_bf16, nt, q, grid, block, lds, s);
    case 4 * 16 + 1: return dispatch_f<4, 1>(fp4, staged, a_bf16, out_bf16, nt, q, grid, block, lds, s);
    case 8 * 16 + 1: return dispatch_f<8, 1>(fp4, staged, a_bf16, out_bf16, nt, q, grid, block, lds, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace moed
