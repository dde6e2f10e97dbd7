// One-pass down kernel for single-token and small-batch decode (one wavefront
// per output out[b][h]; warp-decode post, "How the two kernels work", third
// and fourth paragraphs): the staged kernel's arithmetic in straight-line code
// for the case where a token's k slots form one slot group and a routed row is
// at most one 16-byte chunk per lane.
#include "down_body.h"

namespace moed {

// One-pass form of the staged kernel for the usual decode shape: the token's
// k slots are exactly one group (k = G*JB: JB slots for each of G lane
// groups) and a row is at most one chunk per lane (cpr <= 64/G); float32 a,
// streaming weight loads, 8 wavefronts per workgroup. Everything a wave needs
// is requested in straight-line code before its first wait: the copy of a[b]
// (at most NCP units per thread), the k routed ids and weights (compile-time
// offsets, so one wide scalar load each when G = 1), then every weight chunk
// and scale byte. No loop, no branch and no wait sits among these loads, so
// the weights of all k experts are in flight together from the kernel's
// first memory round trip on. Per output the FMAs, their operands and their
// order are those of moe_down_staged_kernel with the same lane groups, so the
// results are the same floats. The workgroup order is always hidden-major and
// XCD-contiguous (the default order of the other kernels). ONE_TOKEN: B = 1,
// so the token index needs no division. R = 2: the wavefront owns the two
// neighbouring outputs h, h+1 (H even): each lane loads its chunk of both
// rows of every slot (the rows of one expert are contiguous) and each piece
// of a read from LDS serves both, which halves the LDS reads and the copies
// of a[b] per output; per output the arithmetic is unchanged. WPB: 8 or 4
// wavefronts per workgroup (NCP then covers a[b] with WPB*64 threads).
template <int JB, int G, bool OUT_BF16, bool FP4, int NCP, bool ONE_TOKEN, int R = 1, int WPB = 8>
__global__ void __launch_bounds__(WPB * kWave)
moe_down_onepass_kernel(DownArgs p)
{
    extern __shared__ u32x4 a_lds[];
    constexpr int NTH = WPB * kWave;
    constexpr int KS = G * JB;                    // slots per token (= p.k)
    using LG = LaneGroups<G>;
    const int lane = threadIdx.x & (kWave - 1);
    // always the hidden-major, XCD-contiguous workgroup order (no branch on
    // the order argument ahead of the loads)
    const int blk = xcd_contiguous((int)blockIdx.x, (int)gridDim.x);
    const int b = ONE_TOKEN ? 0 : blk % p.B;
    const int h = ((ONE_TOKEN ? blk : blk / p.B) * WPB + (int)(threadIdx.x / kWave)) * R;
    const bool active = h < p.H;                  // idle waves still help copy a[b]
    const int cpr16 = p.I / 16;
    const int cpr = FP4 ? p.I / 32 : cpr16;
    const int nunits = KS * 4 * cpr16;
    const int* ids = p.ids + (size_t)b * KS;
    const float* wts = p.w + (size_t)b * KS;
    const u32x4* asrc = static_cast<const u32x4*>(p.a) + (size_t)b * (size_t)nunits;

    // 1) the copy of a[b]: NCP unconditional loads per thread from clamped
    // addresses (surplus ones re-read the last unit; a guard here would make
    // the compiler wait for each copy before issuing the next). NCP is the
    // exact count ceil(units / 512) for single-token calls with k = 8, else the
    // largest count the shape limits allow.
    u32x4 cp[NCP];
#pragma unroll
    for (int q = 0; q < NCP; ++q) {
        const int u = (int)threadIdx.x + q * NTH;
        cp[q] = asrc[u < nunits ? u : nunits - 1];
    }
    __builtin_amdgcn_sched_barrier(0);
    // 2) ids and routing weights of the lane's slots j = g + G*jj: all k of
    // them by scalar loads at compile-time offsets, then picked per lane group
    // (a per-lane load here would be counted with the copy loads, so the
    // weight loads would wait for the copy as well)
    const int g = LG::group(lane);
    const int lc = LG::chunk(lane);
    int id_all[KS];
    float w_all[KS];
#pragma unroll
    for (int t = 0; t < KS; ++t) {
        id_all[t] = ids[t];
        w_all[t] = wts[t];
    }
    // both arrive in one wait, before the weight loads (left alone, the
    // compiler sinks the weights' scalar load towards its use, where it costs
    // a memory round trip of its own)
#pragma unroll
    for (int t = 0; t < KS; ++t)
        asm volatile("" ::"s"(id_all[t]), "s"(w_all[t]));
    int eid[JB];
    float wt[JB];
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
        eid[jj] = id_all[G * jj];
        wt[jj] = w_all[G * jj];
#pragma unroll
        for (int gg = 1; gg < G; ++gg) {
            eid[jj] = g == gg ? id_all[gg + G * jj] : eid[jj];
            wt[jj] = g == gg ? w_all[gg + G * jj] : wt[jj];
        }
    }
    // 3) every weight chunk and scale byte (an invalid id reads expert 0's row
    // and makes the output NaN; lanes past the row end re-read its last chunk
    // with factor 0)
    const size_t row_bytes = FP4 ? (size_t)(p.I / 2) : (size_t)p.I;
    const int hc = active ? h : 0;
    const int oc = lc < cpr ? lc : cpr - 1;
    const bool lane_live = active && lc < cpr;
    u32x4 wq[R][JB];
    uint32_t ws[R][JB];
    float mask[JB];
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
        const bool ok = (unsigned)eid[jj] < (unsigned)p.E;
        mask[jj] = lane_live ? (ok ? 1.0f : __builtin_nanf("")) : 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const size_t row = (size_t)(ok ? eid[jj] : 0) * (size_t)p.H + (size_t)(hc + r);
            wq[r][jj] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.wd_q + row * row_bytes) + oc);
            ws[r][jj] = p.wd_s[row * (size_t)(p.I / 32) + (FP4 ? oc : oc >> 1)];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < NCP; ++q) {
        const int u = (int)threadIdx.x + q * NTH;
        if (u < nunits)
            a_lds[u] = cp[q];
    }
    __syncthreads();
    if (!active)
        return;                                   // after the only barrier
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        acc[r] = 0.0f;
    down_group_dot_multi<JB, FP4, G, R>(a_lds, KS, lane, cpr, cpr16, wq, ws, wt, mask, acc);
#pragma unroll
    for (int r = 0; r < R; ++r)
        acc[r] = wave_sum(acc[r]);
    if (lane == 0) {
        const size_t o = (size_t)b * p.H + h;
#pragma unroll
        for (int r = 0; r < R; ++r) {             // element stores: out needs no alignment beyond its type
            if constexpr (OUT_BF16)
                static_cast<uint16_t*>(p.out)[o + r] = f32_to_bf16_rne(acc[r]);
            else
                static_cast<float*>(p.out)[o + r] = acc[r];
        }
    }
}

// Copy loads per thread that cover a[b] (KS*4*(I/16) units) for any shape the
// kernel takes: I/16 <= 64/G for MXFP8 and <= 128/G for MXFP4.
constexpr int onepass_max_ncp(int jb, bool fp4) { return fp4 ? jb : (jb >= 2 ? jb / 2 : 1); }

// Blocks form of the one-pass kernel, for batches whose tokens share experts
// (B*k >= E): a workgroup of 8 wavefronts copies a[b] into LDS once and then
// takes RS blocks of 8 neighbouring outputs of its token in turn, one output
// per wavefront per block. The next block's rows are requested before the
// current block's dots, and the loads are cached: the other tokens routed to
// an expert read the same rows, and the workgroup order (token fastest, then
// the output blocks, each XCD a contiguous range) has them read those rows on
// one XCD at about the same time. Per output the loads, the FMAs, their
// operands and order, and the reduction are those of the one-pass kernel, so
// every output is the same float. Measured against the four-outputs-per-
// wavefront and lane-group kernels it replaces (E = 128, H = 2048, I = 768,
// down step alone): B = 16 34.5 -> 30.9 us (MXFP8), 30.6 -> 22.4 us (MXFP4);
// B = 24 46.7 -> 42.3 us, 43.1 -> 30.2 us.
template <int JB, int G, bool OUT_BF16, bool FP4, int NCP, int RS>
__global__ void __launch_bounds__(8 * kWave)
moe_down_blocks_kernel(DownArgs p)
{
    extern __shared__ u32x4 a_lds[];
    constexpr int WPB = 8;
    constexpr int NTH = WPB * kWave;
    constexpr int KS = G * JB;                    // slots per token (= p.k)
    using LG = LaneGroups<G>;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = (int)(threadIdx.x / kWave);
    const int blk = xcd_contiguous((int)blockIdx.x, (int)gridDim.x);
    const int b = blk % p.B;
    const int hb = (blk / p.B) * (RS * WPB);      // the workgroup's first output
    const int cpr16 = p.I / 16;
    const int cpr = FP4 ? p.I / 32 : cpr16;
    const int nunits = KS * 4 * cpr16;
    const int* ids = p.ids + (size_t)b * KS;
    const float* wts = p.w + (size_t)b * KS;
    const u32x4* asrc = static_cast<const u32x4*>(p.a) + (size_t)b * (size_t)nunits;

    // 1) the copy of a[b] (clamped, unconditional loads, as in the one-pass kernel)
    u32x4 cp[NCP];
#pragma unroll
    for (int q = 0; q < NCP; ++q) {
        const int u = (int)threadIdx.x + q * NTH;
        cp[q] = asrc[u < nunits ? u : nunits - 1];
    }
    __builtin_amdgcn_sched_barrier(0);
    // 2) the token's ids and routing weights, picked per lane group
    const int g = LG::group(lane);
    const int lc = LG::chunk(lane);
    int id_all[KS];
    float w_all[KS];
#pragma unroll
    for (int t = 0; t < KS; ++t) {
        id_all[t] = ids[t];
        w_all[t] = wts[t];
    }
#pragma unroll
    for (int t = 0; t < KS; ++t)
        asm volatile("" ::"s"(id_all[t]), "s"(w_all[t]));
    int eid[JB];
    float wt[JB];
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
        eid[jj] = id_all[G * jj];
        wt[jj] = w_all[G * jj];
#pragma unroll
        for (int gg = 1; gg < G; ++gg) {
            eid[jj] = g == gg ? id_all[gg + G * jj] : eid[jj];
            wt[jj] = g == gg ? w_all[gg + G * jj] : wt[jj];
        }
    }
    // 3) the rows of block r: weight chunk and scale byte of each of the lane's
    // slots (an invalid id reads expert 0's row and makes the output NaN; lanes
    // past the row end re-read its last chunk with factor 0)
    const size_t row_bytes = FP4 ? (size_t)(p.I / 2) : (size_t)p.I;
    const int oc = lc < cpr ? lc : cpr - 1;
    const bool lane_live = lc < cpr;
    float mask[JB];
    size_t row0[JB];
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
        const bool ok = (unsigned)eid[jj] < (unsigned)p.E;
        mask[jj] = lane_live ? (ok ? 1.0f : __builtin_nanf("")) : 0.0f;
        row0[jj] = (size_t)(ok ? eid[jj] : 0) * (size_t)p.H;
    }
    u32x4 wq[2][1][JB];
    uint32_t ws[2][1][JB];
    auto load_block = [&](int r, u32x4 (&q)[1][JB], uint32_t (&sc)[1][JB]) {
        const int h = hb + r * WPB + w;
        const size_t hc = (size_t)(h < p.H ? h : p.H - 1);
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
            const size_t row = row0[jj] + hc;
            q[0][jj] = reinterpret_cast<const u32x4*>(p.wd_q + row * row_bytes)[oc];
            sc[0][jj] = p.wd_s[row * (size_t)(p.I / 32) + (FP4 ? oc : oc >> 1)];
        }
    };
    load_block(0, wq[0], ws[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < NCP; ++q) {
        const int u = (int)threadIdx.x + q * NTH;
        if (u < nunits)
            a_lds[u] = cp[q];
    }
    __syncthreads();                              // the only barrier
#pragma unroll
    for (int r = 0; r < RS; ++r) {
        const int cur = r & 1;
        if (r + 1 < RS)
            load_block(r + 1, wq[cur ^ 1], ws[cur ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
        float acc[1] = {0.0f};
        down_group_dot_multi<JB, FP4, G, 1>(a_lds, KS, lane, cpr, cpr16, wq[cur], ws[cur], wt, mask, acc);
        const float v = wave_sum(acc[0]);
        const int h = hb + r * WPB + w;
        if (lane == 0 && h < p.H) {
            const size_t o = (size_t)b * p.H + h;
            if constexpr (OUT_BF16)
                static_cast<uint16_t*>(p.out)[o] = f32_to_bf16_rne(v);
            else
                static_cast<float*>(p.out)[o] = v;
        }
        __builtin_amdgcn_sched_barrier(0);        // one block's loads ahead of its dots, no more
    }
}

template <int JB, int G, bool FP4>
static hipError_t launch_jg(const DownArgs& p, bool out_bf16, int pair_wpb, int ncp, dim3 grid, dim3 block,
                            size_t lds, hipStream_t s)
{
    constexpr int MAXN = onepass_max_ncp(JB, FP4);
    if constexpr (FP4) {
        if (pair_wpb != 0) {                      // two outputs per wavefront, 4 or 8 wavefronts per workgroup
            const int wpb = pair_wpb;
            const dim3 g2((unsigned)((long)p.B * ((p.H / 2 + wpb - 1) / wpb))), b2((unsigned)(wpb * kWave));
            if (wpb == 4) {
                if (out_bf16)
                    hipLaunchKernelGGL((moe_down_onepass_kernel<JB, G, true, FP4, 2 * MAXN, false, 2, 4>), g2, b2,
                                       lds, s, p);
                else
                    hipLaunchKernelGGL((moe_down_onepass_kernel<JB, G, false, FP4, 2 * MAXN, false, 2, 4>), g2, b2,
                                       lds, s, p);
            } else {
                if (out_bf16)
                    hipLaunchKernelGGL((moe_down_onepass_kernel<JB, G, true, FP4, MAXN, false, 2>), g2, b2, lds, s, p);
                else
                    hipLaunchKernelGGL((moe_down_onepass_kernel<JB, G, false, FP4, MAXN, false, 2>), g2, b2, lds, s, p);
            }
            return hipGetLastError();
        }
    }
#define MOED_OP(O, N, ONE) \
    hipLaunchKernelGGL((moe_down_onepass_kernel<JB, G, O, FP4, N, ONE>), grid, block, lds, s, p)
    // single-token calls of k = 8 slots: the exact copy count (one to four loads)
    if constexpr (JB * G == 8) {
        if (p.B == 1 && ncp <= 4) {
            switch (ncp * 2 + (out_bf16 ? 1 : 0)) {
            case 2: MOED_OP(false, 1, true); break;
            case 3: MOED_OP(true, 1, true); break;
            case 4: MOED_OP(false, 2, true); break;
            case 5: MOED_OP(true, 2, true); break;
            case 6: MOED_OP(false, 3, true); break;
            case 7: MOED_OP(true, 3, true); break;
            case 8: MOED_OP(false, 4, true); break;
            default: MOED_OP(true, 4, true); break;
            }
            return hipGetLastError();
        }
    }
    if (out_bf16)
        MOED_OP(true, MAXN, false);
    else
        MOED_OP(false, MAXN, false);
#undef MOED_OP
    return hipGetLastError();
}

template <int G>
static hipError_t launch_g(const DownArgs& p, int jb, bool out_bf16, int pair_wpb, int ncp, dim3 grid, dim3 block,
                           size_t lds, hipStream_t s)
{
    const bool fp4 = p.wfmt == kMXFP4;
    switch (jb * 2 + (fp4 ? 1 : 0)) {
    case 1 * 2 + 0: return launch_jg<1, G, false>(p, out_bf16, pair_wpb, ncp, grid, block, lds, s);
    case 1 * 2 + 1: return launch_jg<1, G, true>(p, out_bf16, pair_wpb, ncp, grid, block, lds, s);
    case 2 * 2 + 0: return launch_jg<2, G, false>(p, out_bf16, pair_wpb, ncp, grid, block, lds, s);
    case 2 * 2 + 1: return launch_jg<2, G, true>(p, out_bf16, pair_wpb, ncp, grid, block, lds, s);
    case 4 * 2 + 0: return launch_jg<4, G, false>(p, out_bf16, pair_wpb, ncp, grid, block, lds, s);
    case 4 * 2 + 1: return launch_jg<4, G, true>(p, out_bf16, pair_wpb, ncp, grid, block, lds, s);
    case 8 * 2 + 0: return launch_jg<8, G, false>(p, out_bf16, pair_wpb, ncp, grid, block, lds, s);
    case 8 * 2 + 1: return launch_jg<8, G, true>(p, out_bf16, pair_wpb, ncp, grid, block, lds, s);
    default: return hipErrorInvalidValue;
    }
}

template <int JB, int G, bool FP4>
static hipError_t launch_blocks_jg(const DownArgs& p, bool out_bf16, size_t lds, hipStream_t s)
{
    constexpr int MAXN = onepass_max_ncp(JB, FP4);
    const dim3 grid((unsigned)((long)p.B * (p.H / (8 * kDownBlocks)))), block(8 * kWave);
    if (out_bf16)
        hipLaunchKernelGGL((moe_down_blocks_kernel<JB, G, true, FP4, MAXN, kDownBlocks>), grid, block, lds, s, p);
    else
        hipLaunchKernelGGL((moe_down_blocks_kernel<JB, G, false, FP4, MAXN, kDownBlocks>), grid, block, lds, s, p);
    return hipGetLastError();
}

template <int G>
static hipError_t launch_blocks_g(const DownArgs& p, int jb, bool out_bf16, size_t lds, hipStream_t s)
{
    const bool fp4 = p.wfmt == kMXFP4;
    switch (jb * 2 + (fp4 ? 1 : 0)) {
    case 1 * 2 + 0: return launch_blocks_jg<1, G, false>(p, out_bf16, lds, s);
    case 1 * 2 + 1: return launch_blocks_jg<1, G, true>(p, out_bf16, lds, s);
    case 2 * 2 + 0: return launch_blocks_jg<2, G, false>(p, out_bf16, lds, s);
    case 2 * 2 + 1: return launch_blocks_jg<2, G, true>(p, out_bf16, lds, s);
    case 4 * 2 + 0: return launch_blocks_jg<4, G, false>(p, out_bf16, lds, s);
    case 4 * 2 + 1: return launch_blocks_jg<4, G, true>(p, out_bf16, lds, s);
    case 8 * 2 + 0: return launch_blocks_jg<8, G, false>(p, out_bf16, lds, s);
    case 8 * 2 + 1: return launch_blocks_jg<8, G, true>(p, out_bf16, lds, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_down_blocks(const DownArgs& p, int jb, int groups, bool out_bf16, size_t lds, hipStream_t s)
{
    if (p.H % (8 * kDownBlocks) != 0)
        return hipErrorInvalidValue;
    if (groups == 1)
        return launch_blocks_g<1>(p, jb, out_bf16, lds, s);
    if (groups == 2)
        return launch_blocks_g<2>(p, jb, out_bf16, lds, s);
    if (groups == 4)
        return launch_blocks_g<4>(p, jb, out_bf16, lds, s);
    return hipErrorInvalidValue;
}

// pair_wpb: 0 = one output per wavefront, 8 wavefronts per workgroup; 4 or 8 =
// two outputs per wavefront (H even; the caller checks) with that many
// wavefronts per workgroup
hipError_t launch_down_onepass(const DownArgs& p, int jb, int groups, bool out_bf16, int pair_wpb, dim3 grid,
                               dim3 block, size_t lds, hipStream_t s)
{
    const int units = p.k * 4 * (p.I / 16);       // float32 a[b] in 16-byte units
    const int ncp = (units + 511) / 512;
    if (groups == 1)
        return launch_g<1>(p, jb, out_bf16, pair_wpb, ncp, grid, block, lds, s);
    if (groups == 2)
        return launch_g<2>(p, jb, out_bf16, pair_wpb, ncp, grid, block, lds, s);
    if (groups == 4)
        return launch_g<4>(p, jb, out_bf16, pair_wpb, ncp, grid, block, lds, s);
    return hipErrorInvalidValue;
}

}  // namespace moed
