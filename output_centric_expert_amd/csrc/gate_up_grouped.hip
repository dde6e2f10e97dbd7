// Gate/up for large decode batches: the same outputs a[b][j][i] as the
// per-slot kernel, computed so that each expert's rows are decoded once per
// 16 slots instead of once per slot.
//
// When many tokens share an expert (batch 32-64 with top-8 of 128-256
// experts), the per-slot kernel re-reads and re-decodes every routed row once
// per (token, slot): 2-10x the unique weight bytes. Here a workgroup owns
// (expert e, 64 neurons; 128 with 8 wavefronts); it compacts the list of
// slots routed to e (in slot order, from topk_ids), and each wavefront
// computes tiles of 16 neurons x 16 of those slots (up to four tiles per
// pass over the rows) with MFMA:
//   A = the gate (or up) rows, decoded exactly from MXFP8 (or MXFP4) to BF16
//       with the block scale folded into the conversion
//       (v_cvt_scalef32_pk_bf16_fp8 / _fp4; exact for scale codes 10..245
//       (E4M3) or 2..252 (E2M1), where the scaled values stay normal, finite
//       BF16 numbers),
//   B = the BF16 activations of the 16 slots' tokens,
//   D = FP32 accumulators (v_mfma_f32_16x16x32_bf16, products exact in FP32).
// Each output is still written once, by the one lane that holds it, as
// SiLU(g) * u into the chunk-interleaved intermediate. There is no gather of
// activations and no per-expert buffer: the slot list is an index list in LDS.
//
// Every routed expert takes the MFMA path, one slot or many: the weight rows
// are read once per item either way, and with streaming loads the tiles keep
// up with a whole-row wavefront even for single-slot experts (a row path for
// experts with up to two slots measured 10-25% slower at batch 8-32).
//
// MFMA lane layout (v_mfma_f32_16x16x32_bf16): lane l supplies A row l%16 and
// B column l%16, both for k = 8*(l/16) .. +7, and receives D rows
// 4*(l/16) .. +3 of column l%16.
#include <type_traits>

#include "gate_up_body.h"
#include "grouped_common.h"

namespace moed {

struct GroupedRow {
    const uint8_t* gq;      // this lane's gate row (codes)
    const uint8_t* uq;      // up row
    const uint8_t* gs;      // gate row scales
    const uint8_t* us;      // up row scales
    int nsteps;             // MX blocks per row = MFMA K steps
    int n0;                 // first neuron of the wavefront's tile
    int kb;                 // lane / 16
    int col;                // lane % 16
};

// x pieces of one 128-value K group for up to kTiles tiles of 16 slots, shared
// by the workgroup's wavefronts through LDS (two buffers): unit
// (tt*16 + col)*16 + (c ^ col) holds x[slot(tt, col)][128g + 8c .. 8c+7] for
// c = 4*kb + q, the piece MFMA step q of lane (col, kb) reads. The XOR by col
// keeps the cooperative writes (16 threads per slot, one 256-byte run of x
// each) and the MFMA reads (16 lanes, one per slot) free of LDS bank
// conflicts.
constexpr int kXUnitsPerTile = 16 * 16;          // 16-byte units per tile and group
constexpr int kWideUnitsPerWave = 2 * 16 * 16;   // wide loads: 16-byte units of one step, per wavefront

struct GroupW {
    u32x4 g0, g1, u0, u1;                        // this lane's codes of the group (g1/u1: MXFP8 only)
    float gsc, usc;                              // block scales
};

template <bool FP4>
__device__ __forceinline__ GroupW load_group_w(const GroupedRow& r, int g)
{
    GroupW w;
    const int kbase = g * 128 + 32 * r.kb;       // this lane's MX block (value index)
    const int bbase = FP4 ? kbase / 2 : kbase;   // its first code byte
    w.g0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(r.gq + bbase));
    w.u0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(r.uq + bbase));
    if constexpr (FP4) {
        w.g1 = w.g0;
        w.u1 = w.u0;
    } else {
        w.g1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(r.gq + bbase + 16));
        w.u1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(r.uq + bbase + 16));
    }
    w.gsc = ue8m0_to_f32(r.gs[4 * g + r.kb]);
    w.usc = ue8m0_to_f32(r.us[4 * g + r.kb]);
    return w;
}

// The four MFMA steps of one 128-code group for NTL tiles: decode this lane's
// codes of the group (wc) and multiply them with the slots' x pieces in LDS
// (xb, the unit layout above).
template <int NTL, bool FP4>
__device__ __forceinline__ void group_mfma(const GroupW& wc, const u32x4* xb, const GroupedRow& r,
                                           f32x4 (&dg)[NTL], f32x4 (&du)[NTL])
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        bf16x8 ag, au;
        if constexpr (FP4) {                      // dword q = codes 8q .. 8q+7
            ag = decode8_scaled_fp4(wc.g0[q], wc.gsc);
            au = decode8_scaled_fp4(wc.u0[q], wc.usc);
        } else {
            const u32x4 gsrc = q < 2 ? wc.g0 : wc.g1;
            const u32x4 usrc = q < 2 ? wc.u0 : wc.u1;
            const u32x2 cgq = (q & 1) ? u32x2{gsrc.z, gsrc.w} : u32x2{gsrc.x, gsrc.y};
            const u32x2 cuq = (q & 1) ? u32x2{usrc.z, usrc.w} : u32x2{usrc.x, usrc.y};
            ag = decode8_scaled(cgq, wc.gsc);
            au = decode8_scaled(cuq, wc.usc);
        }
        const int c = 4 * r.kb + q;
#pragma unroll
        for (int tt = 0; tt < NTL; ++tt) {
            const bf16x8 bx = __builtin_bit_cast(bf16x8, xb[(tt * 16 + r.col) * 16 + (c ^ r.col)]);
            dg[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ag, bx, dg[tt], 0, 0, 0);
            du[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(au, bx, du[tt], 0, 0, 0);
        }
    }
}

// MX blocks after the last whole 128-code group (H/32 not a multiple of 4):
// x straight from global memory, plain k order.
template <int NTL, bool FP4>
__device__ __forceinline__ void leftover_blocks(const GroupedRow& r, const uint16_t* const (&xr)[NTL],
                                                f32x4 (&dg)[NTL], f32x4 (&du)[NTL])
{
    for (int st = 4 * (r.nsteps / 4); st < r.nsteps; ++st) {
        const int k0 = st * 32 + 8 * r.kb;
        bf16x8 ag, au;
        if constexpr (FP4) {
            const uint32_t cg = *reinterpret_cast<const uint32_t*>(r.gq + k0 / 2);
            const uint32_t cu = *reinterpret_cast<const uint32_t*>(r.uq + k0 / 2);
            ag = decode8_scaled_fp4(cg, ue8m0_to_f32(r.gs[st]));
            au = decode8_scaled_fp4(cu, ue8m0_to_f32(r.us[st]));
        } else {
            const u32x2 cg = *reinterpret_cast<const u32x2*>(r.gq + k0);
            const u32x2 cu = *reinterpret_cast<const u32x2*>(r.uq + k0);
            ag = decode8_scaled(cg, ue8m0_to_f32(r.gs[st]));
            au = decode8_scaled(cu, ue8m0_to_f32(r.us[st]));
        }
#pragma unroll
        for (int tt = 0; tt < NTL; ++tt) {
            const bf16x8 bx = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xr[tt] + k0));
            dg[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ag, bx, dg[tt], 0, 0, 0);
            du[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(au, bx, du[tt], 0, 0, 0);
        }
    }
}

// SiLU(g) * u of the tiles' real slots: lane holds D rows 4*kb .. +3 (neurons)
// of column col of each tile.
template <int NTL, bool A_BF16>
__device__ __forceinline__ void store_tiles(const GateUpArgs& p, const GroupedRow& r, const int (&bj)[NTL],
                                            int count, int t0, const f32x4 (&dg)[NTL], const f32x4 (&du)[NTL])
{
#pragma unroll
    for (int tt = 0; tt < NTL; ++tt) {
        if ((t0 + tt) * 16 + r.col < count) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i = r.n0 + 4 * r.kb + q;
                const float v = swiglu(dg[tt][q], du[tt][q]);
                const size_t idx = inter_index<A_BF16>(bj[tt], i, p.I);
                if constexpr (A_BF16)
                    static_cast<uint16_t*>(p.a)[idx] = f32_to_bf16_rne(v);
                else
                    static_cast<float*>(p.a)[idx] = v;
            }
        }
    }
}

// One pass over the rows for NTL tiles of 16 slots (tiles t0 .. t0+NTL-1),
// with the slots' x shared through LDS and the next group's x and weight rows
// loaded while the current group's MFMAs run. Every thread of the workgroup
// calls it (it has barriers); `store` is false for wavefronts whose neurons
// lie past I (they compute on a clamped row and write nothing). K is walked
// in groups of 4 MX blocks (128 codes): inside a group, lane (row, kb)
// supplies block kb's 32 contiguous codes over the 4 MFMA steps and x uses the
// same k order, so the products summed are the row-times-x products, only in
// another order. Leftover blocks (H/32 not a multiple of 4) take x from
// global memory in plain k order.
template <int NTL, bool A_BF16, bool FP4>
__device__ __forceinline__ void grouped_pass(const GateUpArgs& p, const GroupedRow& r, const uint16_t* slots,
                                             int count, int t0, u32x4* xs, bool store)
{
    const int H = p.H;
    const int tid = threadIdx.x;
    const int lcol = tid / 16;                    // cooperative x load: slot column ...
    const int lc = tid % 16;                      // ... and 16-byte piece of the group
    const uint16_t* xl[NTL];                      // x row of this thread's load column, per tile
    int bj[NTL];                                  // slot of this lane's MFMA column, per tile
    const uint16_t* xr[NTL];
#pragma unroll
    for (int tt = 0; tt < NTL; ++tt) {
        const int sl = (t0 + tt) * 16 + lcol;
        xl[tt] = p.x + (size_t)(slots[sl < count ? sl : count - 1] / p.k) * (size_t)H;
        const int si = (t0 + tt) * 16 + r.col;
        bj[tt] = slots[si < count ? si : count - 1];  // extra columns repeat a slot
        xr[tt] = p.x + (size_t)(bj[tt] / p.k) * (size_t)H;
    }
    f32x4 dg[NTL], du[NTL];
#pragma unroll
    for (int tt = 0; tt < NTL; ++tt) {
        dg[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        du[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const int ngroups = r.nsteps / 4;
    constexpr int kBuf = NTL * kXUnitsPerTile;
    u32x4 xreg[NTL];
    GroupW wc{};
    if (ngroups > 0) {
#pragma unroll
        for (int tt = 0; tt < NTL; ++tt)
            xreg[tt] = *reinterpret_cast<const u32x4*>(xl[tt] + 8 * lc);
        wc = load_group_w<FP4>(r, 0);
#pragma unroll
        for (int tt = 0; tt < NTL; ++tt)
            xs[(tt * 16 + lcol) * 16 + (lc ^ lcol)] = xreg[tt];
    }
    __syncthreads();
    for (int g = 0; g < ngroups; ++g) {
        const u32x4* xb = xs + (g & 1) * kBuf;
        const bool more = g + 1 < ngroups;
        GroupW wn = wc;
        if (more) {                               // next group's loads, ahead of this group's MFMAs
#pragma unroll
            for (int tt = 0; tt < NTL; ++tt)
                xreg[tt] = *reinterpret_cast<const u32x4*>(xl[tt] + (g + 1) * 128 + 8 * lc);
            wn = load_group_w<FP4>(r, g + 1);
        }
        group_mfma<NTL, FP4>(wc, xb, r, dg, du);
        if (more) {
            u32x4* xn = xs + ((g + 1) & 1) * kBuf;
#pragma unroll
            for (int tt = 0; tt < NTL; ++tt)
                xn[(tt * 16 + lcol) * 16 + (lc ^ lcol)] = xreg[tt];
        }
        __syncthreads();                          // buffer g&1 read by all, buffer (g+1)&1 written
        wc = wn;
    }
    leftover_blocks<NTL, FP4>(r, xr, dg, du);
    if (store)
        store_tiles<NTL, A_BF16>(p, r, bj, count, t0, dg, du);
}

// Wide weight loads (the default MFMA path when H is a multiple of 512). The
// 128-byte row slices of a 16-row tile, one per lane group, cap the weight
// stream near 4.8 TB/s on MI355X; runs of 256 bytes per row, streamed, with
// the scales in 16-byte blocks, reach about 7 TB/s. So the wavefront reads
// its 16 gate and 16 up rows in steps of 256 bytes per row (two 128-code
// groups of MXFP8, four of MXFP4): load i of lane L takes the 16-byte piece
// L % 16 of row L / 16 + 4i, and each load instruction covers four whole
// 256-byte runs. A step is moved into the MFMA operand layout through a
// wavefront-private LDS region of 2 x 16 rows x 16 pieces (piece b of row n at
// unit 16n + (b ^ n), which keeps both the writes and the operand reads free
// of bank conflicts), and lane (col, kb) reads for group h of the step the
// pieces holding MX block 4h + kb of row col: the codes the 128-byte slices
// give it, in the same order, so the results are the same floats.
template <bool FP4>
struct StepW {
    static constexpr int kGroups = FP4 ? 4 : 2;  // 128-code groups per 256-byte step
    u32x4 g[4], u[4];                            // pieces of rows L/16 + 4i
};

// gq0 / uq0: the wavefront's first gate / up row (wave-uniform); lo: this
// lane's byte offset (lane/16)*rstride + 16*(lane%16); rs4 = 4*rstride. Uniform
// bases plus 32-bit lane offsets shared by both matrices keep the addresses of
// the eight loads in four registers.
template <bool FP4>
__device__ __forceinline__ StepW<FP4> load_step(const uint8_t* gq0, const uint8_t* uq0, uint32_t lo, uint32_t rs4,
                                                int step)
{
    StepW<FP4> w;
    const uint32_t base = lo + 256u * (uint32_t)step;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t o = base + (uint32_t)i * rs4;
        w.g[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(gq0 + o));
        w.u[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(uq0 + o));
    }
    return w;
}

template <bool FP4>
__device__ __forceinline__ void stage_step(const StepW<FP4>& w, u32x4* tb, int lane)
{
    const int b = lane % 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int n = lane / 16 + 4 * i;
        tb[n * 16 + (b ^ n)] = w.g[i];
        tb[256 + n * 16 + (b ^ n)] = w.u[i];
    }
}

template <bool FP4>
__device__ __forceinline__ GroupW staged_group(const u32x4* tb, const GroupedRow& r, int h, float gsc, float usc)
{
    GroupW w;
    const u32x4* row = tb + r.col * 16;
    if constexpr (FP4) {                         // block 4h + kb = piece 4h + kb
        const int q = (4 * h + r.kb) ^ r.col;
        w.g0 = row[q];
        w.u0 = row[256 + q];
        w.g1 = w.g0;
        w.u1 = w.u0;
    } else {                                     // block 4h + kb = pieces 8h + 2kb, +1
        const int q0 = (8 * h + 2 * r.kb) ^ r.col;
        const int q1 = (8 * h + 2 * r.kb + 1) ^ r.col;
        w.g0 = row[q0];
        w.g1 = row[q1];
        w.u0 = row[256 + q0];
        w.u1 = row[256 + q1];
    }
    w.gsc = gsc;
    w.usc = usc;
    return w;
}

// grouped_pass with the wide weight loads (H a multiple of 512, so a row is a
// whole number of 256-byte steps and, for MXFP8, of two-step scale blocks).
// One step of weights is in flight ahead (issued during the step's
// second-to-last group), with it the next scale block, and the slots' x two
// groups ahead in two register sets (group g's set is refilled with x of group
// g+2 once it is in LDS), so neither the L2 latency of x nor that of the rows
// is paid once per group. Each group's wait for its x never waits for weight
// loads issued after it. tb = this wavefront's LDS region (512 units);
// gs0 / us0 / sstride: the scale row of the lane's block-load row slot (gate
// for lanes 0-31, up for 32-63; row (L % 32) / 2) and the scale row stride.
// NW = 8: the workgroup's two halves of 4 wavefronts load alternate x tiles
// (with an odd tile count both load the last one and store the same values).
template <int NTL, bool A_BF16, bool FP4, int NW = kGroupWaves>
__device__ __forceinline__ void grouped_pass_wide(const GateUpArgs& p, const GroupedRow& r, const uint8_t* gq0,
                                                  const uint8_t* uq0, size_t rstride, const uint8_t* sq0,
                                                  const uint16_t* slots, int count, int t0, u32x4* xs, u32x4* tb, bool store)
{
    constexpr int GPS = StepW<FP4>::kGroups;
    constexpr int NH = NW / 4;                    // workgroup halves sharing the x loads
    constexpr int NX = (NTL + NH - 1) / NH;       // x tiles per thread
    const int H = p.H;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int half = NH == 1 ? 0 : tid / 256;
    const int lcol = NH == 1 ? tid / 16 : (tid % 256) / 16;
    const int lc = tid % 16;
    uint32_t xo[NX];                              // element offset of this thread's x row, per x tile
    uint32_t xd[NX];                              // its LDS unit in a group's buffer
#pragma unroll
    for (int i = 0; i < NX; ++i) {
        const int tt = NH * i + half < NTL ? NH * i + half : NTL - 1;
        const int sl = (t0 + tt) * 16 + lcol;
        xo[i] = (uint32_t)(slots[sl < count ? sl : count - 1] / p.k) * (uint32_t)H + 8u * (uint32_t)lc;
        xd[i] = (uint32_t)((tt * 16 + lcol) * 16 + (lc ^ lcol));
    }
    int bj[NTL];
#pragma unroll
    for (int tt = 0; tt < NTL; ++tt) {
        const int si = (t0 + tt) * 16 + r.col;
        bj[tt] = slots[si < count ? si : count - 1];
    }
    f32x4 dg[NTL], du[NTL];
#pragma unroll
    for (int tt = 0; tt < NTL; ++tt) {
        dg[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        du[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const int ngroups = r.nsteps / 4;
    const int nst = ngroups / GPS;                // 256-byte steps (even for MXFP8)
    const uint32_t lo = (uint32_t)(lane / 16) * (uint32_t)rstride + 16u * (uint32_t)(lane % 16);
    const uint32_t rs4 = 4u * (uint32_t)rstride;
    constexpr int kBuf = NTL * kXUnitsPerTile;
    u32x4 xq[2][NX];                              // x of groups g+1 and g+2, by group parity
    auto load_x = [&](u32x4 (&dst)[NX], int g) {
#pragma unroll
        for (int i = 0; i < NX; ++i)
            dst[i] = *reinterpret_cast<const u32x4*>(p.x + (xo[i] + 128u * (uint32_t)g));
    };
    auto put_x = [&](const u32x4 (&src)[NX], int g) {
        u32x4* xn = xs + (g & 1) * kBuf;
#pragma unroll
        for (int i = 0; i < NX; ++i)
            xn[xd[i]] = src[i];
    };
    load_x(xq[0], 0);
    load_x(xq[1], 1);
    StepW<FP4> sw = load_step<FP4>(gq0, uq0, lo, rs4, 0);
    u32x2 sb = load_scale_block(sq0, 0, lane);
    put_x(xq[0], 0);
    __syncthreads();
    // No branch around a load in the step loop (the last groups re-read the last
    // group's x, the last step re-reads the last step): a load behind a branch
    // makes the compiler wait for every load at the join, the ones issued a
    // group or a step ahead included. After the last group put_x fills the
    // other buffer with a copy nobody reads.
    // group g uses x set P = g&1: the caller first requests x of g+2 into it
    // (xload) -- before a step's rows, so that waiting for that x later never
    // waits for rows issued behind it
    // (the scheduling barrier keeps the x loads ahead of the rows requested
    // next: issued after them, waiting for that x would wait for those rows)
    auto xload = [&](auto par, int g) {
        constexpr int P = decltype(par)::value;
        load_x(xq[P], g + 2 < ngroups ? g + 2 : ngroups - 1);
        __builtin_amdgcn_sched_barrier(0);
    };
    // group g = step group h with the lane's gate and up scales: the MFMAs on
    // x buffer g&1, then x of g+1 (set 1-P) into the other buffer
    auto group = [&](auto par, int g, int h, float gsc, float usc) {
        constexpr int P = decltype(par)::value;
        group_mfma<NTL, FP4>(staged_group<FP4>(tb, r, h, gsc, usc), xs + (g & 1) * kBuf, r, dg, du);
        put_x(xq[1 - P], g + 1 < ngroups ? g + 1 : ngroups - 1);
        __syncthreads();
    };
    constexpr auto P0 = std::integral_constant<int, 0>{};
    constexpr auto P1 = std::integral_constant<int, 1>{};
    if constexpr (GPS == 2) {
        // MXFP8: a scale block spans two steps, so steps go in pairs; the next
        // step's rows (and, in the second step, the next block) are requested
        // during each step's first group
        for (int s = 0; s < nst; s += 2) {
            const int g0 = 2 * s;
            // each step's two groups' scales at the step start (sb is refilled
            // in the second step, after its scales are taken)
            float gsc0 = block_scale<0>(sb, r.col, r.kb), usc0 = block_scale<0>(sb, 16 + r.col, r.kb);
            float gsc1 = block_scale<1>(sb, r.col, r.kb), usc1 = block_scale<1>(sb, 16 + r.col, r.kb);
            stage_step<FP4>(sw, tb, lane);
            xload(P0, g0);
            sw = load_step<FP4>(gq0, uq0, lo, rs4, s + 1);
            group(P0, g0, 0, gsc0, usc0);
            xload(P1, g0 + 1);
            group(P1, g0 + 1, 1, gsc1, usc1);
            gsc0 = block_scale<2>(sb, r.col, r.kb);
            usc0 = block_scale<2>(sb, 16 + r.col, r.kb);
            gsc1 = block_scale<3>(sb, r.col, r.kb);
            usc1 = block_scale<3>(sb, 16 + r.col, r.kb);
            stage_step<FP4>(sw, tb, lane);
            const int sn = s + 2 < nst ? s + 2 : s + 1;
            xload(P0, g0 + 2);
            sw = load_step<FP4>(gq0, uq0, lo, rs4, sn);
            sb = load_scale_block(sq0, sn / 2, lane);
            group(P0, g0 + 2, 0, gsc0, usc0);
            xload(P1, g0 + 3);
            group(P1, g0 + 3, 1, gsc1, usc1);
        }
    } else {
        // MXFP4: one scale block per step; the next step and block are
        // requested at the step start, a whole step (four groups) ahead. Every
        // x the step waits for is requested before them: x of the step's groups
        // 2..4 ahead of its rows (set (g % 4) of xq4 holds x of group g), x of
        // group 1 a step earlier, x of the next step's group 1 during group 2
        // (first waited for after the next step's rows are in).
        u32x4 xq4[4][NX];
#pragma unroll
        for (int i = 0; i < NX; ++i)
            xq4[1][i] = xq[1][i];
        auto xput = [&](int g, const u32x4 (&src)[NX], int h, float gsc, float usc) {
            group_mfma<NTL, FP4>(staged_group<FP4>(tb, r, h, gsc, usc), xs + (g & 1) * kBuf, r, dg, du);
            put_x(src, g + 1 < ngroups ? g + 1 : ngroups - 1);
            __syncthreads();
        };
        auto clampg = [&](int g) { return g < ngroups ? g : ngroups - 1; };
        for (int s = 0; s < nst; ++s) {
            const int g0 = 4 * s;
            // all four groups' scales at the step start (four groups per step: taking
            // them per group would put a ds_bpermute round trip before each decode)
            float gsc[4], usc[4];
            gsc[0] = block_scale<0>(sb, r.col, r.kb);
            usc[0] = block_scale<0>(sb, 16 + r.col, r.kb);
            gsc[1] = block_scale<1>(sb, r.col, r.kb);
            usc[1] = block_scale<1>(sb, 16 + r.col, r.kb);
            gsc[2] = block_scale<2>(sb, r.col, r.kb);
            usc[2] = block_scale<2>(sb, 16 + r.col, r.kb);
            gsc[3] = block_scale<3>(sb, r.col, r.kb);
            usc[3] = block_scale<3>(sb, 16 + r.col, r.kb);
            stage_step<FP4>(sw, tb, lane);
            load_x(xq4[2], clampg(g0 + 2));
            load_x(xq4[3], clampg(g0 + 3));
            load_x(xq4[0], clampg(g0 + 4));
            __builtin_amdgcn_sched_barrier(0);
            const int sn = s + 1 < nst ? s + 1 : s;
            sw = load_step<FP4>(gq0, uq0, lo, rs4, sn);
            sb = load_scale_block(sq0, sn, lane);
            __builtin_amdgcn_sched_barrier(0);
            xput(g0, xq4[1], 0, gsc[0], usc[0]);
            xput(g0 + 1, xq4[2], 1, gsc[1], usc[1]);
            load_x(xq4[1], clampg(g0 + 5));
            __builtin_amdgcn_sched_barrier(0);
            xput(g0 + 2, xq4[3], 2, gsc[2], usc[2]);
            xput(g0 + 3, xq4[0], 3, gsc[3], usc[3]);
        }
    }
    if (store)
        store_tiles<NTL, A_BF16>(p, r, bj, count, t0, dg, du);
}

// One item: expert e, neurons n_block .. n_block+16*NW-1, the count >= 1 slots
// routed to e in slots[] (slot order). Every thread of the workgroup calls it.
template <bool A_BF16, bool FP4, bool WIDE, int NW = kGroupWaves>
__device__ __forceinline__ void gate_up_item(const GateUpArgs& p, int e, int n_block, int count, const uint16_t* slots,
                                             u32x4* xs)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int I = p.I;
    const int H = p.H;
    const int n0 = n_block + 16 * w;              // this wavefront's 16 neurons
    const bool store = n0 < I;                    // wavefronts past I still take part in the barriers

    const int kb = lane / 16;                     // which quarter of a k group
    const int col = lane % 16;                    // A row (neuron) / B column (slot)
    const int nr = store ? n0 + col : I - 1;      // a valid row for the wavefronts past I
    const size_t row = (size_t)e * (size_t)I + (size_t)(nr < I ? nr : I - 1);
    const size_t row_bytes = FP4 ? (size_t)(H / 2) : (size_t)H;
    const uint8_t* gq = p.wg_q + row * row_bytes;
    const uint8_t* uq = p.wu_q + row * row_bytes;
    const uint8_t* gs = p.wg_s + row * (size_t)(H / 32);
    const uint8_t* us = p.wu_s + row * (size_t)(H / 32);
    const int nsteps = H / 32;                    // MX blocks per row = MFMA K steps
    const int ntiles = (count + 15) / 16;

    // Each pass covers up to kTiles tiles of 16 slots, so a row is decoded once
    // per 16*kTiles slots; the tile count of a pass is a template argument, so
    // the hot loop has no per-tile branches.
    const GroupedRow r{gq, uq, gs, us, nsteps, n0, kb, col};
    if constexpr (WIDE) {
        // the wavefront's first row (all 16 rows clamped to I-1 past I), its
        // row stride, and its LDS region for the wide loads
        // (wave-uniform: readfirstlane lets the loads take them from SGPRs)
        const int wrow_i = __builtin_amdgcn_readfirstlane(store ? n0 : I - 1);
        const size_t wrow = (size_t)e * (size_t)I + (size_t)wrow_i;
        const size_t rstride = store ? row_bytes : 0;
        const uint8_t* gq0 = p.wg_q + wrow * row_bytes;
        const uint8_t* uq0 = p.wu_q + wrow * row_bytes;
        // the lane's scale row for the block loads: gate rows for lanes 0-31,
        // up rows for 32-63, row (lane % 32) / 2 of the wavefront's 16
        const size_t srow = wrow + (store ? (size_t)((lane % 32) / 2) : 0);
        const uint8_t* sq0 = (lane < 32 ? p.wg_s : p.wu_s) + srow * (size_t)(H / 32);
        u32x4* tb = xs + 2 * kTiles * kXUnitsPerTile + w * kWideUnitsPerWave;
        for (int t0 = 0; t0 < ntiles; t0 += kTiles) {
            const int nt = ntiles - t0 < kTiles ? ntiles - t0 : kTiles;
            switch (nt) {
            case 1: grouped_pass_wide<1, A_BF16, FP4, NW>(p, r, gq0, uq0, rstride, sq0, slots, count, t0, xs, tb, store); break;
            case 2: grouped_pass_wide<2, A_BF16, FP4, NW>(p, r, gq0, uq0, rstride, sq0, slots, count, t0, xs, tb, store); break;
            case 3: grouped_pass_wide<3, A_BF16, FP4, NW>(p, r, gq0, uq0, rstride, sq0, slots, count, t0, xs, tb, store); break;
            default: grouped_pass_wide<4, A_BF16, FP4, NW>(p, r, gq0, uq0, rstride, sq0, slots, count, t0, xs, tb, store); break;
            }
        }
    } else {
        for (int t0 = 0; t0 < ntiles; t0 += kTiles) {
            const int nt = ntiles - t0 < kTiles ? ntiles - t0 : kTiles;
            switch (nt) {
            case 1: grouped_pass<1, A_BF16, FP4>(p, r, slots, count, t0, xs, store); break;
            case 2: grouped_pass<2, A_BF16, FP4>(p, r, slots, count, t0, xs, store); break;
            case 3: grouped_pass<3, A_BF16, FP4>(p, r, slots, count, t0, xs, store); break;
            default: grouped_pass<4, A_BF16, FP4>(p, r, slots, count, t0, xs, store); break;
            }
        }
    }
}

// The grouped gate/up: invalid slots first (workgroup q < blocks writes NaN
// for neuron block q of every slot whose id is outside [0, E)), then the
// items (expert, block of 16*NW neurons): with the work list (wl_off >= 0, its
// place in the dynamic LDS) the routed experts' items with a stride of the
// grid size, else one item per workgroup over all E experts.
template <bool A_BF16, bool FP4, bool WIDE, int NW, bool WIN>
__device__ __forceinline__ void gate_up_grouped_body(const GateUpArgs& p, int wl_off)
{
    // up to kSlotCap slot entries of 16 bits (B*k < 65536), the x tiles, then
    // the work list
    extern __shared__ int smem[];
    uint16_t* slots = reinterpret_cast<uint16_t*>(smem);
    __shared__ int wave_cnt[NW];
    constexpr int kNeurons = 16 * NW;            // neurons per item
    const int nblk = (p.I + kNeurons - 1) / kNeurons;
    const int nslots = p.B * p.k;
    const int E = p.E;
    const int I = p.I;

    if ((int)blockIdx.x < nblk) {
        const int n_block = (int)blockIdx.x * kNeurons;
        auto bad = [&](int v) { return (unsigned)v >= (unsigned)E; };
        for (int lo = 0;; lo += kSlotCap) {       // in windows of kSlotCap invalid slots
            int nw;
            if constexpr (WIN) {
                const int nbad = compact_slots<NW, decltype(bad), uint16_t, true>(nslots, p.ids, slots, wave_cnt,
                                                                                  bad, lo, kSlotCap);
                nw = nbad - lo < kSlotCap ? nbad - lo : kSlotCap;
            } else {
                nw = compact_slots<NW>(nslots, p.ids, slots, wave_cnt, bad);   // the whole list at once
            }
            for (int q = threadIdx.x; q < nw * kNeurons; q += blockDim.x) {
                const int bj = slots[q / kNeurons];
                const int i = n_block + q % kNeurons;
                if (i < I) {
                    const size_t idx = inter_index<A_BF16>(bj, i, I);
                    if constexpr (A_BF16)
                        static_cast<uint16_t*>(p.a)[idx] = 0x7FC0u;
                    else
                        static_cast<float*>(p.a)[idx] = __builtin_nanf("");
                }
            }
            __syncthreads();                      // the list is rewritten next
            if (!WIN || nw < kSlotCap)
                break;
        }
    }
    const int cap = WIN ? kSlotCap : nslots;
    u32x4* xs = reinterpret_cast<u32x4*>(slots + ((cap + 7) & ~7));   // x tiles, after the slot list
    const int* act = nullptr;
    if constexpr (WIN) {
        // items (expert, neuron block, window of kSlotCap slots)
        int nwin = (nslots + kSlotCap - 1) / kSlotCap;   // without the work list: as many as B*k could need
        int n_items;
        if (wl_off >= 0) {
            int* mark = smem + wl_off;
            int* list = mark + E;
            n_items = routed_experts_windows<NW>(nslots, p.ids, E, mark, list, wave_cnt, nwin) * nblk * nwin;
            act = list;
        } else {
            n_items = E * nblk * nwin;
        }
        const int ipe = nblk * nwin;
        for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
            const int e = act ? act[item / ipe] : item / ipe;
            const int lo = (item % nwin) * kSlotCap;
            auto mine = [&](int v) { return v == e; };
            const int count = compact_slots<NW, decltype(mine), uint16_t, true>(nslots, p.ids, slots, wave_cnt, mine,
                                                                                lo, kSlotCap);
            if (count <= lo)
                continue;                         // whole workgroup (no slots in this window)
            gate_up_item<A_BF16, FP4, WIDE, NW>(p, e, ((item % ipe) / nwin) * kNeurons,
                                                count - lo < kSlotCap ? count - lo : kSlotCap, slots, xs);
            __syncthreads();                      // the next item rewrites the slot list and the x tiles
        }
    } else {
        // items (expert, neuron block), every slot in one list
        int n_items = E * nblk;
        if (wl_off >= 0) {
            int* mark = smem + wl_off;
            int* list = mark + E;
            n_items = routed_experts<NW>(nslots, p.ids, E, mark, list, wave_cnt) * nblk;
            act = list;
        }
        for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
            const int e = act ? act[item / nblk] : item / nblk;
            const int count = compact_slots<NW>(nslots, p.ids, slots, wave_cnt, [&](int v) { return v == e; });
            if (count == 0)
                continue;                         // whole workgroup (only without the work list)
            gate_up_item<A_BF16, FP4, WIDE, NW>(p, e, (item % nblk) * kNeurons, count, slots, xs);
            __syncthreads();                      // the next item rewrites the slot list and the x tiles
        }
    }
}

// WIN: the slots of an expert taken in windows of kSlotCap (B*k > kSlotCap)
template <bool A_BF16, bool FP4, bool WIN>
__global__ void __launch_bounds__(kGroupWaves * kWave)
moe_gate_up_grouped_kernel(GateUpArgs p, int wl_off)
{
    gate_up_grouped_body<A_BF16, FP4, false, kGroupWaves, WIN>(p, wl_off);
}

// The wide loads need 8 KiB of LDS per wavefront: two workgroups of 4
// wavefronts share a CU, or one of 8 (items of 128 neurons, each x tile
// loaded once for twice the rows); the register budget is set to match (two
// wavefronts per SIMD).
template <bool A_BF16, bool FP4, int NW, bool WIN>
__global__ void __launch_bounds__(NW * kWave, 8 / NW)
moe_gate_up_grouped_wide_kernel(GateUpArgs p, int wl_off)
{
    gate_up_grouped_body<A_BF16, FP4, true, NW, WIN>(p, wl_off);
}

// The slot list holds all B*k entries while they fit in 64 KiB of LDS with the
// x tiles and the work list (B*k up to about 16000); beyond that, windows of
// kSlotCap. (Windows at smaller batches were measured slower here: each
// workgroup first counts the slots of every expert.)
static bool gate_up_windowed(int B, int k, int E)
{
    const long nslots = (long)B * (long)k;
    return nslots > kSlotCap &&
           (size_t)(nslots + 7) / 8 * 16 + 2 * (size_t)kTiles * kXUnitsPerTile * sizeof(u32x4) + worklist_lds(E) > 65536;
}

size_t gate_up_grouped_lds(int B, int k, int E, bool wide, int nw)
{
    // slot list (16-bit entries, rounded up to 16 bytes; kSlotCap of them with
    // windows), two buffers of x tiles, with the wide loads one 8 KiB region
    // per wavefront, then the work list
    const long nslots = gate_up_windowed(B, k, E) ? kSlotCap : (long)B * (long)k;
    const size_t list = (size_t)(nslots + 7) / 8 * 16;
    return list + 2 * (size_t)kTiles * kXUnitsPerTile * sizeof(u32x4) +
           (wide ? (size_t)nw * kWideUnitsPerWave * sizeof(u32x4) : 0) + worklist_lds(E);
}

template <bool A_BF16, bool FP4, int NW, bool WIN>
static hipError_t launch_wide(dim3 grid, size_t lds, hipStream_t s, const GateUpArgs& p, int wl_off)
{
    // allow dynamic LDS beyond the default 64 KiB, once per device: up to
    // 64 KiB for the slot list and x tiles plus the wide-load regions
    const hipError_t attr =
        set_max_dynamic_lds(reinterpret_cast<const void*>(&moe_gate_up_grouped_wide_kernel<A_BF16, FP4, NW, WIN>),
                            65536 + NW * kWideUnitsPerWave * (int)sizeof(u32x4));
    if (attr != hipSuccess)
        return attr;
    hipLaunchKernelGGL((moe_gate_up_grouped_wide_kernel<A_BF16, FP4, NW, WIN>), grid, dim3(NW * kWave), lds, s, p,
                       wl_off);
    return hipGetLastError();
}

template <bool A_BF16, bool FP4, bool WIDE, bool WIN>
hipError_t launch_grouped_win(dim3 grid, dim3 block, size_t lds, hipStream_t s, const GateUpArgs& p, int wl_off,
                              int nw)
{
    if constexpr (WIDE) {
        return nw == 8 ? launch_wide<A_BF16, FP4, 8, WIN>(grid, lds, s, p, wl_off)
                       : launch_wide<A_BF16, FP4, kGroupWaves, WIN>(grid, lds, s, p, wl_off);
    } else {
        hipLaunchKernelGGL((moe_gate_up_grouped_kernel<A_BF16, FP4, WIN>), grid, block, lds, s, p, wl_off);
    }
    return hipGetLastError();
}

template <bool A_BF16, bool FP4, bool WIDE>
hipError_t launch_grouped(dim3 grid, dim3 block, size_t lds, hipStream_t s, const GateUpArgs& p, int wl_off,
                          int nw)
{
    return gate_up_windowed(p.B, p.k, p.E) ? launch_grouped_win<A_BF16, FP4, WIDE, true>(grid, block, lds, s, p, wl_off, nw)
                                           : launch_grouped_win<A_BF16, FP4, WIDE, false>(grid, block, lds, s, p, wl_off, nw);
}

hipError_t launch_gate_up_grouped(const GateUpArgs& p, bool a_bf16, const Tuning& t, hipStream_t s)
{
    if ((long)p.B * p.k == 0)
        return hipSuccess;
    // wide loads: rows of whole 256-byte steps and whole scale blocks, read as
    // 8-byte pieces (scale arrays at 8-byte aligned bases; else the slices,
    // which give the same floats)
    const bool wide = t.gu_wide != 0 && p.H % 512 == 0 && (((uintptr_t)p.wg_s | (uintptr_t)p.wu_s) & 7u) == 0;
    // 8 wavefronts (items of 128 neurons) pay off once experts average 32 slots
    // or more, where each 64-neuron item would fetch as many bytes of x from
    // L2 as of weights from HBM; below that one 8-wave workgroup per CU hides
    // its barriers worse than two of 4
    const int nw = !wide ? kGroupWaves
                         : t.gu_waves == 8 || (t.gu_waves == 0 && (long)p.B * p.k >= 32L * p.E) ? 8 : kGroupWaves;
    const int nblk = (p.I + 16 * nw - 1) / (16 * nw);
    // items: (expert, neuron block[, window of slots]); without the work list
    // as many windows as B*k slots could need
    const long items = (long)p.E * nblk * (gate_up_windowed(p.B, p.k, p.E) ? ((long)p.B * p.k + kSlotCap - 1) / kSlotCap : 1);
    const size_t lds = gate_up_grouped_lds(p.B, p.k, p.E, wide, nw);
    const size_t wl = worklist_lds(p.E);
    // with the work list: at most gu_grid workgroups (and at least one per
    // neuron block, for the invalid-slot pass) walk the routed experts' items
    const bool use_wl = wl > 0 && t.gu_grid > 0;
    const int wl_off = use_wl ? (int)((lds - wl) / sizeof(int)) : -1;
    long nwg = use_wl && items > t.gu_grid ? t.gu_grid : items;
    if (nwg < nblk)
        nwg = nblk;
    const dim3 grid((unsigned)nwg);
    const dim3 block(kGroupWaves * kWave);
    const bool fp4 = p.wfmt == kMXFP4;
    if (fp4) {
        if (a_bf16)
            return wide ? launch_grouped<true, true, true>(grid, block, lds, s, p, wl_off, nw)
                        : launch_grouped<true, true, false>(grid, block, lds, s, p, wl_off, nw);
        return wide ? launch_grouped<false, true, true>(grid, block, lds, s, p, wl_off, nw)
                    : launch_grouped<false, true, false>(grid, block, lds, s, p, wl_off, nw);
    }
    if (a_bf16)
        return wide ? launch_grouped<true, false, true>(grid, block, lds, s, p, wl_off, nw)
                    : launch_grouped<true, false, false>(grid, block, lds, s, p, wl_off, nw);
    return wide ? launch_grouped<false, false, true>(grid, block, lds, s, p, wl_off, nw)
                : launch_grouped<false, false, false>(grid, block, lds, s, p, wl_off, nw);
}

}  // namespace moed
