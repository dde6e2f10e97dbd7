// Gate/up for large decode batches: the same outputs a[b][j][i] as the
// per-slot kernel, computed so that each expert's rows are decoded once per
// 16 slots instead of once per slot.
//
// When many tokens share an expert (batch 32-64 with top-8 of 128-256
// experts), the per-slot kernel re-reads and re-decodes every routed row once
// per (token, slot): 2-10x the unique weight bytes. Here a workgroup owns
// (expert e, 64 neurons); it compacts the list of slots routed to e (in slot
// order, from topk_ids), and each wavefront computes tiles of 16 neurons x 16
// of those slots (up to four tiles per pass over the rows) with MFMA:
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
// MFMA lane layout (v_mfma_f32_16x16x32_bf16): lane l supplies A row l%16 and
// B column l%16, both for k = 8*(l/16) .. +7, and receives D rows
// 4*(l/16) .. +3 of column l%16.
#include "launch.h"
#include "mx_device.h"

namespace moed {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kGroupWaves = 4;                  // wavefronts per workgroup, 16 neurons each
constexpr int kGroupNeurons = 16 * kGroupWaves;
constexpr int kTiles = 4;                       // 16-slot tiles per pass over a row

// 8 E4M3 codes (two dwords) times 2^(s-127) -> 8 BF16 values, exactly.
__device__ __forceinline__ bf16x8 decode8_scaled(u32x2 codes, float scale)
{
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.x, scale, false);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.x, scale, true);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.y, scale, false);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.y, scale, true);
    bf16x8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// 8 E2M1 codes (one dword, element 2t in the low nibble of byte t) times
// 2^(s-127) -> 8 BF16 values, exactly while the scaled values stay normal,
// finite BF16 numbers (scale codes 2..252).
__device__ __forceinline__ bf16x8 decode8_scaled_fp4(uint32_t codes, float scale)
{
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
    bf16x8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// Deterministic compaction: slots[0..count) = the indices t < n (in increasing
// order) with pred(t). All threads of the workgroup must call it.
template <typename Pred>
__device__ __forceinline__ int compact_slots(int n, int* slots, int* wave_cnt, Pred pred)
{
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    int total = 0;
    for (int base = 0; base < n; base += kGroupWaves * kWave) {
        const int t = base + tid;
        const bool f = t < n && pred(t);
        const unsigned long long m = __ballot(f);
        const int before = __popcll(m & ((1ull << lane) - 1ull));
        if (lane == 0)
            wave_cnt[w] = __popcll(m);
        __syncthreads();
        int off = total;
        for (int q = 0; q < w; ++q)
            off += wave_cnt[q];
        if (f)
            slots[off + before] = t;
        int sum = 0;
        for (int q = 0; q < kGroupWaves; ++q)
            sum += wave_cnt[q];
        __syncthreads();
        total += sum;
    }
    return total;
}

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

// One pass over the rows for NTL tiles of 16 slots (tiles t0 .. t0+NTL-1).
// K is walked in groups of 4 MX blocks (128 codes); inside a group, lane
// (row, kb) supplies block kb's 32 contiguous codes over the 4 MFMA steps
// (8 per step) and x uses the same k order, so the products summed are the
// row-times-x products, only in another order. One 32-byte (MXFP8) or
// 16-byte (MXFP4) load per row and one scale byte per row per group.
template <int NTL, bool A_BF16, bool FP4>
__device__ __forceinline__ void grouped_pass(const GateUpArgs& p, const GroupedRow& r, const int* slots,
                                             int count, int t0)
{
    const int H = p.H;
    int bj[NTL];
    const uint16_t* xr[NTL];
#pragma unroll
    for (int tt = 0; tt < NTL; ++tt) {
        const int si = (t0 + tt) * 16 + r.col;
        const int sidx = si < count ? si : count - 1;   // extra columns repeat a slot
        bj[tt] = slots[sidx];
        xr[tt] = p.x + (size_t)(bj[tt] / p.k) * (size_t)H;
    }
    f32x4 dg[NTL], du[NTL];
#pragma unroll
    for (int tt = 0; tt < NTL; ++tt) {
        dg[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        du[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    int st = 0;
    for (; st + 4 <= r.nsteps; st += 4) {
        const int kbase = st * 32 + 32 * r.kb;    // this lane's MX block (value index)
        const int bbase = FP4 ? kbase / 2 : kbase;   // its first code byte
        const u32x4 g0 = *reinterpret_cast<const u32x4*>(r.gq + bbase);
        const u32x4 u0 = *reinterpret_cast<const u32x4*>(r.uq + bbase);
        const u32x4 g1 = FP4 ? g0 : *reinterpret_cast<const u32x4*>(r.gq + bbase + 16);
        const u32x4 u1 = FP4 ? u0 : *reinterpret_cast<const u32x4*>(r.uq + bbase + 16);
        const float sgf = ue8m0_to_f32(r.gs[st + r.kb]);
        const float suf = ue8m0_to_f32(r.us[st + r.kb]);
        u32x4 xv[NTL][4];
#pragma unroll
        for (int tt = 0; tt < NTL; ++tt)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xv[tt][q] = *reinterpret_cast<const u32x4*>(xr[tt] + kbase + 8 * q);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            bf16x8 ag, au;
            if constexpr (FP4) {                  // dword q = codes 8q .. 8q+7
                ag = decode8_scaled_fp4(g0[q], sgf);
                au = decode8_scaled_fp4(u0[q], suf);
            } else {
                const u32x4 gsrc = q < 2 ? g0 : g1;
                const u32x4 usrc = q < 2 ? u0 : u1;
                const u32x2 cgq = (q & 1) ? u32x2{gsrc.z, gsrc.w} : u32x2{gsrc.x, gsrc.y};
                const u32x2 cuq = (q & 1) ? u32x2{usrc.z, usrc.w} : u32x2{usrc.x, usrc.y};
                ag = decode8_scaled(cgq, sgf);
                au = decode8_scaled(cuq, suf);
            }
#pragma unroll
            for (int tt = 0; tt < NTL; ++tt) {
                const bf16x8 bx = __builtin_bit_cast(bf16x8, xv[tt][q]);
                dg[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ag, bx, dg[tt], 0, 0, 0);
                du[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(au, bx, du[tt], 0, 0, 0);
            }
        }
    }
    for (; st < r.nsteps; ++st) {                 // leftover blocks: plain k order
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
    // lane holds D rows 4*kb .. +3 (neurons) of column col of each tile
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

template <bool A_BF16, bool FP4>
__global__ void __launch_bounds__(kGroupWaves * kWave)
moe_gate_up_grouped_kernel(GateUpArgs p)
{
    extern __shared__ int slots[];               // B*k entries
    __shared__ int wave_cnt[kGroupWaves];
    const int nblk = (p.I + kGroupNeurons - 1) / kGroupNeurons;
    const int e = blockIdx.x / nblk;
    const int n_block = (blockIdx.x % nblk) * kGroupNeurons;
    const int nslots = p.B * p.k;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int* ids = p.ids;
    const int E = p.E;
    const int I = p.I;
    const int H = p.H;

    // slots routed to an id outside [0, E) get NaN, written by expert 0's workgroups
    if (e == 0) {
        const int nbad = compact_slots(nslots, slots, wave_cnt,
                                       [&](int t) { return (unsigned)ids[t] >= (unsigned)E; });
        for (int q = threadIdx.x; q < nbad * kGroupNeurons; q += blockDim.x) {
            const int bj = slots[q / kGroupNeurons];
            const int i = n_block + q % kGroupNeurons;
            if (i < I) {
                const size_t idx = inter_index<A_BF16>(bj, i, I);
                if constexpr (A_BF16)
                    static_cast<uint16_t*>(p.a)[idx] = 0x7FC0u;
                else
                    static_cast<float*>(p.a)[idx] = __builtin_nanf("");
            }
        }
        __syncthreads();                          // the list is reused below
    }
    const int count = compact_slots(nslots, slots, wave_cnt, [&](int t) { return ids[t] == e; });
    if (count == 0)
        return;                                   // whole workgroup: no barrier follows
    const int n0 = n_block + 16 * w;              // this wavefront's 16 neurons
    if (n0 >= I)
        return;

    const int kb = lane / 16;                     // which quarter of a k group
    const int col = lane % 16;                    // A row (neuron) / B column (slot)
    const size_t row = (size_t)e * (size_t)I + (size_t)(n0 + col);
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
    for (int t0 = 0; t0 < ntiles; t0 += kTiles) {
        const int nt = ntiles - t0 < kTiles ? ntiles - t0 : kTiles;
        const GroupedRow r{gq, uq, gs, us, nsteps, n0, kb, col};
        switch (nt) {
        case 1: grouped_pass<1, A_BF16, FP4>(p, r, slots, count, t0); break;
        case 2: grouped_pass<2, A_BF16, FP4>(p, r, slots, count, t0); break;
        case 3: grouped_pass<3, A_BF16, FP4>(p, r, slots, count, t0); break;
        default: grouped_pass<4, A_BF16, FP4>(p, r, slots, count, t0); break;
        }
    }
}

size_t gate_up_grouped_lds(int B, int k)
{
    return (size_t)B * (size_t)k * sizeof(int);
}

hipError_t launch_gate_up_grouped(const GateUpArgs& p, bool a_bf16, const Tuning& t, hipStream_t s)
{
    if ((long)p.B * p.k == 0)
        return hipSuccess;
    const int nblk = (p.I + kGroupNeurons - 1) / kGroupNeurons;
    const dim3 grid((unsigned)((long)p.E * nblk));
    const dim3 block(kGroupWaves * kWave);
    const size_t lds = gate_up_grouped_lds(p.B, p.k);
    (void)t;                                      // rows are re-read per pass: cached loads
    const bool fp4 = p.wfmt == kMXFP4;
    if (fp4) {
        if (a_bf16)
            hipLaunchKernelGGL((moe_gate_up_grouped_kernel<true, true>), grid, block, lds, s, p);
        else
            hipLaunchKernelGGL((moe_gate_up_grouped_kernel<false, true>), grid, block, lds, s, p);
    } else {
        if (a_bf16)
            hipLaunchKernelGGL((moe_gate_up_grouped_kernel<true, false>), grid, block, lds, s, p);
        else
            hipLaunchKernelGGL((moe_gate_up_grouped_kernel<false, false>), grid, block, lds, s, p);
    }
    return hipGetLastError();
}

}  // namespace moed
