// Down for large decode batches (tokens sharing experts): expert-major, so
// each routed down row is read and decoded once per workgroup pass instead of
// once per (token, slot). A pass takes up to 4 tiles of 16 slots with the
// wide loads and a float32 intermediate (two halves of 2 tiles), 3 with bf16;
// with the 128-byte slices 3 tiles of float32, 4 of bf16.
//
// Step 1, moe_down_expert_kernel: a workgroup owns (expert e, RT*64 output
// rows), four wavefronts of RT tiles of 16 rows each. It compacts the list of slots
// s = (b, j) routed to e (in slot order, from topk_ids) and computes, for
// tiles of 16 of those slots, the MFMA product
//   A = Wd[e][h][:], decoded exactly from MXFP8 / MXFP4 to BF16 with the
//       block scale folded into the conversion,
//   B[:, s] = a[s][:], a float32 value carried as two BF16 numbers hi + lo
//       (hi = RNE(v), lo = RNE(v - hi); about 16 significant bits), so that
//       both products are exact in FP32 (a BF16 intermediate needs only hi),
//   D += A * B_hi + A * B_lo   (v_mfma_f32_16x16x32_bf16, FP32 accumulation),
// and writes the slot's weighted partial y[s][h] = w[s] * D[h][s]. The slots'
// a is split once per workgroup and shared by its wavefronts through
// double-buffered LDS tiles (the unit layout of the grouped gate/up kernel);
// each B operand read from LDS serves the wavefront's RT row tiles. K is
// walked in groups of 4 MX blocks with the weight codes requested two groups
// ahead.
//
// Step 2, moe_down_combine_kernel: out[b][h] = sum over j of y[(b, j)][h], the
// token's k slots added in slot order and stored once; a token with an
// expert id outside [0, E) gets NaN.
//
// The per-slot partials are the price of reading each routed row once: they
// take B*k*H*4 bytes of workspace and a second, small HBM-bound launch.
#include <type_traits>

#include "grouped_common.h"

namespace moed {

namespace {

constexpr int kDnUnits = 16 * 16;                // 16-byte units per tile and K group (one of hi / lo)

// 8 float32 values -> 8 bf16 hi and 8 bf16 lo (hi + lo = v to about 2^-17
// relative): hi = RNE(v), lo = RNE(v - hi), two values per conversion.
__device__ __forceinline__ void split8(const f32x4& v0, const f32x4& v1, u32x4& hi, u32x4& lo)
{
    const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t h[4], l[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        h[t] = f32x2_to_bf16x2_rne(v[2 * t], v[2 * t + 1]);
        l[t] = f32x2_to_bf16x2_rne(v[2 * t] - bf16_lo(h[t]), v[2 * t + 1] - bf16_hi(h[t]));
    }
    hi = u32x4{h[0], h[1], h[2], h[3]};
    lo = u32x4{l[0], l[1], l[2], l[3]};
}

// a[s][i0 .. i0+7] (i0 a multiple of 8) from the chunk-interleaved
// intermediate, as loaded: one 16-byte unit of bf16, or two of float32.
template <bool A_BF16>
struct ARaw {
    static constexpr int N = A_BF16 ? 1 : 2;
    u32x4 v[N];
};

template <bool A_BF16>
__device__ __forceinline__ ARaw<A_BF16> load_a8(const void* a, int s, int i0, int I)
{
    const size_t cpr16 = (size_t)(I / 16);
    const size_t o = (size_t)(i0 / 16);
    const u32x4* a16 = static_cast<const u32x4*>(a);
    ARaw<A_BF16> r;
    if constexpr (A_BF16) {
        r.v[0] = a16[((size_t)s * 2 + (size_t)((i0 / 8) % 2)) * cpr16 + o];
    } else {
        const size_t t = (size_t)((i0 / 4) % 4);  // 0 or 2
        r.v[0] = a16[((size_t)s * 4 + t) * cpr16 + o];
        r.v[1] = a16[((size_t)s * 4 + t + 1) * cpr16 + o];
    }
    return r;
}

// The B operand pieces of those 8 values: hi (and lo for float32 a).
template <bool A_BF16>
__device__ __forceinline__ void split_a8(const ARaw<A_BF16>& r, u32x4& hi, u32x4& lo)
{
    if constexpr (A_BF16) {
        hi = r.v[0];
        lo = u32x4{0u, 0u, 0u, 0u};
    } else {
        split8(__builtin_bit_cast(f32x4, r.v[0]), __builtin_bit_cast(f32x4, r.v[1]), hi, lo);
    }
}

// The lane's rows: row tile t of the wavefront is rows h0 + 16t .. +15, the
// lane supplying row h0 + 16t + col.
template <int RT>
struct DnRow {
    const uint8_t* q[RT];   // codes
    const uint8_t* s[RT];   // scales
    int nsteps;             // MX blocks per row (I/32) = MFMA K steps
    int kb;                 // lane / 16
    int col;                // lane % 16
};

struct DnGroupW {
    u32x4 c0, c1;           // codes of the lane's MX block in the group (c1: MXFP8 only)
    uint32_t sb;            // its UE8M0 scale byte, as loaded (turned into a float only when
                            // decoded: converting at the load would wait for it there)
};

template <bool FP4, int RT>
__device__ __forceinline__ void load_dn_w(const DnRow<RT>& r, int g, DnGroupW (&w)[RT])
{
    const int kbase = g * 128 + 32 * r.kb;
    const int bbase = FP4 ? kbase / 2 : kbase;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        w[t].c0 = *reinterpret_cast<const u32x4*>(r.q[t] + bbase);
        w[t].c1 = FP4 ? w[t].c0 : *reinterpret_cast<const u32x4*>(r.q[t] + bbase + 16);
        w[t].sb = r.s[t][4 * g + r.kb];
    }
}

// MFMA step q of the group: codes 8q .. 8q+7 of the lane's block.
template <bool FP4>
__device__ __forceinline__ bf16x8 dn_decode(const DnGroupW& w, int q)
{
    const float sc = ue8m0_to_f32(w.sb);
    if constexpr (FP4)
        return decode8_scaled_fp4(w.c0[q], sc);
    const u32x4 src = q < 2 ? w.c0 : w.c1;
    return decode8_scaled((q & 1) ? u32x2{src.z, src.w} : u32x2{src.x, src.y}, sc);
}

}  // namespace

// One pass over the rows for NTL tiles of 16 slots (tiles t0 .. t0+NTL-1).
// Every thread of the workgroup calls it (it has barriers); `store` is false
// for wavefronts whose rows lie past H (they compute on clamped rows and
// write nothing). Inside a K group lane (row, kb) supplies block kb's 32
// codes over the 4 MFMA steps and the B operand uses the same k order;
// leftover blocks (I/32 not a multiple of 4) take a from global memory in
// plain k order. Each B operand read from LDS serves the RT row tiles.
//
// Loads in flight: the weight codes and the slots' a of a group are both
// requested two groups ahead (two register sets each, used alternately, so
// the loop carries no register copies that would wait for them); a group's a
// is split into its LDS buffer after the previous group's MFMAs.
template <int NTL, int RT, bool A_BF16, bool FP4>
__device__ __forceinline__ void expert_down_pass(const DownArgs& p, const DnRow<RT>& r, const uint16_t* slots,
                                                 int count, int t0, u32x4* xs, bool store, int h0, float* y)
{
    const int I = p.I;
    const int tid = threadIdx.x;
    const int lcol = tid / 16;                    // cooperative load: slot column ...
    const int lc = tid % 16;                      // ... and 8-value piece of the group
    constexpr int kHalf = NTL * kDnUnits;         // lo tiles follow the hi tiles
    constexpr int kBuf = (A_BF16 ? 1 : 2) * kHalf;
    int ls[NTL];                                  // slot of this thread's load column, per tile
    int bj[NTL];                                  // slot of this lane's MFMA column, per tile
#pragma unroll
    for (int tt = 0; tt < NTL; ++tt) {
        const int sl = (t0 + tt) * 16 + lcol;
        ls[tt] = slots[sl < count ? sl : count - 1];
        const int si = (t0 + tt) * 16 + r.col;
        bj[tt] = slots[si < count ? si : count - 1];  // extra columns repeat a slot
    }
    f32x4 d[RT][NTL];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int tt = 0; tt < NTL; ++tt)
            d[t][tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int ngroups = r.nsteps / 4;
    ARaw<A_BF16> raw[2][NTL];                     // a of groups g+1 and g+2, by group parity
    auto load_a = [&](ARaw<A_BF16> (&dst)[NTL], int g) {
#pragma unroll
        for (int tt = 0; tt < NTL; ++tt)
            dst[tt] = load_a8<A_BF16>(p.a, ls[tt], g * 128 + 8 * lc, I);
    };
    auto put_a = [&](const ARaw<A_BF16> (&src)[NTL], u32x4* buf) {
#pragma unroll
        for (int tt = 0; tt < NTL; ++tt) {
            u32x4 hi, lo;
            split_a8<A_BF16>(src[tt], hi, lo);
            const int u = (tt * 16 + lcol) * 16 + (lc ^ lcol);
            buf[u] = hi;
            if constexpr (!A_BF16)
                buf[kHalf + u] = lo;
        }
    };
    DnGroupW wA[RT], wB[RT];
    if (ngroups > 0) {
        load_a(raw[0], 0);
        if (ngroups > 1)
            load_a(raw[1], 1);
        load_dn_w<FP4>(r, 0, wA);
        load_dn_w<FP4>(r, ngroups > 1 ? 1 : 0, wB);
        put_a(raw[0], xs);
    }
    __syncthreads();
    // group g (parity P): a of g+2 into set P, the MFMAs on buffer g&1, a of
    // g+1 (set 1-P) split into the other buffer
    auto group = [&](auto par, int g, DnGroupW (&w)[RT]) {
        constexpr int P = decltype(par)::value;
        const u32x4* xb = xs + (g & 1) * kBuf;
        // unconditional (the last two groups re-read the last one): a load
        // behind a branch makes the compiler wait for every load at the join,
        // the ones just issued two groups ahead included
        load_a(raw[P], g + 2 < ngroups ? g + 2 : ngroups - 1);
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 aw[RT][4];
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                aw[t][q] = dn_decode<FP4>(w[t], q);
        load_dn_w<FP4>(r, g + 2 < ngroups ? g + 2 : ngroups - 1, w);   // two groups ahead
        // the group's loads stay ahead of its other work (the split of the next
        // group's a would otherwise be hoisted above them, waiting for older loads first)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = 4 * r.kb + q;
#pragma unroll
            for (int tt = 0; tt < NTL; ++tt) {
                const int u = (tt * 16 + r.col) * 16 + (c ^ r.col);
                const bf16x8 bh = __builtin_bit_cast(bf16x8, xb[u]);
#pragma unroll
                for (int t = 0; t < RT; ++t)
                    d[t][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[t][q], bh, d[t][tt], 0, 0, 0);
                if constexpr (!A_BF16) {
                    const bf16x8 bl = __builtin_bit_cast(bf16x8, xb[kHalf + u]);
#pragma unroll
                    for (int t = 0; t < RT; ++t)
                        d[t][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[t][q], bl, d[t][tt], 0, 0, 0);
                }
            }
        }
        // (after the last group this fills the other buffer with a copy nobody reads)
        put_a(raw[1 - P], xs + ((g + 1) & 1) * kBuf);
        __syncthreads();                          // buffer g&1 read by all, buffer (g+1)&1 written
    };
    // pairs of groups with no branch inside the loop body, so the wait before
    // each group's decode covers exactly that group's weights and not the loads
    // in flight behind them
    for (int g = 0; g + 1 < ngroups; g += 2) {
        group(std::integral_constant<int, 0>{}, g, wA);
        group(std::integral_constant<int, 1>{}, g + 1, wB);
    }
    if (ngroups & 1)
        group(std::integral_constant<int, 0>{}, ngroups - 1, wA);
    for (int st = 4 * ngroups; st < r.nsteps; ++st) {   // leftover blocks: plain k order
        const int k0 = st * 32 + 8 * r.kb;
        bf16x8 aw[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            if constexpr (FP4)
                aw[t] = decode8_scaled_fp4(*reinterpret_cast<const uint32_t*>(r.q[t] + k0 / 2),
                                           ue8m0_to_f32(r.s[t][st]));
            else
                aw[t] = decode8_scaled(*reinterpret_cast<const u32x2*>(r.q[t] + k0), ue8m0_to_f32(r.s[t][st]));
        }
#pragma unroll
        for (int tt = 0; tt < NTL; ++tt) {
            u32x4 hi, lo;
            split_a8<A_BF16>(load_a8<A_BF16>(p.a, bj[tt], k0, I), hi, lo);
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                d[t][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[t], __builtin_bit_cast(bf16x8, hi), d[t][tt],
                                                                   0, 0, 0);
                if constexpr (!A_BF16)
                    d[t][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[t], __builtin_bit_cast(bf16x8, lo),
                                                                       d[t][tt], 0, 0, 0);
            }
        }
    }
    if (!store)
        return;
    // lane holds D rows 4*kb .. +3 (outputs h) of column col (slot) of each tile
#pragma unroll
    for (int tt = 0; tt < NTL; ++tt) {
        if ((t0 + tt) * 16 + r.col < count) {
            const int s = bj[tt];
            const float wgt = p.w[s];
#pragma unroll
            for (int t = 0; t < RT; ++t)
                *reinterpret_cast<f32x4*>(y + (size_t)s * (size_t)p.H + (size_t)(h0 + 16 * t + 4 * r.kb)) =
                    wgt * d[t][tt];
        }
    }
}

// Wide weight loads. The 128-byte row slices above (lane group kb of a 16-row
// tile reads 32 bytes of each row per group) keep the weight stream near
// 4.5 TB/s; runs of 256 bytes per row go faster (the same change in the
// grouped gate/up). The wavefront reads its 16*RT rows in steps of 256 bytes
// per row (two 128-code groups of MXFP8, four of MXFP4): load i of lane L
// takes the 16-byte piece L % 16 of row L / 16 + 4i, so each load instruction
// covers four whole 256-byte runs. A step goes through a wavefront-private LDS
// region of 16*RT rows x 16 pieces (piece b of row n at unit 16n + (b ^ (n % 16)),
// free of bank conflicts for the writes and the operand reads), and lane
// (col, kb) reads for group h of the step the pieces holding MX block 4h + kb
// of its rows: the codes load_dn_w gives it, so the results are the same floats.
template <bool FP4, int RT>
struct DnStep {
    static constexpr int kGroups = FP4 ? 4 : 2;  // 128-code groups per 256-byte step
    u32x4 v[4 * RT];                             // pieces of rows L/16 + 4i
};

// 16-byte LDS units of one step, per wavefront
template <int RT>
constexpr int kDnWideUnits = 16 * RT * 16;

// q0: the wavefront's first row (wave-uniform); lo: this lane's byte offset
// (lane/16)*rstride + 16*(lane%16); rs4 = 4*rstride. A uniform base plus 32-bit
// lane offsets keeps the addresses of the 4*RT loads in a few registers.
template <bool FP4, int RT>
__device__ __forceinline__ void load_dn_step(const uint8_t* q0, uint32_t lo, uint32_t rs4, int step,
                                             DnStep<FP4, RT>& w)
{
    const uint32_t base = lo + 256u * (uint32_t)step;
#pragma unroll
    for (int i = 0; i < 4 * RT; ++i)
        w.v[i] = *reinterpret_cast<const u32x4*>(q0 + (base + (uint32_t)i * rs4));
}

template <bool FP4, int RT>
__device__ __forceinline__ void stage_dn_step(const DnStep<FP4, RT>& w, u32x4* tb, int lane)
{
    const int b = lane % 16;
#pragma unroll
    for (int i = 0; i < 4 * RT; ++i) {
        const int n = lane / 16 + 4 * i;
        tb[n * 16 + (b ^ (n & 15))] = w.v[i];
    }
}

// Group h of the staged step, row tile t: the lane's codes of MX block 4h + kb.
template <bool FP4, int RT>
__device__ __forceinline__ DnGroupW staged_dn_group(const u32x4* tb, const DnRow<RT>& r, int h, int t,
                                                    uint32_t sb)
{
    const u32x4* row = tb + (16 * t + r.col) * 16;
    DnGroupW w;
    if constexpr (FP4) {                         // block 4h + kb = piece 4h + kb
        w.c0 = row[(4 * h + r.kb) ^ r.col];
        w.c1 = w.c0;
    } else {                                     // block 4h + kb = pieces 8h + 2kb, +1
        w.c0 = row[(8 * h + 2 * r.kb) ^ r.col];
        w.c1 = row[(8 * h + 2 * r.kb + 1) ^ r.col];
    }
    w.sb = sb;
    return w;
}

// expert_down_pass with the wide weight loads (I a multiple of 512: whole
// 256-byte steps and, for MXFP8, whole two-step scale blocks): one step of
// weights in flight ahead (requested once the group before the step's last two
// has taken its a loads), with it the next scale block (16 bytes per row, two
// lanes per row, handed out by ds_bpermute: see load_scale_block), the slots' a
// two groups ahead as before; each wait for a group's a therefore never waits
// for rows issued behind it. q0 / rstride: the wavefront's first row and its
// row stride (0 for a wavefront past H, which reads row H-1 throughout); sq0:
// the scale row of the lane's block-load row slot ((lane / 2) % (16*RT)); tb:
// the wavefront's LDS region.
//
// NH = 2 (float32 a): 2*NTL tiles in one pass over the rows, in two halves of
// NTL tiles that take turns in the two LDS buffers of NTL tiles: each K group
// is decoded once and multiplied with half 0's a (buffer 0), then, after a
// barrier, with half 1's a (buffer 1). The a of a half is requested one K
// group ahead (two half-groups ahead, as with NH = 1). So 2*NTL tiles of
// slots read the rows once, with the LDS of an NTL-tile pass; per output the
// MFMAs, their operands and their order are those of the NTL-tile passes, so
// the results are the same floats.
template <int NTL, int RT, bool A_BF16, bool FP4, int NH = 1>
__device__ __forceinline__ void expert_down_pass_wide(const DownArgs& p, const DnRow<RT>& r, const uint8_t* q0,
                                                      size_t rstride, const uint8_t* sq0, const uint16_t* slots, int count,
                                                      int t0, u32x4* xs, u32x4* tb, bool store, int h0, float* y)
{
    static_assert(NH == 1 || (NH == 2 && !A_BF16), "two halves only for float32 a");
    constexpr int GPS = DnStep<FP4, RT>::kGroups;
    constexpr int NT = NH * NTL;                  // tiles of the pass
    const int I = p.I;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int lcol = tid / 16;
    const int lc = tid % 16;
    constexpr int kHalf = NTL * kDnUnits;
    constexpr int kBuf = (A_BF16 ? 1 : 2) * kHalf;
    int ls[NT];
    int bj[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        const int sl = (t0 + tt) * 16 + lcol;
        ls[tt] = slots[sl < count ? sl : count - 1];
        const int si = (t0 + tt) * 16 + r.col;
        bj[tt] = slots[si < count ? si : count - 1];
    }
    f32x4 d[RT][NT];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
            d[t][tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int ngroups = r.nsteps / 4;
    const int nst = ngroups / GPS;                // 256-byte steps (even for MXFP8)
    const uint32_t lo = (uint32_t)(lane / 16) * (uint32_t)rstride + 16u * (uint32_t)(lane % 16);
    const uint32_t rs4 = 4u * (uint32_t)rstride;
    // NH = 1: a of groups g+1 and g+2, by group parity; NH = 2: a of half 0
    // and of half 1 (of the next K group, or of this one until it is in LDS)
    ARaw<A_BF16> raw[2][NTL];
    auto load_a = [&](ARaw<A_BF16> (&dst)[NTL], int g, int half) {
#pragma unroll
        for (int tt = 0; tt < NTL; ++tt)
            dst[tt] = load_a8<A_BF16>(p.a, ls[half * NTL + tt], g * 128 + 8 * lc, I);
    };
    auto put_a = [&](const ARaw<A_BF16> (&src)[NTL], u32x4* buf) {
#pragma unroll
        for (int tt = 0; tt < NTL; ++tt) {
            u32x4 hi, lo16;
            split_a8<A_BF16>(src[tt], hi, lo16);
            const int u = (tt * 16 + lcol) * 16 + (lc ^ lcol);
            buf[u] = hi;
            if constexpr (!A_BF16)
                buf[kHalf + u] = lo16;
        }
    };
    DnStep<FP4, RT> sw;
    if constexpr (NH == 1) {
        load_a(raw[0], 0, 0);
        load_a(raw[1], 1, 0);
    } else {
        load_a(raw[0], 0, 0);
        load_a(raw[1], 0, 1);
    }
    load_dn_step<FP4, RT>(q0, lo, rs4, 0, sw);
    u32x2 sb = load_scale_block(sq0, 0, lane);
    put_a(raw[0], xs);
    __syncthreads();
    // NH = 1: a of group g+2 into set P = g & 1; NH = 2: half 0's a of group
    // g+1 into set 0 (unconditional: the last groups re-read the last group's
    // a, so no load sits behind a branch)
    // (the scheduling barrier keeps the loads issued ahead of the group's other
    // work: the split of the next group's a would otherwise be hoisted above
    // them and wait for every older load first)
    auto aload = [&](auto par, int g) {
        constexpr int P = decltype(par)::value;
        if constexpr (NH == 1)
            load_a(raw[P], g + 2 < ngroups ? g + 2 : ngroups - 1, 0);
        else
            load_a(raw[0], g + 1 < ngroups ? g + 1 : ngroups - 1, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    // the MFMAs of the decoded group on one LDS buffer, into tiles T0 .. T0+NTL-1
    auto mfmas = [&](auto tfirst, const bf16x8 (&aw)[RT][4], const u32x4* xb) {
        constexpr int T0 = decltype(tfirst)::value;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = 4 * r.kb + q;
#pragma unroll
            for (int tt = 0; tt < NTL; ++tt) {
                const int u = (tt * 16 + r.col) * 16 + (c ^ r.col);
                const bf16x8 bh = __builtin_bit_cast(bf16x8, xb[u]);
#pragma unroll
                for (int t = 0; t < RT; ++t)
                    d[t][T0 + tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[t][q], bh, d[t][T0 + tt], 0, 0, 0);
                if constexpr (!A_BF16) {
                    const bf16x8 bl = __builtin_bit_cast(bf16x8, xb[kHalf + u]);
#pragma unroll
                    for (int t = 0; t < RT; ++t)
                        d[t][T0 + tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[t][q], bl, d[t][T0 + tt], 0, 0, 0);
                }
            }
        }
    };
    // group g = step group h with the scale codes of the lane's RT rows. NH = 1:
    // the MFMAs on buffer g&1, then a of g+1 (set 1-P) split into the other
    // buffer. NH = 2: half 0 on buffer 0, half 1's a (set 1) into buffer 1; then
    // half 1's a of group g+1 requested and half 1 on buffer 1, half 0's a of
    // group g+1 (set 0) into buffer 0.
    auto decode = [&](int h, const uint32_t (&codes)[RT], bf16x8 (&aw)[RT][4]) {
        DnGroupW w[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t)
            w[t] = staged_dn_group<FP4, RT>(tb, r, h, t, codes[t]);
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                aw[t][q] = dn_decode<FP4>(w[t], q);
    };
    auto group = [&](auto par, int g, int h, const uint32_t (&codes)[RT]) {
        constexpr int P = decltype(par)::value;
        bf16x8 aw[RT][4];
        decode(h, codes, aw);
        if constexpr (NH == 1) {
            mfmas(std::integral_constant<int, 0>{}, aw, xs + (g & 1) * kBuf);
            put_a(raw[1 - P], xs + ((g + 1) & 1) * kBuf);
            __syncthreads();                      // buffer g&1 read by all, buffer (g+1)&1 written
        } else {
            mfmas(std::integral_constant<int, 0>{}, aw, xs);
            put_a(raw[1], xs + kBuf);
            __syncthreads();                      // buffer 0 read by all, buffer 1 written
            load_a(raw[1], g + 1 < ngroups ? g + 1 : ngroups - 1, 1);
            __builtin_amdgcn_sched_barrier(0);
            // decoded again from the staged step rather than held across the
            // barrier (the registers are the scarce part)
            bf16x8 aw1[RT][4];
            decode(h, codes, aw1);
            mfmas(std::integral_constant<int, NTL>{}, aw1, xs + kBuf);
            put_a(raw[0], xs);
            __syncthreads();                      // buffer 1 read by all, buffer 0 written
        }
    };
    constexpr auto P0 = std::integral_constant<int, 0>{};
    constexpr auto P1 = std::integral_constant<int, 1>{};
    if constexpr (GPS == 2) {
        // MXFP8: steps in pairs (one scale block); the next step (and, in the
        // second step, the next block) requested during each step's first group
        for (int s = 0; s < nst; s += 2) {
            const int g0 = 2 * s;
            // each step's scale codes at the step start (sb is refilled in the
            // second step, after its codes are taken)
            uint32_t c0[RT], c1[RT];
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                c0[t] = block_scale_code<0>(sb, 16 * t + r.col, r.kb);
                c1[t] = block_scale_code<1>(sb, 16 * t + r.col, r.kb);
            }
            stage_dn_step<FP4, RT>(sw, tb, lane);
            aload(P0, g0);
            load_dn_step<FP4, RT>(q0, lo, rs4, s + 1, sw);
            __builtin_amdgcn_sched_barrier(0);
            group(P0, g0, 0, c0);
            aload(P1, g0 + 1);
            group(P1, g0 + 1, 1, c1);
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                c0[t] = block_scale_code<2>(sb, 16 * t + r.col, r.kb);
                c1[t] = block_scale_code<3>(sb, 16 * t + r.col, r.kb);
            }
            stage_dn_step<FP4, RT>(sw, tb, lane);
            const int sn = s + 2 < nst ? s + 2 : s + 1;
            aload(P0, g0 + 2);
            load_dn_step<FP4, RT>(q0, lo, rs4, sn, sw);
            sb = load_scale_block(sq0, sn / 2, lane);
            __builtin_amdgcn_sched_barrier(0);
            group(P0, g0 + 2, 0, c0);
            aload(P1, g0 + 3);
            group(P1, g0 + 3, 1, c1);
        }
    } else {
        // MXFP4: one scale block per step; the next step and block requested
        // during the step's third group
        for (int s = 0; s < nst; ++s) {
            const int g0 = 4 * s;
            // all four groups' scale codes at the step start (per group, a
            // ds_bpermute round trip would sit before each decode)
            uint32_t sc[4][RT];
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                sc[0][t] = block_scale_code<0>(sb, 16 * t + r.col, r.kb);
                sc[1][t] = block_scale_code<1>(sb, 16 * t + r.col, r.kb);
                sc[2][t] = block_scale_code<2>(sb, 16 * t + r.col, r.kb);
                sc[3][t] = block_scale_code<3>(sb, 16 * t + r.col, r.kb);
            }
            stage_dn_step<FP4, RT>(sw, tb, lane);
            const int sn = s + 1 < nst ? s + 1 : s;
            aload(P0, g0);
            group(P0, g0, 0, sc[0]);
            aload(P1, g0 + 1);
            group(P1, g0 + 1, 1, sc[1]);
            aload(P0, g0 + 2);
            load_dn_step<FP4, RT>(q0, lo, rs4, sn, sw);
            sb = load_scale_block(sq0, sn, lane);
            __builtin_amdgcn_sched_barrier(0);
            group(P0, g0 + 2, 2, sc[2]);
            aload(P1, g0 + 3);
            group(P1, g0 + 3, 3, sc[3]);
        }
    }
    if (!store)
        return;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        if ((t0 + tt) * 16 + r.col < count) {
            const int s = bj[tt];
            const float wgt = p.w[s];
#pragma unroll
            for (int t = 0; t < RT; ++t)
                *reinterpret_cast<f32x4*>(y + (size_t)s * (size_t)p.H + (size_t)(h0 + 16 * t + 4 * r.kb)) =
                    wgt * d[t][tt];
        }
    }
}

// An item is (expert e, RT*64 rows); wavefront w takes the rows
// hb + 16*RT*w .. +16*RT-1. H is a multiple of 16*RT. wl_off >= 0: the work
// list sits wl_off ints into the dynamic LDS and the workgroups walk the
// items of the routed experts with a stride of the grid size; wl_off < 0: one
// item per workgroup over all E experts (the grid is E * blocks).
template <int RT, bool A_BF16, bool FP4, bool WIDE>
__device__ __forceinline__ void expert_down_item(const DownArgs& p, float* y, int max_tiles, int e, int hb,
                                                 int count, const uint16_t* slots, u32x4* xs)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int h0 = hb + 16 * RT * w;              // this wavefront's rows
    const bool store = h0 < p.H;                  // wavefronts past H still take part in the barriers
    const int col = lane % 16;
    const size_t row_bytes = FP4 ? (size_t)(p.I / 2) : (size_t)p.I;
    DnRow<RT> r;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int hr = h0 + 16 * t + col < p.H ? h0 + 16 * t + col : p.H - 1;
        const size_t row = (size_t)e * (size_t)p.H + (size_t)hr;
        r.q[t] = p.wd_q + row * row_bytes;
        r.s[t] = p.wd_s + row * (size_t)(p.I / 32);
    }
    r.nsteps = p.I / 32;
    r.kb = lane / 16;
    r.col = col;
    const int ntiles = (count + 15) / 16;
    if constexpr (WIDE) {
        // the wavefront's first row (all rows clamped to H-1 past H), its row
        // stride, and its LDS region after the a tiles
        const int wrow = __builtin_amdgcn_readfirstlane(store ? h0 : p.H - 1);   // wave-uniform
        const uint8_t* q0 = p.wd_q + ((size_t)e * (size_t)p.H + (size_t)wrow) * row_bytes;
        const size_t rstride = store ? row_bytes : 0;
        // the lane's scale row for the block loads: row slot (lane / 2) % (16*RT)
        const int srow = store ? h0 + (lane / 2) % (16 * RT) : p.H - 1;
        const uint8_t* sq0 = p.wd_s + ((size_t)e * (size_t)p.H + (size_t)srow) * (size_t)(p.I / 32);
        u32x4* tb = xs + 2 * (A_BF16 ? 1 : 2) * max_tiles * kDnUnits + w * kDnWideUnits<RT>;
        // at most 2 tiles of float32 a (3 of bf16) per pass here: the step
        // registers take the place of the last tile's (the launcher sizes the
        // LDS for the same)
        constexpr int kCap = A_BF16 ? 3 : 2;
        const int mt = max_tiles < kCap ? max_tiles : kCap;
        int t0 = 0;
        if constexpr (!A_BF16) {
            // float32 a, more than 2 tiles: 4 per pass over the rows in two
            // halves of 2 (the last may be partly empty), then the rest
            if (mt == 2 && p.split != 0) {
                for (; ntiles - t0 > 2; t0 += 4)
                    expert_down_pass_wide<2, RT, A_BF16, FP4, 2>(p, r, q0, rstride, sq0, slots, count, t0, xs, tb,
                                                                 store, h0, y);
            }
        }
        for (; t0 < ntiles; t0 += mt) {
            const int nt = ntiles - t0 < mt ? ntiles - t0 : mt;
            if (nt == 1) {
                expert_down_pass_wide<1, RT, A_BF16, FP4>(p, r, q0, rstride, sq0, slots, count, t0, xs, tb, store, h0, y);
            } else if (nt == 2) {
                expert_down_pass_wide<2, RT, A_BF16, FP4>(p, r, q0, rstride, sq0, slots, count, t0, xs, tb, store, h0, y);
            } else if constexpr (A_BF16) {
                expert_down_pass_wide<3, RT, A_BF16, FP4>(p, r, q0, rstride, sq0, slots, count, t0, xs, tb, store, h0, y);
            }
        }
        return;
    }
    for (int t0 = 0; t0 < ntiles; t0 += max_tiles) {
        const int nt = ntiles - t0 < max_tiles ? ntiles - t0 : max_tiles;
        switch (nt) {
        case 1: expert_down_pass<1, RT, A_BF16, FP4>(p, r, slots, count, t0, xs, store, h0, y); break;
        case 2: expert_down_pass<2, RT, A_BF16, FP4>(p, r, slots, count, t0, xs, store, h0, y); break;
        case 3: expert_down_pass<3, RT, A_BF16, FP4>(p, r, slots, count, t0, xs, store, h0, y); break;
        default:                                  // 4 tiles of float32 a do not fit in 64 KiB of LDS
            if constexpr (A_BF16)
                expert_down_pass<4, RT, A_BF16, FP4>(p, r, slots, count, t0, xs, store, h0, y);
            break;
        }
    }
}

// WIN: B*k > kSlotCap, the slots of an expert taken in windows of kSlotCap
template <int RT, bool A_BF16, bool FP4, bool WIDE, bool WIN>
__global__ void __launch_bounds__(kGroupWaves * kWave) __attribute__((amdgpu_waves_per_eu(4 - RT)))
moe_down_expert_kernel(DownArgs p, float* y, int max_tiles, int wl_off)
{
    // up to kSlotCap slot entries of 16 bits (B*k < 65536; a list of fixed
    // size keeps two tiles of a per pass at any batch), the a tiles, then the
    // work list
    extern __shared__ int smem[];
    uint16_t* slots = reinterpret_cast<uint16_t*>(smem);
    __shared__ int wave_cnt[kGroupWaves];
    constexpr int kRows = 16 * RT * kGroupWaves;
    const int nblk = (p.H + kRows - 1) / kRows;
    const int nslots = p.B * p.k;
    const int cap = nslots < kSlotCap ? nslots : kSlotCap;
    u32x4* xs = reinterpret_cast<u32x4*>(slots + ((cap + 7) & ~7));
    const int* act = nullptr;
    if constexpr (WIN) {
        // items (expert, row block, window of kSlotCap slots)
        int nwin = (nslots + kSlotCap - 1) / kSlotCap;   // without the work list: as many as B*k could need
        int n_items;
        if (wl_off >= 0) {
            int* mark = smem + wl_off;
            int* list = mark + p.E;
            n_items = routed_experts_windows(nslots, p.ids, p.E, mark, list, wave_cnt, nwin) * nblk * nwin;
            act = list;
        } else {
            n_items = p.E * nblk * nwin;
        }
        const int ipe = nblk * nwin;
        for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
            const int e = act ? act[item / ipe] : item / ipe;
            const int hb = ((item % ipe) / nwin) * kRows;
            const int lo = (item % nwin) * kSlotCap;
            auto mine = [&](int v) { return v == e; };
            const int count = compact_slots<kGroupWaves, decltype(mine), uint16_t, true>(nslots, p.ids, slots,
                                                                                         wave_cnt, mine, lo, kSlotCap);
            if (count <= lo)
                continue;                         // whole workgroup (no slots in this window)
            expert_down_item<RT, A_BF16, FP4, WIDE>(p, y, max_tiles, e, hb,
                                                    count - lo < kSlotCap ? count - lo : kSlotCap, slots, xs);
            __syncthreads();                      // the next item rewrites the slot list and the a tiles
        }
    } else {
        // B*k <= kSlotCap: items (expert, row block), every slot in one list
        int n_items = p.E * nblk;
        if (wl_off >= 0) {
            int* mark = smem + wl_off;
            int* list = mark + p.E;
            n_items = routed_experts(nslots, p.ids, p.E, mark, list, wave_cnt) * nblk;
            act = list;
        }
        for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
            const int e = act ? act[item / nblk] : item / nblk;
            const int hb = (item % nblk) * kRows;
            const int count = compact_slots(nslots, p.ids, slots, wave_cnt, [&](int v) { return v == e; });
            if (count == 0)
                continue;                         // whole workgroup (only without the work list)
            expert_down_item<RT, A_BF16, FP4, WIDE>(p, y, max_tiles, e, hb, count, slots, xs);
            __syncthreads();                      // the next item rewrites the slot list and the a tiles
        }
    }
}

// Four consecutive outputs per thread (H is a multiple of 4).
template <bool OUT_BF16>
__global__ void __launch_bounds__(256)
moe_down_combine_kernel(const float* y, const int32_t* ids, int B, int E, int k, int H, void* out)
{
    const long q = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const int hq = H / 4;
    if (q >= (long)B * hq)
        return;
    const int b = (int)(q / hq);
    const int h = (int)(q % hq) * 4;
    // ids first, then every partial unconditionally (in bounds; the partial of a
    // slot with an invalid id was never written and is masked below), so the k
    // loads are all in flight at once; added in slot order
    const int32_t* idb = ids + (size_t)b * (size_t)k;
    bool bad = false;
    for (int j = 0; j < k; ++j)
        bad |= (unsigned)idb[j] >= (unsigned)E;
    const float* yb = y + (size_t)b * (size_t)k * (size_t)H + (size_t)h;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
    for (int j = 0; j < k; ++j)
        acc += *reinterpret_cast<const f32x4*>(yb + (size_t)j * (size_t)H);
    if (bad)
        acc = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    const size_t o = (size_t)b * (size_t)H + (size_t)h;
    // one vector store when out is aligned for it (the usual case), else four
    // element stores: the caller's out needs no alignment beyond its type
    if constexpr (OUT_BF16) {
        uint16_t* ob = static_cast<uint16_t*>(out) + o;
        const uint32_t lo = f32x2_to_bf16x2_rne(acc.x, acc.y);
        const uint32_t hi = f32x2_to_bf16x2_rne(acc.z, acc.w);
        if (((uintptr_t)out & 7u) == 0) {
            *reinterpret_cast<u32x2*>(ob) = u32x2{lo, hi};
        } else {
            ob[0] = (uint16_t)(lo & 0xFFFFu);
            ob[1] = (uint16_t)(lo >> 16);
            ob[2] = (uint16_t)(hi & 0xFFFFu);
            ob[3] = (uint16_t)(hi >> 16);
        }
    } else {
        float* of = static_cast<float*>(out) + o;
        if (((uintptr_t)out & 15u) == 0) {
            *reinterpret_cast<f32x4*>(of) = acc;
        } else {
            of[0] = acc.x;
            of[1] = acc.y;
            of[2] = acc.z;
            of[3] = acc.w;
        }
    }
}

size_t down_grouped_lds(int B, int k, int E, bool a_bf16, int max_tiles, int row_tiles, bool wide)
{
    // slot list (at most kSlotCap 16-bit entries, rounded up to 16 bytes), two
    // buffers of hi (and lo) tiles, with the wide loads one step region per
    // wavefront, then the work list
    const long nslots = (long)B * (long)k;
    const size_t list = (size_t)((nslots < kSlotCap ? nslots : kSlotCap) + 7) / 8 * 16;
    const size_t stage = wide ? (size_t)kGroupWaves * 16 * (size_t)row_tiles * 16 * sizeof(u32x4) : 0;
    return list + 2 * (a_bf16 ? 1 : 2) * (size_t)max_tiles * kDnUnits * sizeof(u32x4) + stage + worklist_lds(E);
}

// Dynamic LDS limits: without the wide loads the default 64 KiB; with them up
// to 96 KiB may be requested, and the automatic choice keeps two workgroups
// per CU (80 KiB each).
constexpr size_t kDnLdsMax = 65536;
constexpr size_t kDnLdsMaxWide = 98304;
constexpr size_t kDnLdsAutoWide = 81920;

int down_grouped_tiles(int B, int k, int E, bool a_bf16, int requested, int row_tiles, bool wide)
{
    if ((long)B * (long)k > 65535)
        return 0;                                 // the slot list holds 16-bit slot indices
    const int cap = wide ? (a_bf16 ? 3 : 2) : kTiles;   // wide loads: 2 tiles of float32 a, 3 of bf16
    if (requested > 0) {
        const int mt = requested < cap ? requested : cap;
        return down_grouped_lds(B, k, E, a_bf16, mt, row_tiles, wide) <= (wide ? kDnLdsMaxWide : kDnLdsMax) ? mt : 0;
    }
    for (int mt = cap; mt >= 1; --mt)
        if (down_grouped_lds(B, k, E, a_bf16, mt, row_tiles, wide) <= (wide ? kDnLdsAutoWide : kDnLdsMax))
            return mt;
    return 0;
}

template <int RT, bool A, bool F, bool W, bool WIN>
hipError_t launch_expert_win(dim3 grid, dim3 block, size_t lds, hipStream_t s, const DownArgs& p, float* y,
                             int max_tiles, int wl_off)
{
    if constexpr (W) {
        // allow dynamic LDS beyond the default 64 KiB, once per device
        const hipError_t attr = set_max_dynamic_lds(
            reinterpret_cast<const void*>(&moe_down_expert_kernel<RT, A, F, W, WIN>), (int)kDnLdsMaxWide);
        if (attr != hipSuccess)
            return attr;
    }
    hipLaunchKernelGGL((moe_down_expert_kernel<RT, A, F, W, WIN>), grid, block, lds, s, p, y, max_tiles, wl_off);
    return hipGetLastError();
}

template <int RT, bool A, bool F, bool W>
hipError_t launch_expert(dim3 grid, dim3 block, size_t lds, hipStream_t s, const DownArgs& p, float* y,
                         int max_tiles, int wl_off)
{
    return (long)p.B * p.k > kSlotCap ? launch_expert_win<RT, A, F, W, true>(grid, block, lds, s, p, y, max_tiles, wl_off)
                                      : launch_expert_win<RT, A, F, W, false>(grid, block, lds, s, p, y, max_tiles, wl_off);
}

hipError_t launch_down_grouped(const DownArgs& p, bool a_bf16, bool out_bf16, float* y, int max_tiles,
                               int row_tiles, bool wide, int grid_cap, hipStream_t s)
{
    if ((long)p.B * p.k == 0)
        return hipSuccess;
    if (max_tiles < 1 || max_tiles > (a_bf16 ? kTiles : 3) || (row_tiles != 1 && row_tiles != 2) ||
        (p.H % (16 * row_tiles)) != 0)
        return hipErrorInvalidValue;
    const int nblk = (p.H + 16 * row_tiles * kGroupWaves - 1) / (16 * row_tiles * kGroupWaves);
    const long items = (long)p.E * nblk * (((long)p.B * p.k + kSlotCap - 1) / kSlotCap);   // x windows of slots
    const size_t lds = down_grouped_lds(p.B, p.k, p.E, a_bf16, max_tiles, row_tiles, wide);
    if (lds > (wide ? kDnLdsMaxWide : kDnLdsMax))
        return hipErrorInvalidValue;
    const size_t wl = worklist_lds(p.E);
    // with the work list: at most grid_cap workgroups walk the routed experts' items
    const bool use_wl = wl > 0 && grid_cap > 0;
    const int wl_off = use_wl ? (int)((lds - wl) / sizeof(int)) : -1;
    const dim3 grid((unsigned)(use_wl && items > grid_cap ? grid_cap : items)), block(kGroupWaves * kWave);
    const bool fp4 = p.wfmt == kMXFP4;
    hipError_t err;
#define MOED_DX(RT, W)                                                                                   \
    err = fp4 ? (a_bf16 ? launch_expert<RT, true, true, W>(grid, block, lds, s, p, y, max_tiles, wl_off)  \
                        : launch_expert<RT, false, true, W>(grid, block, lds, s, p, y, max_tiles, wl_off)) \
              : (a_bf16 ? launch_expert<RT, true, false, W>(grid, block, lds, s, p, y, max_tiles, wl_off) \
                        : launch_expert<RT, false, false, W>(grid, block, lds, s, p, y, max_tiles, wl_off))
    if (row_tiles == 2) {
        if (wide) MOED_DX(2, true); else MOED_DX(2, false);
    } else {
        if (wide) MOED_DX(1, true); else MOED_DX(1, false);
    }
#undef MOED_DX
    if (err != hipSuccess)
        return err;
    const long n = (long)p.B * (p.H / 4);
    const dim3 g2((unsigned)((n + 255) / 256)), b2(256);
    if (out_bf16)
        hipLaunchKernelGGL((moe_down_combine_kernel<true>), g2, b2, 0, s, y, p.ids, p.B, p.E, p.k, p.H, p.out);
    else
        hipLaunchKernelGGL((moe_down_combine_kernel<false>), g2, b2, 0, s, y, p.ids, p.B, p.E, p.k, p.H, p.out);
    return hipGetLastError();
}

}  // namespace moed
