// Down for large decode batches (tokens sharing experts): expert-major, so
// each routed down row is read and decoded once per workgroup pass (up to 64
// slots) instead of once per (token, slot).
//
// Step 1, moe_down_expert_kernel: a workgroup owns (expert e, 64 output rows
// hb .. hb+63), four wavefronts of 16 rows each. It compacts the list of slots
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
// K is walked in groups of 4 MX blocks, the next group's loads issued before
// the current group's MFMAs.
//
// Step 2, moe_down_combine_kernel: out[b][h] = sum over j of y[(b, j)][h], the
// token's k slots added in slot order and stored once; a token with an
// expert id outside [0, E) gets NaN.
//
// The per-slot partials are the price of reading each routed row once: they
// take B*k*H*4 bytes of workspace and a second, small HBM-bound launch.
#include "grouped_common.h"

namespace moed {

namespace {

constexpr int kDnUnits = 16 * 16;                // 16-byte units per tile and K group (one of hi / lo)

// 8 float32 values -> 8 bf16 hi and 8 bf16 lo (hi + lo = v to about 2^-17 relative).
__device__ __forceinline__ void split8(const f32x4& v0, const f32x4& v1, u32x4& hi, u32x4& lo)
{
    const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t h[8], l[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        h[t] = f32_to_bf16_rne(v[t]);
        l[t] = f32_to_bf16_rne(v[t] - __uint_as_float(h[t] << 16));
    }
    hi = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    lo = u32x4{l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16)};
}

// a[s][i0 .. i0+7] (i0 a multiple of 8) from the chunk-interleaved
// intermediate, as hi / lo bf16 (a bf16 intermediate: hi only).
template <bool A_BF16>
__device__ __forceinline__ void load_a8_split(const void* a, int s, int i0, int I, u32x4& hi, u32x4& lo)
{
    const size_t cpr16 = (size_t)(I / 16);
    const size_t o = (size_t)(i0 / 16);
    if constexpr (A_BF16) {
        const u32x4* a16 = static_cast<const u32x4*>(a);
        hi = a16[((size_t)s * 2 + (size_t)((i0 / 8) % 2)) * cpr16 + o];
        lo = u32x4{0u, 0u, 0u, 0u};
    } else {
        const f32x4* a32 = static_cast<const f32x4*>(a);
        const size_t t = (size_t)((i0 / 4) % 4);  // 0 or 2
        const f32x4 v0 = a32[((size_t)s * 4 + t) * cpr16 + o];
        const f32x4 v1 = a32[((size_t)s * 4 + t + 1) * cpr16 + o];
        split8(v0, v1, hi, lo);
    }
}

struct DnRow {
    const uint8_t* q;       // this lane's down row (codes)
    const uint8_t* s;       // its scales
    int nsteps;             // MX blocks per row (I/32) = MFMA K steps
    int kb;                 // lane / 16
    int col;                // lane % 16
};

struct DnGroupW {
    u32x4 c0, c1;           // codes of the lane's MX block in the group (c1: MXFP8 only)
    float sc;
};

template <bool FP4>
__device__ __forceinline__ DnGroupW load_dn_w(const DnRow& r, int g)
{
    DnGroupW w;
    const int kbase = g * 128 + 32 * r.kb;
    const int bbase = FP4 ? kbase / 2 : kbase;
    w.c0 = *reinterpret_cast<const u32x4*>(r.q + bbase);
    w.c1 = FP4 ? w.c0 : *reinterpret_cast<const u32x4*>(r.q + bbase + 16);
    w.sc = ue8m0_to_f32(r.s[4 * g + r.kb]);
    return w;
}

// MFMA step q of the group: codes 8q .. 8q+7 of the lane's block.
template <bool FP4>
__device__ __forceinline__ bf16x8 dn_decode(const DnGroupW& w, int q)
{
    if constexpr (FP4)
        return decode8_scaled_fp4(w.c0[q], w.sc);
    const u32x4 src = q < 2 ? w.c0 : w.c1;
    return decode8_scaled((q & 1) ? u32x2{src.z, src.w} : u32x2{src.x, src.y}, w.sc);
}

}  // namespace

// One pass over the rows for NTL tiles of 16 slots (tiles t0 .. t0+NTL-1).
// Every thread of the workgroup calls it (it has barriers); `store` is false
// for wavefronts whose rows lie past H (they compute on a clamped row and
// write nothing). Inside a K group lane (row, kb) supplies block kb's 32
// codes over the 4 MFMA steps and the B operand uses the same k order;
// leftover blocks (I/32 not a multiple of 4) take a from global memory in
// plain k order.
template <int NTL, bool A_BF16, bool FP4>
__device__ __forceinline__ void expert_down_pass(const DownArgs& p, const DnRow& r, const int* slots, int count,
                                                 int t0, u32x4* xs, bool store, int h0, float* y)
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
    f32x4 d[NTL];
#pragma unroll
    for (int tt = 0; tt < NTL; ++tt)
        d[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int ngroups = r.nsteps / 4;
    u32x4 hreg[NTL], lreg[NTL];
    DnGroupW wc{};
    if (ngroups > 0) {
#pragma unroll
        for (int tt = 0; tt < NTL; ++tt)
            load_a8_split<A_BF16>(p.a, ls[tt], 8 * lc, I, hreg[tt], lreg[tt]);
        wc = load_dn_w<FP4>(r, 0);
#pragma unroll
        for (int tt = 0; tt < NTL; ++tt) {
            const int u = (tt * 16 + lcol) * 16 + (lc ^ lcol);
            xs[u] = hreg[tt];
            if constexpr (!A_BF16)
                xs[kHalf + u] = lreg[tt];
        }
    }
    __syncthreads();
    for (int g = 0; g < ngroups; ++g) {
        const u32x4* xb = xs + (g & 1) * kBuf;
        const bool more = g + 1 < ngroups;
        DnGroupW wn = wc;
        if (more) {                               // next group's loads, ahead of this group's MFMAs
#pragma unroll
            for (int tt = 0; tt < NTL; ++tt)
                load_a8_split<A_BF16>(p.a, ls[tt], (g + 1) * 128 + 8 * lc, I, hreg[tt], lreg[tt]);
            wn = load_dn_w<FP4>(r, g + 1);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bf16x8 aw = dn_decode<FP4>(wc, q);
            const int c = 4 * r.kb + q;
#pragma unroll
            for (int tt = 0; tt < NTL; ++tt) {
                const int u = (tt * 16 + r.col) * 16 + (c ^ r.col);
                d[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, __builtin_bit_cast(bf16x8, xb[u]), d[tt], 0, 0,
                                                                0);
                if constexpr (!A_BF16)
                    d[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        aw, __builtin_bit_cast(bf16x8, xb[kHalf + u]), d[tt], 0, 0, 0);
            }
        }
        if (more) {
            u32x4* xn = xs + ((g + 1) & 1) * kBuf;
#pragma unroll
            for (int tt = 0; tt < NTL; ++tt) {
                const int u = (tt * 16 + lcol) * 16 + (lc ^ lcol);
                xn[u] = hreg[tt];
                if constexpr (!A_BF16)
                    xn[kHalf + u] = lreg[tt];
            }
        }
        __syncthreads();                          // buffer g&1 read by all, buffer (g+1)&1 written
        wc = wn;
    }
    for (int st = 4 * ngroups; st < r.nsteps; ++st) {   // leftover blocks: plain k order
        const int k0 = st * 32 + 8 * r.kb;
        bf16x8 aw;
        if constexpr (FP4)
            aw = decode8_scaled_fp4(*reinterpret_cast<const uint32_t*>(r.q + k0 / 2), ue8m0_to_f32(r.s[st]));
        else
            aw = decode8_scaled(*reinterpret_cast<const u32x2*>(r.q + k0), ue8m0_to_f32(r.s[st]));
#pragma unroll
        for (int tt = 0; tt < NTL; ++tt) {
            u32x4 hi, lo;
            load_a8_split<A_BF16>(p.a, bj[tt], k0, I, hi, lo);
            d[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, __builtin_bit_cast(bf16x8, hi), d[tt], 0, 0, 0);
            if constexpr (!A_BF16)
                d[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, __builtin_bit_cast(bf16x8, lo), d[tt], 0, 0, 0);
        }
    }
    if (!store)
        return;
    // lane holds D rows 4*kb .. +3 (outputs h, H a multiple of 16) of column col (slot)
#pragma unroll
    for (int tt = 0; tt < NTL; ++tt) {
        if ((t0 + tt) * 16 + r.col < count) {
            const int s = bj[tt];
            const float wgt = p.w[s];
            *reinterpret_cast<f32x4*>(y + (size_t)s * (size_t)p.H + (size_t)(h0 + 4 * r.kb)) = wgt * d[tt];
        }
    }
}

template <bool A_BF16, bool FP4>
__global__ void __launch_bounds__(kGroupWaves * kWave)
moe_down_expert_kernel(DownArgs p, float* y, int max_tiles)
{
    extern __shared__ int slots[];                // B*k entries, then the a tiles
    __shared__ int wave_cnt[kGroupWaves];
    const int nblk = (p.H + kGroupNeurons - 1) / kGroupNeurons;
    const int e = blockIdx.x / nblk;
    const int hb = (blockIdx.x % nblk) * kGroupNeurons;
    const int nslots = p.B * p.k;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int* ids = p.ids;
    const int count = compact_slots(nslots, slots, wave_cnt, [&](int t) { return ids[t] == e; });
    if (count == 0)
        return;                                   // whole workgroup: no barrier follows
    u32x4* xs = reinterpret_cast<u32x4*>(slots + ((nslots + 3) & ~3));
    const int h0 = hb + 16 * w;                   // this wavefront's 16 rows
    const bool store = h0 < p.H;                  // wavefronts past H still take part in the barriers
    const int col = lane % 16;
    const int hr = h0 + col < p.H ? h0 + col : p.H - 1;
    const size_t row = (size_t)e * (size_t)p.H + (size_t)hr;
    const size_t row_bytes = FP4 ? (size_t)(p.I / 2) : (size_t)p.I;
    const DnRow r{p.wd_q + row * row_bytes, p.wd_s + row * (size_t)(p.I / 32), p.I / 32, lane / 16, col};
    const int ntiles = (count + 15) / 16;
    for (int t0 = 0; t0 < ntiles; t0 += max_tiles) {
        const int nt = ntiles - t0 < max_tiles ? ntiles - t0 : max_tiles;
        switch (nt) {
        case 1: expert_down_pass<1, A_BF16, FP4>(p, r, slots, count, t0, xs, store, h0, y); break;
        case 2: expert_down_pass<2, A_BF16, FP4>(p, r, slots, count, t0, xs, store, h0, y); break;
        case 3: expert_down_pass<3, A_BF16, FP4>(p, r, slots, count, t0, xs, store, h0, y); break;
        default: expert_down_pass<4, A_BF16, FP4>(p, r, slots, count, t0, xs, store, h0, y); break;
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
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    bool bad = false;
    for (int j = 0; j < k; ++j) {
        const size_t s = (size_t)b * (size_t)k + (size_t)j;
        if ((unsigned)ids[s] >= (unsigned)E)
            bad = true;
        else
            acc += *reinterpret_cast<const f32x4*>(y + s * (size_t)H + (size_t)h);
    }
    if (bad)
        acc = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    const size_t o = (size_t)b * (size_t)H + (size_t)h;
    if constexpr (OUT_BF16) {
        const uint32_t lo = f32_to_bf16_rne(acc.x) | ((uint32_t)f32_to_bf16_rne(acc.y) << 16);
        const uint32_t hi = f32_to_bf16_rne(acc.z) | ((uint32_t)f32_to_bf16_rne(acc.w) << 16);
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + o) = u32x2{lo, hi};
    } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + o) = acc;
    }
}

size_t down_grouped_lds(int B, int k, bool a_bf16, int max_tiles)
{
    // slot list (rounded up to 16 bytes), then two buffers of hi (and lo) tiles
    const size_t list = ((size_t)B * (size_t)k + 3) / 4 * 16;
    return list + 2 * (a_bf16 ? 1 : 2) * (size_t)max_tiles * kDnUnits * sizeof(u32x4);
}

int down_grouped_tiles(int B, int k, bool a_bf16, int requested)
{
    if (requested > 0)
        return down_grouped_lds(B, k, a_bf16, requested) <= 65536 ? requested : 0;
    for (int mt = kTiles; mt >= 1; --mt)
        if (down_grouped_lds(B, k, a_bf16, mt) <= 65536)
            return mt;
    return 0;
}

hipError_t launch_down_grouped(const DownArgs& p, bool a_bf16, bool out_bf16, float* y, int max_tiles,
                               hipStream_t s)
{
    if ((long)p.B * p.k == 0)
        return hipSuccess;
    if (max_tiles < 1 || max_tiles > kTiles || (p.H % 16) != 0)
        return hipErrorInvalidValue;
    const int nblk = (p.H + kGroupNeurons - 1) / kGroupNeurons;
    const dim3 grid((unsigned)((long)p.E * nblk)), block(kGroupWaves * kWave);
    const size_t lds = down_grouped_lds(p.B, p.k, a_bf16, max_tiles);
    const bool fp4 = p.wfmt == kMXFP4;
    if (fp4) {
        if (a_bf16)
            hipLaunchKernelGGL((moe_down_expert_kernel<true, true>), grid, block, lds, s, p, y, max_tiles);
        else
            hipLaunchKernelGGL((moe_down_expert_kernel<false, true>), grid, block, lds, s, p, y, max_tiles);
    } else {
        if (a_bf16)
            hipLaunchKernelGGL((moe_down_expert_kernel<true, false>), grid, block, lds, s, p, y, max_tiles);
        else
            hipLaunchKernelGGL((moe_down_expert_kernel<false, false>), grid, block, lds, s, p, y, max_tiles);
    }
    hipError_t err = hipGetLastError();
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
