// Down for large decode batches: still output-centric -- every out[b][h] is
// accumulated in one FP32 accumulator over all of token b's routed experts
// and stored once -- but a workgroup owns a tile of 16 outputs h x 16 tokens
// b, so each routed down row is decoded once per 16 tokens instead of once
// per token.
//
// The workgroup lists (in increasing expert order) the experts its tokens are
// routed to and loops over them. For expert e the contribution to the tile is
// the MFMA product
//   A = Wd[e][h0 .. h0+15][:], decoded exactly from MXFP8 to BF16 with the
//       block scale folded into the conversion,
//   B[:, c] = sum over token c's slots j routed to e of w[c][j] * a[c][j][:]
//       (zero for tokens not routed to e), an FP32 value carried as two BF16
//       numbers hi + lo (hi = RNE(v), lo = RNE(v - hi); about 16 significant
//       bits), so that both products are exact in FP32,
//   D += A * B_hi + A * B_lo   (v_mfma_f32_16x16x32_bf16, FP32 accumulation).
// The routing weight is folded into B before the product. The four
// wavefronts of the workgroup split I between them; their FP32 partial tiles
// are added in a fixed order through LDS, and lane (h, b) stores out[b][h].
// Tokens with an expert id outside [0, E) get NaN outputs.
#include "launch.h"
#include "mx_device.h"

namespace moed {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int kDnWaves = 4;                      // wavefronts per workgroup, splitting I
constexpr int kDnMaxExperts = 2048;              // expert bitmap capacity (E <= this)
constexpr int kDnMaxK = 64;                      // routed slots per token (k <= this)

__device__ __forceinline__ bf16x8 decode8_scaled_dn(u32x2 codes, float scale)
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

// v (8 float32) -> hi, lo (8 bf16 each) with hi + lo = v to ~2^-17 relative.
__device__ __forceinline__ void split_hi_lo(const f32x8& v, bf16x8& hi, bf16x8& lo)
{
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint16_t hb = f32_to_bf16_rne(v[t]);
        const float hf = __uint_as_float((uint32_t)hb << 16);
        const uint16_t lb = f32_to_bf16_rne(v[t] - hf);
        hi[t] = __builtin_bit_cast(__bf16, hb);
        lo[t] = __builtin_bit_cast(__bf16, lb);
    }
}

template <bool A_BF16>
__device__ __forceinline__ f32x8 load_a8(const void* a, int bj, int i0, int I)
{
    // 8 consecutive values a[bj][i0 .. i0+7] (i0 % 8 == 0) from the
    // chunk-interleaved intermediate
    f32x8 v;
    const size_t cpr = (size_t)(I / 16);
    const size_t o = (size_t)(i0 >> 4);
    if constexpr (A_BF16) {
        const size_t idx = (((size_t)bj * 2 + (size_t)((i0 >> 3) & 1)) * cpr + o) * 8;
        const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a) + idx);
        v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
        v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
    } else {
        const size_t q0 = (size_t)((i0 >> 2) & 3);
        const float* af = static_cast<const float*>(a);
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(af + (((size_t)bj * 4 + q0) * cpr + o) * 4);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(af + (((size_t)bj * 4 + q0 + 1) * cpr + o) * 4);
        v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
        v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
    }
    return v;
}

template <bool A_BF16, bool OUT_BF16>
__global__ void __launch_bounds__(kDnWaves * kWave)
moe_down_grouped_kernel(DownArgs p)
{
    __shared__ unsigned bitmap[kDnMaxExperts / 32];
    __shared__ int experts[kDnMaxExperts];
    __shared__ int wave_cnt[kDnWaves];
    __shared__ f32x4 partial[kDnWaves - 1][kWave];
    __shared__ int tile_ids[16 * kDnMaxK];
    __shared__ float tile_w[16 * kDnMaxK];

    const int H = p.H, I = p.I, k = p.k, E = p.E, B = p.B;
    const int nht = H / 16;                       // H is a multiple of 32
    const int h0 = (blockIdx.x % nht) * 16;
    const int b0 = (blockIdx.x / nht) * 16;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int kb = lane / 16;
    const int col = lane % 16;

    // 1) the tile's expert set as a bitmap, then an ordered list
    const int nwords = (E + 31) / 32;
    for (int q = tid; q < nwords; q += blockDim.x)
        bitmap[q] = 0u;
    __syncthreads();
    const int ntok = B - b0 < 16 ? B - b0 : 16;
    for (int q = tid; q < ntok * k; q += blockDim.x) {
        const int e = p.ids[(size_t)b0 * k + q];
        tile_ids[q] = e;
        tile_w[q] = p.w[(size_t)b0 * k + q];
        if ((unsigned)e < (unsigned)E)
            atomicOr(&bitmap[e >> 5], 1u << (e & 31));
    }
    __syncthreads();
    int nexp = 0;
    for (int base = 0; base < nwords; base += kDnWaves * kWave) {
        const int q = base + tid;
        const unsigned word = q < nwords ? bitmap[q] : 0u;
        const int cnt = __popc(word);
        // exclusive prefix of cnt over the workgroup (wave scan + wave totals)
        int incl = cnt;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int y = __shfl_up(incl, d);
            if (lane >= d)
                incl += y;
        }
        if (lane == kWave - 1)
            wave_cnt[w] = incl;
        __syncthreads();
        int off = nexp;
        for (int r = 0; r < w; ++r)
            off += wave_cnt[r];
        int pos = off + incl - cnt;
        unsigned m = word;
        while (m) {
            const int bit = __ffs(m) - 1;
            experts[pos++] = q * 32 + bit;
            m &= m - 1u;
        }
        int sum = 0;
        for (int r = 0; r < kDnWaves; ++r)
            sum += wave_cnt[r];
        __syncthreads();
        nexp += sum;
    }

    // 2) this lane's token (column col) and whether it has an invalid id
    const int ccol = col < ntok ? col : 0;
    const int bcol = b0 + ccol;
    bool bad = false;
    for (int j = 0; j < k; ++j)
        bad |= (unsigned)tile_ids[ccol * k + j] >= (unsigned)E;

    // 3) the wavefront's share of I: 128-code groups w, w+4, ...; leftover
    //    32-code blocks (I/32 % 4) go to wavefront 0 in plain k order
    const size_t row_base = (size_t)(h0 + col);
    const int ngroups = I / 128;
    const int nleft = (I / 32) % 4;
    f32x4 d = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int x = 0; x < nexp; ++x) {
        const int e = experts[x];
        // this column's coefficient and slot for expert e
        float coef = 0.0f;
        int jsel = -1;
        for (int j = 0; j < k; ++j) {
            if (tile_ids[ccol * k + j] == e) {
                coef += tile_w[ccol * k + j];
                jsel = jsel < 0 ? j : jsel;
            }
        }
        const bool has = jsel >= 0 && col < ntok;
        const int bj = bcol * k + (jsel < 0 ? 0 : jsel);
        const size_t row = (size_t)e * (size_t)H + row_base;
        const uint8_t* wq = p.wd_q + row * (size_t)I;
        const uint8_t* ws = p.wd_s + row * (size_t)(I / 32);
        for (int g = w; g < ngroups; g += kDnWaves) {
            const int kbase = g * 128 + 32 * kb;  // this lane's MX block (permuted k order)
            const u32x4 c0 = *reinterpret_cast<const u32x4*>(wq + kbase);
            const u32x4 c1 = *reinterpret_cast<const u32x4*>(wq + kbase + 16);
            const float sc = ue8m0_to_f32(ws[g * 4 + kb]);
            f32x8 av[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (has) {
                    av[q] = load_a8<A_BF16>(p.a, bj, kbase + 8 * q, I);
                } else {
#pragma unroll
                    for (int t = 0; t < 8; ++t)
                        av[q][t] = 0.0f;
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4 src = q < 2 ? c0 : c1;
                const u32x2 cq = (q & 1) ? u32x2{src.z, src.w} : u32x2{src.x, src.y};
                const bf16x8 aw = decode8_scaled_dn(cq, sc);
                f32x8 v;
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    v[t] = coef * av[q][t];
                bf16x8 bhi, blo;
                split_hi_lo(v, bhi, blo);
                d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, bhi, d, 0, 0, 0);
                d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, blo, d, 0, 0, 0);
            }
        }
        if (w == 0) {
            for (int st = ngroups * 4; st < ngroups * 4 + nleft; ++st) {
                const int k0 = st * 32 + 8 * kb;
                const u32x2 cq = *reinterpret_cast<const u32x2*>(wq + k0);
                const bf16x8 aw = decode8_scaled_dn(cq, ue8m0_to_f32(ws[st]));
                f32x8 v;
                if (has) {
                    const f32x8 av = load_a8<A_BF16>(p.a, bj, k0, I);
#pragma unroll
                    for (int t = 0; t < 8; ++t)
                        v[t] = coef * av[t];
                } else {
#pragma unroll
                    for (int t = 0; t < 8; ++t)
                        v[t] = 0.0f;
                }
                bf16x8 bhi, blo;
                split_hi_lo(v, bhi, blo);
                d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, bhi, d, 0, 0, 0);
                d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, blo, d, 0, 0, 0);
            }
        }
    }

    // 4) add the four partial tiles in a fixed order; one store per output
    if (w > 0)
        partial[w - 1][lane] = d;
    __syncthreads();
    if (w != 0)
        return;
#pragma unroll
    for (int r = 0; r < kDnWaves - 1; ++r)
        d += partial[r][lane];
    if (col < ntok) {
        const int b = b0 + col;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int h = h0 + 4 * kb + r;
            const float v = bad ? __builtin_nanf("") : d[r];
            if constexpr (OUT_BF16)
                static_cast<uint16_t*>(p.out)[(size_t)b * H + h] = f32_to_bf16_rne(v);
            else
                static_cast<float*>(p.out)[(size_t)b * H + h] = v;
        }
    }
}

hipError_t launch_down_grouped(const DownArgs& p, bool a_bf16, bool out_bf16, const Tuning& t, hipStream_t s)
{
    (void)t;
    if ((long)p.B * p.H == 0)
        return hipSuccess;
    const dim3 grid((unsigned)((long)(p.H / 16) * ((p.B + 15) / 16)));
    const dim3 block(kDnWaves * kWave);
    if (a_bf16) {
        if (out_bf16) hipLaunchKernelGGL((moe_down_grouped_kernel<true, true>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((moe_down_grouped_kernel<true, false>), grid, block, 0, s, p);
    } else {
        if (out_bf16) hipLaunchKernelGGL((moe_down_grouped_kernel<false, true>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((moe_down_grouped_kernel<false, false>), grid, block, 0, s, p);
    }
    return hipGetLastError();
}

bool down_grouped_fits(int E, int k) { return E <= kDnMaxExperts && k <= kDnMaxK; }

}  // namespace moed
