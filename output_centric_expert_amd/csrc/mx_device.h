// Device helpers shared by the gate/up and down kernels (gfx950 / CDNA4 only).
//
// MXFP8 decode: a weight is E4M3(code) * 2^(scale - 127), one UE8M0 scale per
// 32 codes along the reduction axis. A 16-code chunk always lies inside one
// 32-code block, so a lane sums its 16 products at scale 1 and multiplies the
// partial by the block scale once; the scale is a power of two, so this is
// the same value as scaling every product (barring float32 under/overflow).
//
// Both conversions used here are exact: every E4M3 value is representable in
// bfloat16 (3 mantissa bits, exponents 2^-9 .. 2^8) and in float32, and the
// product of an E4M3 value with a bfloat16 activation (4 x 8 significant bits)
// is exact in float32. Only the float32 accumulation rounds.
//
// MXFP4 decode: a weight is E2M1(code) * 2^(scale - 127), codes two per byte
// (element 2t in the low nibble of byte t). A 16-byte chunk holds 32 codes,
// exactly one MX block, so the block scale is again applied once per lane
// partial. E2M1 values (2 significant bits, 0.5 .. 6) are exact in bfloat16 and
// float32, and so are their products with bfloat16 activations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moed {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

template <bool NT, typename T>
__device__ __forceinline__ T ld(const T* p)
{
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

// UE8M0 byte -> 2^(s-127) as float32. s = 0 is the float32 subnormal 2^-127;
// s = 255 is NaN.
__device__ __forceinline__ float ue8m0_to_f32(uint32_t s)
{
    uint32_t bits = s << 23;
    bits = (s == 0u) ? 0x00400000u : bits;
    bits = (s == 255u) ? 0x7FC00000u : bits;
    return __uint_as_float(bits);
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v)
{
    return __builtin_bit_cast(bf16x2, v);
}

// bfloat16 pair in one dword -> the two float32 values (low half first).
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// acc + sum_{t<4} E4M3(codes.byte[t]) * x[t], with x[0..3] packed as two bf16 pairs.
// FP8 -> BF16 (v_cvt_scalef32_pk_bf16_fp8, scale 1; exact) and a BF16 dot2
// with FP32 accumulation (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot4_bf16(uint32_t codes, uint32_t x01, uint32_t x23, float acc)
{
    const bf16x2 w01 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, false);
    const bf16x2 w23 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, true);
    acc = __builtin_amdgcn_fdot2_f32_bf16(w01, as_bf16x2(x01), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(w23, as_bf16x2(x23), acc, false);
    return acc;
}

// acc + sum_{t<8} E2M1(nibble t of codes) * x[t], x[0..7] as 8 bf16 in a u32x4
// (dword d = the pair 2d, 2d+1): byte d of the codes converts to the same pair
// (v_cvt_scalef32_pk_bf16_fp4, scale 1), then one BF16 dot2 per pair.
__device__ __forceinline__ float dot8_fp4_bf16(uint32_t codes, u32x4 x, float acc)
{
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, 0),
                                          as_bf16x2(x.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, 1),
                                          as_bf16x2(x.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, 2),
                                          as_bf16x2(x.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, 3),
                                          as_bf16x2(x.w), acc, false);
    return acc;
}

// acc + sum_{t<8} E2M1(nibble t of codes) * a[t] with float32 activations
// a[0..3] = lo, a[4..7] = hi (v_cvt_scalef32_pk_f32_fp4, scale 1, then FMAs).
__device__ __forceinline__ float dot8_fp4_f32a(uint32_t codes, f32x4 lo, f32x4 hi, float acc)
{
    const f32x2 w0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
    const f32x2 w1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
    const f32x2 w2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
    const f32x2 w3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
    acc = __builtin_fmaf(w0.x, lo.x, acc);
    acc = __builtin_fmaf(w0.y, lo.y, acc);
    acc = __builtin_fmaf(w1.x, lo.z, acc);
    acc = __builtin_fmaf(w1.y, lo.w, acc);
    acc = __builtin_fmaf(w2.x, hi.x, acc);
    acc = __builtin_fmaf(w2.y, hi.y, acc);
    acc = __builtin_fmaf(w3.x, hi.z, acc);
    acc = __builtin_fmaf(w3.y, hi.w, acc);
    return acc;
}

// acc + sum_{t<4} E4M3(codes.byte[t]) * a[t] with float32 activations.
__device__ __forceinline__ float dot4_f32a(uint32_t codes, f32x4 a, float acc)
{
    const f32x2 w01 = __builtin_amdgcn_cvt_pk_f32_fp8(codes, false);
    const f32x2 w23 = __builtin_amdgcn_cvt_pk_f32_fp8(codes, true);
    acc = __builtin_fmaf(w01.x, a.x, acc);
    acc = __builtin_fmaf(w01.y, a.y, acc);
    acc = __builtin_fmaf(w23.x, a.z, acc);
    acc = __builtin_fmaf(w23.y, a.w, acc);
    return acc;
}

// Sum over the 64 lanes of a wavefront; every lane gets the total. The order
// is fixed, so results are deterministic. Inside each 16-lane row the partial
// sums are exchanged with DPP (quad_perm xor 1, xor 2, row_half_mirror,
// row_mirror); rows 0/1 and 2/3 are combined with a ds_swizzle (lane ^ 16
// within each 32-lane half), and the two halves by reading lanes 0 and 32.
// No LDS memory, no barrier. All 64 lanes must be active.
__device__ __forceinline__ float wave_sum(float v)
{
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x141, 0xF, 0xF, true);  // row_half_mirror
    v += __builtin_amdgcn_update_dpp(0.0f, v, 0x140, 0xF, 0xF, true);  // row_mirror
    // ds_swizzle bit mode: and_mask 0x1F, or_mask 0, xor_mask 0x10 -> lane ^ 16
    v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (0x10 << 10) | 0x1F));
    const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    return lo + hi;
}

// Workgroups go to the 8 XCDs of the chip in turn (workgroup i to XCD i % 8),
// and each XCD has its own L2. xcd_contiguous(i, n) renumbers the n
// workgroups of a launch so that every XCD runs one contiguous range of
// logical indices: work that reads the same bytes and sits at neighbouring
// logical indices then meets in one L2. It is a bijection of [0, n).
__device__ __forceinline__ int xcd_contiguous(int i, int n)
{
    // XCD x starts at x*q + min(x, r): the first r XCDs take q + 1 indices,
    // the others q (written without a branch, so a kernel's argument loads
    // are not split around it)
    const int x = i % 8, slot = i / 8;
    const int q = n / 8, r = n % 8;
    return x * q + (x < r ? x : r) + slot;
}

// Two float32 -> two bfloat16, round to nearest even (v_cvt_pk_bf16_f32), a
// in the low half. NaN stays NaN. Over all 2^32 float32 inputs it gives the
// same bits as rounding the bit pattern (add 0x7FFF plus the kept lsb, keep
// the high half) for every non-NaN input, and a NaN exactly for NaN inputs.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// float32 -> bfloat16 bits, round to nearest even; NaN stays a NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    return (uint16_t)(f32x2_to_bf16x2_rne(f, 0.0f) & 0xFFFFu);
}

// Position of a[b][j][i] (bj = b*k + j) in the intermediate buffer. The
// buffer is chunk-interleaved so that the down kernel's loads are contiguous
// across lanes: row bj is split into 16-value chunks o = i / 16, and each
// chunk into 16-byte pieces q (4 float32 values, or 8 bf16 values); piece q of
// every chunk of the row is stored contiguously:
//   float32: index ((bj*4 + q) * (I/16) + o) * 4 + i % 4,  q = (i / 4) % 4
//   bf16:    index ((bj*2 + q) * (I/16) + o) * 8 + i % 8,  q = (i / 8) % 2
template <bool BF16>
__device__ __forceinline__ size_t inter_index(int bj, int i, int I)
{
    const size_t cpr = (size_t)(I / 16);
    const size_t o = (size_t)(i >> 4);
    if constexpr (BF16)
        return (((size_t)bj * 2 + (size_t)((i >> 3) & 1)) * cpr + o) * 8 + (size_t)(i & 7);
    else
        return (((size_t)bj * 4 + (size_t)((i >> 2) & 3)) * cpr + o) * 4 + (size_t)(i & 3);
}

// SiLU(g) * u with SiLU(t) = t / (1 + exp(-t)), from the hardware base-2
// exponential and reciprocal (v_exp_f32, v_rcp_f32; about 1e-6 relative for
// |t| < 100). Overflow of exp(-t) gives rcp(inf) = 0, so the result is -0,
// never NaN.
__device__ __forceinline__ float swiglu(float g, float u)
{
    const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

}  // namespace moed
