// Diagnostic kernel: decodes MXFP8 and MXFP4 values with exactly the
// in-register routes the layer kernels use, so a test can check all 256 E4M3
// codes and all 16 E2M1 codes (and a range of UE8M0 scales) bit for bit
// against the format definitions.
//
// MXFP4 paths: codes[t] holds one E2M1 code in its low nibble; the kernel
// places it at nibble t % 8 of a dword of filler nibbles (element 2u in the
// low and 2u+1 in the high nibble of byte u), converts byte (t % 8) / 2 and
// takes element t % 2 of the pair, so every byte select and both nibble
// positions are exercised.
#include "launch.h"
#include "mx_device.h"

namespace moed {

__global__ void __launch_bounds__(256)
moe_selftest_decode_kernel(const uint8_t* codes, const uint8_t* scales, float* out, int n, int path)
{
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n)
        return;
    const uint32_t c = codes[t];
    const float s = ue8m0_to_f32(scales[t]);
    if (path >= 3) {
        const int nib = t & 7;
        const uint32_t word = (0x3C3C3C3Cu & ~(0xFu << (4 * nib))) | ((c & 0xFu) << (4 * nib));
        float v;
        if (path == 5) {                          // E2M1 -> BF16, scale folded (the grouped route)
            bf16x2 w;
            switch (nib >> 1) {
            case 0: w = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, s, 0); break;
            case 1: w = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, s, 1); break;
            case 2: w = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, s, 2); break;
            default: w = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, s, 3); break;
            }
            out[t] = (float)((nib & 1) ? w.y : w.x);
            return;
        }
        if (path == 3) {                          // E2M1 -> BF16 (the gate/up dot2 route)
            bf16x2 w;
            switch (nib >> 1) {
            case 0: w = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 0); break;
            case 1: w = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 1); break;
            case 2: w = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 2); break;
            default: w = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, 3); break;
            }
            v = (float)((nib & 1) ? w.y : w.x);
        } else {                                  // E2M1 -> FP32 (the down kernel's route)
            f32x2 w;
            switch (nib >> 1) {
            case 0: w = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0); break;
            case 1: w = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1); break;
            case 2: w = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2); break;
            default: w = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3); break;
            }
            v = (nib & 1) ? w.y : w.x;
        }
        out[t] = v * s;
        return;
    }
    // place the code at byte position t % 4 of a dword whose other bytes are
    // filler, so every byte lane of both conversions is exercised
    const int pos = t & 3;
    const uint32_t word = (0x5A5A5A5Au & ~(0xFFu << (8 * pos))) | (c << (8 * pos));
    float v;
    if (path == 2) {
        // the grouped kernel's route: FP8 -> BF16 with the block scale folded in
        const bf16x2 w = pos >= 2 ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, s, true)
                                  : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, s, false);
        out[t] = (float)((pos & 1) ? w.y : w.x);
        return;
    }
    if (path == 0) {
        const f32x2 w = pos >= 2 ? __builtin_amdgcn_cvt_pk_f32_fp8(word, true)
                                 : __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
        v = (pos & 1) ? w.y : w.x;
    } else {
        const bf16x2 w = pos >= 2 ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, true)
                                  : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, false);
        v = (float)((pos & 1) ? w.y : w.x);
    }
    out[t] = v * s;
}

hipError_t launch_selftest_decode(const uint8_t* codes, const uint8_t* scales, float* out, int n,
                                  int path, hipStream_t s)
{
    if (n == 0)
        return hipSuccess;
    hipLaunchKernelGGL(moe_selftest_decode_kernel, dim3((n + 255) / 256), dim3(256), 0, s,
                       codes, scales, out, n, path);
    return hipGetLastError();
}

}  // namespace moed
