// Diagnostic kernel: decodes MXFP8 values with exactly the in-register routes
// the layer kernels use, so a test can check all 256 E4M3 codes (and a range
// of UE8M0 scales) bit for bit against the format definition.
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
