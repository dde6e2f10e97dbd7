/*
 * libmoedecode -- output-centric MoE decode expert layer for MI355X (gfx950).
 *
 * The layer is the routed SwiGLU expert block of a mixture-of-experts model at
 * decode time, computed the way the warp-decode post describes it
 * (cursor.com/blog/warp-decode, sections "What changed" and "How the two
 * kernels work"): parallelism is organised around OUTPUTS, not experts.
 *
 *   gate/up kernel: one 64-lane wavefront owns one intermediate neuron i of one
 *     (token b, routed slot j) pair. It reads the routed expert id e, streams
 *     the MXFP8 gate and up rows Wg[e][i][:] and Wu[e][i][:], decodes them in
 *     registers, dots both against x[b][:] (read once for both projections),
 *     reduces across lanes and writes one value  a[b][j][i] = SiLU(g) * u.
 *   down kernel: one wavefront owns one output out[b][h]. It loops over the k
 *     routed experts, streams Wd[e_j][h][:] against a[b][j][:], and folds each
 *     routing weight w[b][j] into a single FP32 accumulator before one store.
 *
 * There are no gather, pad or scatter buffers and no per-expert output buffer
 * ("Buffer removal" section); the only intermediate is a[B][k][I].
 *
 * Weight formats (argument weight_format; both from the GC-MoE summary,
 * onedev.kr/papers/1690, section "How to use", which names FP8 E4M3 and FP4
 * E2M1 block formats with one UE8M0 scale per 32 values along K):
 *  - MOED_MXFP8: codes are OCP FP8 E4M3 (bias 7, NaN = 0x7F/0xFF, no
 *    infinities), one byte each; a row of K values is K bytes.
 *  - MOED_MXFP4: codes are OCP FP4 E2M1 (bias 1; values 0, 0.5, 1, 1.5, 2,
 *    3, 4, 6 and negatives; no NaN, no infinities), two per byte: element 2t
 *    in the low nibble (bits 3..0) of byte t, element 2t+1 in the high nibble;
 *    a row of K values is K/2 bytes.
 * In both, every 32 consecutive values along the reduction axis share one
 * UE8M0 scale byte, value 2^(s-127) (0xFF = NaN), in a separate [..][K/32]
 * tensor. Decoded weight = element(code) * 2^(scale-127).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA
 *    memory) on the current device, C-contiguous, no strides. The caller owns
 *    every buffer; the library allocates nothing on these paths.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream) and never synchronise. They keep no state between calls: the
 *    launch shape comes from a built-in table, or from the moed_tuning a
 *    *_tuned call is handed. Calls may be made from any number of host
 *    threads at once; concurrent calls need distinct workspaces/outputs.
 *  - Argument errors are reported before anything is launched. A launch
 *    failure returns MOED_ERR_HIP; moed_last_hip_error() gives the raw code.
 *  - Expert ids outside [0, E) are not an error: every output of the affected
 *    token becomes NaN (no out-of-bounds read is made). NaN codes or scales
 *    in the weights propagate as NaN.
 *  - Opt-in check: with MOED_CHECK=1 in the environment (read on every call)
 *    moe_decode, moe_decode_gate_up and moe_decode_down first run a check
 *    kernel on `stream` and return MOED_ERR_SHAPE, launching nothing else,
 *    if an expert id lies outside [0, E) or a routed expert's rows (of the
 *    matrices the call uses) hold a NaN code (E4M3 S.1111.111) or a NaN scale
 *    (UE8M0 0xFF), and MOED_ERR_SCALE if the call takes a large-batch kernel
 *    (see moe_decode) and a routed block scale of the matrices it decodes
 *    lies outside the range that kernel decodes exactly. This mode
 *    synchronises the stream (so it cannot be used under graph capture). Its
 *    flag word is a device array of the library (no allocation); checked
 *    calls that overlap on one device share it and race.
 *  - Duplicate ids within a token's row are legal and their terms add; the
 *    routing weights need not sum to 1.
 *  - Results are deterministic run to run (fixed reduction order).
 */
#ifndef MOEDECODE_H
#define MOEDECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOED_OK = 0,
    MOED_ERR_NULL = 1,       /* a required pointer is NULL                       */
    MOED_ERR_SHAPE = 2,      /* B<0, E<1, k<1, k>E, H or I not a positive multiple of 32,
                                or a size beyond the limits below                */
    MOED_ERR_DTYPE = 3,      /* unknown moed_dtype or moed_wformat                */
    MOED_ERR_WORKSPACE = 4,  /* workspace smaller than moed_workspace_bytes()     */
    MOED_ERR_ALIGN = 5,      /* x, a, workspace or a weight-code base not 16-byte aligned */
    MOED_ERR_HIP = 6,        /* a HIP launch failed; see moed_last_hip_error()    */
    MOED_ERR_SCALE = 7,      /* (MOED_CHECK only) a routed block scale outside the exact
                                range of the large-batch kernel the call takes     */
    MOED_ERR_TUNING = 8      /* a moed_tuning not filled by moed_tuning_init()    */
} moed_status;

typedef enum {
    MOED_BF16 = 0,           /* bfloat16, round-to-nearest-even on store          */
    MOED_F32 = 1             /* IEEE float32                                      */
} moed_dtype;

typedef enum {
    MOED_MXFP8 = 0,          /* E4M3 codes, one per byte                          */
    MOED_MXFP4 = 1           /* E2M1 codes, two per byte (low nibble first)       */
} moed_wformat;

/* Size limits (checked): B*k*I and B*H below 2^31, k*I/16 below 2^22. */

/*
 * Bytes of workspace moe_decode() needs. The post's two kernels hand over one
 * intermediate value per (token, slot, neuron) ("How the two kernels work":
 * the gate/up kernel writes one intermediate value, the down kernel reads the
 * row it needs); it is the only buffer between them ("Buffer removal"). So:
 * the intermediate a[B][k][I]
 * (B*k*I*4 bytes for inter_dtype MOED_F32, the accuracy-gated path; *2 for
 * MOED_BF16), rounded up to 256 bytes, then B*k*H float32 per-slot partials
 * y[b][j][h] = topk_w[b][j] * (Wd^[e]·a[b][j])_h, which the expert-major down
 * step writes when tokens share experts (batches with B*k >= 2E) and adds up
 * per token in slot order. Returns 0 for B = 0 and for invalid arguments.
 */
size_t moed_workspace_bytes(int B, int k, int H, int I, int inter_dtype);

/*
 * The whole layer (steps gate/up then down on `stream`): the routed SwiGLU
 * expert block of the warp-decode post ("What changed": two kernels, the
 * first one wavefront per intermediate neuron, the second one wavefront per
 * output; "How the two kernels work": each output folds every routed
 * expert's weighted contribution into one FP32 accumulator and is stored
 * once):
 *   out[b][h] = sum_j topk_w[b][j] * sum_i Wd^[e][h][i] * SiLU(g_i) * u_i,
 *   g_i = sum_h' Wg^[e][i][h'] x[b][h'],  u_i = sum_h' Wu^[e][i][h'] x[b][h'],
 *   e = topk_ids[b][j], W^ the decoded MX weights.
 *   x         [B][H]  bfloat16 activations
 *   topk_ids  [B][k]  int32 routed expert ids
 *   topk_w    [B][k]  float32 routing weights (folded in the down kernel)
 *   wg_q/wu_q [E][I][H] uint8 codes of the gate / up projections, K = H
 *             ([E][I][H/2] for MOED_MXFP4)
 *   wg_s/wu_s [E][I][H/32] uint8 UE8M0 scales
 *   wd_q      [E][H][I] uint8 codes of the down projection, K = I
 *             ([E][H][I/2] for MOED_MXFP4)
 *   wd_s      [E][H][I/32] uint8 UE8M0 scales
 *   weight_format  MOED_MXFP8 or MOED_MXFP4 (all three projections)
 *   out       [B][H]  out_dtype
 *   workspace >= moed_workspace_bytes(B, k, H, I, inter_dtype) bytes, 16-aligned
 * B = 0 is valid and launches nothing.
 *
 * Once tokens share experts (B*k >= 2E) the down step runs expert-major: the
 * decoded rows of each routed expert serve every slot routed to it, each slot's
 * weighted partial goes to the workspace, and a second launch adds each
 * token's k partials in slot order and stores the output once. Smaller batches
 * use the one-wavefront-per-output down of moe_decode_down(). Likewise the
 * gate/up step runs expert-grouped (MFMA) once 4*B*k >= 3*E, or for rows of
 * H >= 6144 values once min(B*k, E)*ceil(I/64) >= 512. Both large-batch forms
 * hold slot indices in 16 bits: at B*k >= 65536 the layer keeps the per-slot
 * gate/up and the per-output down (same results within the tolerance, slower).
 *
 * Exact range of the large-batch kernels: they decode a weight to BF16 with
 * its block scale folded into the conversion, which is exact while every
 * scaled value is a normal, finite BF16 number -- scale codes 10..245 for
 * MXFP8 and 2..252 for MXFP4 (weights quantized from real value ranges sit
 * far inside; the synthetic ones use codes near 115). Outside that range
 * those kernels flush tiny blocks to zero or overflow huge ones where the
 * single-token kernels stay exact; MOED_CHECK=1 reports such scales.
 */
int moe_decode(const void *x, const int32_t *topk_ids, const float *topk_w,
               const uint8_t *wg_q, const uint8_t *wg_s,
               const uint8_t *wu_q, const uint8_t *wu_s,
               const uint8_t *wd_q, const uint8_t *wd_s, int weight_format,
               void *out, int out_dtype, int inter_dtype,
               int B, int E, int k, int H, int I,
               void *workspace, size_t workspace_bytes, void *stream);

/*
 * The whole layer without a workspace argument, for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation. Arguments, results and errors as moe_decode() without
 * its workspace; the intermediate and the per-slot partials go to a scratch
 * array the library holds in device memory instead: 32 MiB per device, part of
 * the library's code object, kept until the process ends (its address is
 * taken on the first call on each device). Sizes whose
 * moed_workspace_bytes(B, k, H, I, inter_dtype) exceeds 32 MiB return
 * MOED_ERR_WORKSPACE before anything is launched (every workload of up to
 * B = 64 tokens at H = 7168, I = 2048, k = 8 fits). Nothing in the array has
 * to start at zero: every call writes what it reads. All calls on one device
 * share the array, so calls that overlap on one device (from other streams
 * or host threads) race; the caller serialises them. Allocates nothing.
 */
int moe_decode_noalloc(const void *x, const int32_t *topk_ids, const float *topk_w,
                       const uint8_t *wg_q, const uint8_t *wg_s,
                       const uint8_t *wu_q, const uint8_t *wu_s,
                       const uint8_t *wd_q, const uint8_t *wd_s, int weight_format,
                       void *out, int out_dtype, int inter_dtype,
                       int B, int E, int k, int H, int I, void *stream);

/*
 * Gate/up step alone: a[b][j][i] = SiLU(Wg^[e]·x[b])_i * (Wu^[e]·x[b])_i with
 * e = topk_ids[b][j], stored as inter_dtype into `a` (B*k*I elements).
 * SiLU(t) = t / (1 + exp(-t)).  (Warp-decode post, "How the two kernels work",
 * first two paragraphs.)
 *
 * Layout of `a` (the same buffer moe_decode() keeps in its workspace): row
 * bj = b*k + j is chunk-interleaved so the down kernel's loads are contiguous
 * across a wavefront. With o = i/16 and cpr = I/16:
 *   MOED_F32:  element index ((bj*4 + (i/4)%4) * cpr + o) * 4 + i%4
 *   MOED_BF16: element index ((bj*2 + (i/8)%2) * cpr + o) * 8 + i%8
 */
int moe_decode_gate_up(const void *x, const int32_t *topk_ids,
                       const uint8_t *wg_q, const uint8_t *wg_s,
                       const uint8_t *wu_q, const uint8_t *wu_s, int weight_format,
                       void *a, int inter_dtype,
                       int B, int E, int k, int H, int I, void *stream);

/*
 * Down step alone: out[b][h] = sum_j topk_w[b][j] * (Wd^[e_j]·a[b][j])_h.
 * `a` is in the layout moe_decode_gate_up() writes. (Warp-decode post, "How
 * the two kernels work", third and fourth paragraphs.)
 *   partials  NULL: one wavefront per output, one FP32 accumulator over the k
 *             routed experts, one store.
 *             Else float32 scratch of partials_bytes >= B*k*H*4 bytes,
 *             16-aligned, owned by the caller: once tokens share experts
 *             (B*k >= 2E) the expert-major form runs (the form moe_decode()
 *             uses), writing topk_w[b][j] * (Wd^[e_j]·a[b][j]) there and then
 *             adding each token's k partials in slot order; smaller batches
 *             still take the per-output form and leave it untouched.
 *             Too small: MOED_ERR_WORKSPACE; misaligned: MOED_ERR_ALIGN.
 */
int moe_decode_down(const void *a, int inter_dtype, const int32_t *topk_ids,
                    const float *topk_w, const uint8_t *wd_q, const uint8_t *wd_s,
                    int weight_format, void *out, int out_dtype,
                    int B, int E, int k, int H, int I,
                    float *partials, size_t partials_bytes, void *stream);

/*
 * Router front-end: the layer's topk_ids / topk_w from float32 router logits
 * [B][E] (device), on `stream`. Per token: the k experts with the largest
 * logits, in descending order, ties to the lower expert id (the top-k of the
 * routing probabilities softmax(logits), which is strictly increasing); their
 * weights exp(l_j - m) / sum_j' exp(l_j' - m) * routed_scale with m the largest
 * logit (the renormalised top-k probabilities, computed in float32); then
 * n_shared shared-expert slots with ids E, E+1, ... and weight 1. Rows of
 * topk_ids (int32) and topk_w (float32) hold k + n_shared entries.
 *
 * Shared experts: store each shared expert as an extra expert after the E
 * routed ones in the weight tensors (a shared expert of intermediate size
 * n*I as n such experts) and call moe_decode with E + n_shared experts and
 * k + n_shared slots: its term is then folded into the same accumulator as
 * the routed ones, and every output is still stored once (the GC-MoE
 * summary, onedev.kr/papers/1690, "How to use", fuses shared experts into the
 * routed-expert pass in the same way).
 *
 * A NaN logit is never selected; if fewer than k experts can be selected the
 * missing slots get id -1 (the layer then writes NaN for that token) and a NaN
 * weight. Limits (MOED_ERR_SHAPE): 1 <= k <= min(E, 64), E <= 2048,
 * n_shared >= 0. B = 0 launches nothing.
 */
int moe_route(const float *logits, int B, int E, int k, int n_shared, float routed_scale,
              int32_t *topk_ids, float *topk_w, void *stream);

/*
 * Diagnostic: decode n block-scaled values with the kernels' own in-register
 * decoders, so a test can compare every code bit for bit with the format
 * definitions. out[t] = element(codes[t]) * 2^(scales[t]-127) as float32:
 *   path 0: E4M3, FP8 -> FP32 conversion, scale applied afterwards;
 *   path 1: E4M3, FP8 -> BF16 conversion, scale applied afterwards;
 *   path 2: E4M3, FP8 -> BF16 with the block scale folded into the conversion
 *           (the large-batch route; exact for scale codes 10..245);
 *   path 3: E2M1 (low nibble of codes[t]), FP4 -> BF16, scale afterwards;
 *   path 4: E2M1 (low nibble of codes[t]), FP4 -> FP32, scale afterwards;
 *   path 5: E2M1, FP4 -> BF16 with the block scale folded into the conversion
 *           (the large-batch route; exact for scale codes 2..252).
 * The E2M1 paths place code t at nibble t % 8 of a packed dword, so every
 * byte select and both nibble positions are exercised.
 * Device pointers; n >= 0; path in {0, ..., 5}.
 */
int moed_selftest_decode(const uint8_t *codes, const uint8_t *scales, float *out,
                         int n, int path, void *stream);

/*
 * Measurement kernels (not part of the layer).
 * moed_bench_read: streams `bytes` from `src` with contiguous 16-byte loads --
 *   the peak-read reference the warp-decode post compares against (section
 *   "Hardware efficiency": peak measured with a copy kernel over contiguous
 *   reads). `sink` (>= 4096 bytes, device) is scratch that is almost never
 *   written. bytes % 16 == 0, src 16-byte aligned.
 * moed_bench_copy: dst[0..bytes) = src[0..bytes); a kernel of known traffic
 *   used to calibrate HBM byte counters. bytes % 16 == 0, both 16-aligned,
 *   the ranges must not overlap.
 * Both are asynchronous on `stream`; errors as for moe_decode().
 */
int moed_bench_read(const void *src, size_t bytes, void *sink, size_t sink_bytes, void *stream);
int moed_bench_copy(const void *src, void *dst, size_t bytes, void *stream);
/*
 * moed_bench_read_cfg: the same read with a chosen launch shape, to find the
 *   fastest a single launch can stream a given byte count: workgroups of
 *   waves_per_group (1..16) wavefronts, each wavefront reading chunks of
 *   unroll (1, 2, 4, 8 or 16) 16-byte units per lane with all of a chunk's
 *   loads in flight together; groups = 0 gives a grid that covers the bytes
 *   in one pass, groups > 0 that many workgroups looping over the chunks.
 *   Argument errors as moed_bench_read (MOED_ERR_SHAPE for a bad shape).
 */
int moed_bench_read_cfg(const void *src, size_t bytes, void *sink, size_t sink_bytes, int unroll,
                        int waves_per_group, int groups, void *stream);

/* Human-readable name of a moed_status value. Never NULL. */
const char *moed_status_string(int status);

/* Raw hipError_t of the last MOED_ERR_HIP returned on this thread (0 if none). */
int moed_last_hip_error(void);

/*
 * Launch-shape choice for one call, for launch-shape sweeps and for tests of
 * the alternative kernels (every choice computes the same layer). A plain
 * value owned by the caller; the library keeps no copy.
 * moed_tuning_init fills *t with the built-in table, then applies `spec`, a
 * comma-separated list of key=value pairs (e.g. "gu_group=0,dn_group=0");
 * NULL or "" leaves the built-in table. Returns MOED_OK, MOED_ERR_NULL for a
 * NULL t, or MOED_ERR_SHAPE for an unknown key or value (t is then left
 * unfilled).
 * The *_tuned calls are the calls above with a trailing `tuning` (NULL = the
 * built-in table, as in the plain calls); MOED_ERR_TUNING if *tuning was not
 * filled by moed_tuning_init.
 */
typedef struct { int32_t words[48]; } moed_tuning;

int moed_tuning_init(moed_tuning *t, const char *spec);
int moe_decode_tuned(const void *x, const int32_t *topk_ids, const float *topk_w,
                     const uint8_t *wg_q, const uint8_t *wg_s,
                     const uint8_t *wu_q, const uint8_t *wu_s,
                     const uint8_t *wd_q, const uint8_t *wd_s, int weight_format,
                     void *out, int out_dtype, int inter_dtype,
                     int B, int E, int k, int H, int I,
                     void *workspace, size_t workspace_bytes, void *stream,
                     const moed_tuning *tuning);
int moe_decode_gate_up_tuned(const void *x, const int32_t *topk_ids,
                             const uint8_t *wg_q, const uint8_t *wg_s,
                             const uint8_t *wu_q, const uint8_t *wu_s, int weight_format,
                             void *a, int inter_dtype,
                             int B, int E, int k, int H, int I, void *stream,
                             const moed_tuning *tuning);
int moe_decode_down_tuned(const void *a, int inter_dtype, const int32_t *topk_ids,
                          const float *topk_w, const uint8_t *wd_q, const uint8_t *wd_s,
                          int weight_format, void *out, int out_dtype,
                          int B, int E, int k, int H, int I,
                          float *partials, size_t partials_bytes, void *stream,
                          const moed_tuning *tuning);

#ifdef __cplusplus
}
#endif

#endif /* MOEDECODE_H */
