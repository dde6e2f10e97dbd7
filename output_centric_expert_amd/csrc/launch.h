// Internal interface between the C-ABI layer and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moed {

// Launch-shape knobs. The defaults are the built-in choice; moed_set_tuning()
// can override them for sweeps.
struct Tuning {
    int gu_wpb = 4;     // gate/up: wavefronts per workgroup (1..4)
    int gu_pair = 1;    // exact-fit gate/up, MXFP4 at B > 1: two neighbouring neurons per wavefront
                        // (0 = one)
    int gu_order = 1;   // exact-fit gate/up at B > 1: neuron-block order with XCD-contiguous workgroups
                        // (slots sharing an expert meet in one L2) for MXFP8 (1) or both formats (2);
                        // 0 = slot-major
    int gu_exact = 1;   // gate/up (per-slot kernel): 1 = exact-fit kernel when a row is exactly 64*U
                        // chunks (U <= gu_umax), one neuron per wavefront, BF16 route, streaming
    int dn_wpb = 8;     // down: wavefronts per workgroup (1..8; at most 4 unstaged)
    int dn_stage = 1;   // down: 1 = copy a[b] into LDS once per workgroup (when it fits)
    int dn_group = 2;   // down inside moe_decode: 0 = one wavefront per output; 1 = expert-major
                        // MFMA tiles writing per-slot partials to the workspace, then a combine
                        // (each routed row decoded once per 64 slots); 2 = expert-major once B*k >= 2E
    int dn_tiles = 0;   // expert-major down: 16-slot tiles per pass over a row (1..4; 0 = as many
                        // as fit in 64 KiB of LDS)
    int gu_wide = 1;    // expert-grouped gate/up, MFMA path: 1 = weight rows read in 256-byte runs per
                        // row and moved to the operand layout through LDS; 0 = 128-byte tile slices
    int dn_split = 1;   // expert-major down, float32 a, wide loads: 1 = experts with 33..64 slots in one
                        // pass over their rows (two halves of 2 tiles), 0 = passes of 2 tiles
    int dn_rt = 2;      // expert-major down: 16-row tiles per wavefront (1 or 2; 2 lets each LDS read
                        // of the slots' a serve two MFMAs)
    int dn_wide = 1;    // expert-major down: 1 = weight rows read in 256-byte runs per row and moved to the
                        // operand layout through LDS (when I is a multiple of 512), 0 = 128-byte slices
    int gu_umax = 8;    // gate/up: max 16-byte chunks per lane per row held in flight
    int gu_group = 2;   // gate/up: 0 = one wavefront per (token, slot, neuron); 1 = expert-grouped
                        // MFMA tiles (rows decoded once per 16 slots); 2 = grouped once 4*B*k >= 3*E,
                        // or H >= 6144 with min(B*k, E)*ceil(I/64) >= 512
    int dn_umax = 8;    // down: max 16-byte chunks per lane held in flight
    int dn_lanegroups = 1; // down (staged): 1 = short rows share a wavefront among 2 or 4 slots
    int dn_onepass = 1; // down (staged, one output per wavefront): 1 = straight-line kernel when the
                        // token's slots form one group and a row is one chunk per lane
    int dn_pair = 1;    // one-pass down, MXFP4 at B > 1 (H even): 1 = two neighbouring outputs per
                        // wavefront sharing each read of a; 0 = one
    int gu_waves = 0;   // grouped gate/up with wide loads: wavefronts per workgroup (4 or 8; 8 = items of
                        // 128 neurons, the slots' x loaded once per 128 instead of 64 neurons);
                        // 0 = 8 once B*k >= 32*E
    int gu_grid = 512;  // grouped gate/up: at most this many workgroups walk the items of the routed
                        // experts (0 = one workgroup per item of all E experts, empty ones included)
    int dn_grid = 2048; // expert-major down: the same for its items
};

// Weight formats (moed_wformat in the C ABI).
constexpr int kMXFP8 = 0;   // E4M3 codes, one per byte
constexpr int kMXFP4 = 1;   // E2M1 codes, two per byte (element 2t in the low nibble of byte t)

struct GateUpArgs {
    const uint16_t* x;      // [B][H] bf16
    const int32_t* ids;     // [B][k]
    const uint8_t* wg_q;    // [E][I][H]
    const uint8_t* wg_s;    // [E][I][H/32]
    const uint8_t* wu_q;
    const uint8_t* wu_s;
    void* a;                // [B][k][I] f32 or bf16
    int B, E, k, H, I;
    int wfmt;               // kMXFP8 or kMXFP4 (codes [E][I][H/2])
};

struct DownArgs {
    const void* a;          // [B][k][I] f32 or bf16
    const int32_t* ids;     // [B][k]
    const float* w;         // [B][k]
    const uint8_t* wd_q;    // [E][H][I]
    const uint8_t* wd_s;    // [E][H][I/32]
    void* out;              // [B][H] f32 or bf16
    int B, E, k, H, I;
    float inv_cpr;          // 1 / (I/16), for the chunk -> (slot, offset) split
    int wfmt;               // kMXFP8 or kMXFP4 (codes [E][H][I/2])
    int split;              // expert-major down, float32 a: 1 = up to 4 tiles per pass in two halves
};

hipError_t launch_gate_up(const GateUpArgs& p, bool a_bf16, const Tuning& t, hipStream_t s);
hipError_t launch_gate_up_grouped(const GateUpArgs& p, bool a_bf16, const Tuning& t, hipStream_t s);
size_t gate_up_grouped_lds(int B, int k, int E, bool wide, int nw = 4);
hipError_t launch_down(const DownArgs& p, bool a_bf16, bool out_bf16, const Tuning& t, hipStream_t s);
// One-pass down (float32 a, streaming loads, 8 wavefronts per workgroup): k = groups * jb slots,
// rows of at most 64/groups chunks; hipErrorInvalidValue for a (jb, groups) it has no kernel for.
hipError_t launch_down_onepass(const DownArgs& p, int jb, int groups, bool out_bf16, int pair_wpb, dim3 grid, dim3 block,
                               size_t lds, hipStream_t s);
// Blocks form of the one-pass down (float32 a, cached loads, B*k >= E): each
// workgroup of 8 wavefronts takes kDownBlocks blocks of 8 outputs of one token;
// H must be a multiple of 8*kDownBlocks (hipErrorInvalidValue otherwise).
constexpr int kDownBlocks = 8;
hipError_t launch_down_blocks(const DownArgs& p, int jb, int groups, bool out_bf16, size_t lds, hipStream_t s);
hipError_t launch_bench_read(const void* src, size_t bytes, void* sink, hipStream_t s);
hipError_t launch_bench_copy(const void* src, void* dst, size_t bytes, hipStream_t s);
hipError_t launch_bench_read_cfg(const void* src, size_t bytes, void* sink, int unroll, int waves_per_group,
                                 int groups, hipStream_t s);
// Expert-major down (y: B*k*H float32 per-slot partials, then out).
hipError_t launch_down_grouped(const DownArgs& p, bool a_bf16, bool out_bf16, float* y, int max_tiles,
                               int row_tiles, bool wide, int grid_cap, hipStream_t s);
size_t down_grouped_lds(int B, int k, int E, bool a_bf16, int max_tiles, int row_tiles, bool wide);
// 0: does not fit
int down_grouped_tiles(int B, int k, int E, bool a_bf16, int requested, int row_tiles, bool wide);
// Router front-end (router.hip): top-k of float32 logits with renormalised
// softmax weights, plus shared-expert slots.
constexpr int kRouteMaxE = 2048;
constexpr int kRouteMaxK = 64;
hipError_t launch_route(const float* logits, int B, int E, int k, int n_shared, float routed_scale, int32_t* ids,
                        float* w, hipStream_t s);
// Opt-in input check (check.hip). Pointers not used by a step may be null:
// the gate/up step passes no down matrix and the down step no gate/up ones.
struct CheckArgs {
    const int32_t* ids;
    const uint8_t *wg_q, *wg_s, *wu_q, *wu_s, *wd_q, *wd_s;
    int B, E, k, H, I, wfmt;
};
// Bits of the check flag word.
constexpr uint32_t kCheckBadId = 1u;          // an expert id outside [0, E)
constexpr uint32_t kCheckNaN = 2u;            // a NaN code or scale in a routed expert's rows
constexpr uint32_t kCheckScaleGateUp = 4u;    // a routed gate/up block scale the grouped gate/up does not decode exactly
constexpr uint32_t kCheckScaleDown = 8u;      // a routed down block scale the expert-major down does not decode exactly
// Block-scale codes the large-batch kernels decode exactly (the scale folded
// into the BF16 conversion keeps every scaled value a normal, finite BF16).
constexpr int kExactScaleLoFP8 = 10, kExactScaleHiFP8 = 245;
constexpr int kExactScaleLoFP4 = 2, kExactScaleHiFP4 = 252;
hipError_t launch_check(const CheckArgs& c, uint32_t* flag, hipStream_t s);
constexpr int kMaxDevices = 64;               // devices the per-device tables hold
// Device address of the check flag word of the current device (a file-scope
// device array; its address is taken once per device).
hipError_t check_flag(uint32_t** flag);
// hipFuncAttributeMaxDynamicSharedMemorySize for `func`, set once per device.
hipError_t set_max_dynamic_lds(const void* func, int bytes);
hipError_t launch_selftest_decode(const uint8_t* codes, const uint8_t* scales, float* out, int n,
                                  int path, hipStream_t s);

}  // namespace moed
