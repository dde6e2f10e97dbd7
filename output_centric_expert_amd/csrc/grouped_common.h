// Helpers shared by the expert-grouped kernels (large decode batches): exact
// MXFP8 / MXFP4 -> BF16 decode with the block scale folded in (the MFMA A
// operand), the deterministic slot-list compaction, and the common launch
// shape (workgroups of 4 wavefronts, 16-row MFMA tiles, up to 4 tiles of 16
// slots per pass over a row).
#pragma once

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

// Block scales for the wide weight loads. The scale bytes of a row's MX blocks
// 16b .. 16b+15 (one "scale block": four 128-code groups of four blocks) are
// fetched with one 8-byte load per lane, two lanes per row: lane L holds bytes
// 8*(L % 2) .. +7 of row slot L / 2. Requested this way, a wavefront's scale
// loads touch each row's scale line once per 16 blocks instead of once per
// group and lane, which keeps their L2 requests well below the weight stream's
// (per-lane byte loads cost the grouped kernels 4-9% of their bandwidth). The
// lane that decodes block 4*gi + kb of row slot n (gi: group within the block)
// takes the byte from lane 2n + gi/2, dword gi % 2, byte kb, by ds_bpermute.
__device__ __forceinline__ u32x2 load_scale_block(const uint8_t* row_scales, int blk, int lane)
{
    return *reinterpret_cast<const u32x2*>(row_scales + 16 * (size_t)blk + 8 * (size_t)(lane % 2));
}

template <int GI>
__device__ __forceinline__ uint32_t block_scale_code(u32x2 sb, int row_slot, int kb)
{
    const uint32_t v = (GI & 1) ? sb.y : sb.x;
    const uint32_t d = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (2 * row_slot + GI / 2), (int)v);
    return (d >> (8 * kb)) & 255u;
}

template <int GI>
__device__ __forceinline__ float block_scale(u32x2 sb, int row_slot, int kb)
{
    return ue8m0_to_f32(block_scale_code<GI>(sb, row_slot, kb));
}

// Deterministic compaction: slots[0..count) = the indices t < n (in increasing
// order) with pred(ids[t]), stored as S (int, or uint16_t for n < 65536); with
// WIN, only those of rank lo .. lo+cap-1 are stored (at slots[rank - lo]).
// Returns the count of all of them. All threads of the workgroup (NW
// wavefronts) must call it. The ids of up to four 256-slot chunks are loaded
// together, so the list costs one round trip to L2 per 1024 slots.
//
// Windows of slots (the expert-major down once B*k > kSlotCap, the grouped
// gate/up once all B*k entries no longer fit in its LDS): at most kSlotCap
// slots of an expert are in LDS at a time, and an expert with more is taken in
// windows of kSlotCap (a multiple of the 16 slots of a tile, so each tile holds
// the same slots as with one list): an item is (expert, block, window), with as
// many windows per expert as the busiest routed expert needs (one unless an
// expert has more than kSlotCap).
constexpr int kSlotCap = 4096;
template <int NW = kGroupWaves, typename Pred, typename S = int, bool WIN = false>
__device__ __forceinline__ int compact_slots(int n, const int* ids, S* slots, int* wave_cnt, Pred pred, int lo = 0,
                                             int cap = 0)
{
    constexpr int kChunk = NW * kWave;
    constexpr int kBatch = 4;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    int total = 0;
    for (int base0 = 0; base0 < n; base0 += kBatch * kChunk) {
        int v[kBatch];
#pragma unroll
        for (int c = 0; c < kBatch; ++c) {
            const int t = base0 + c * kChunk + tid;
            v[c] = t < n ? ids[t] : 0;
        }
#pragma unroll
        for (int c = 0; c < kBatch; ++c) {
            const int base = base0 + c * kChunk;
            if (base >= n)                        // workgroup-uniform
                break;
            const int t = base + tid;
            const bool f = t < n && pred(v[c]);
            const unsigned long long m = __ballot(f);
            const int before = __popcll(m & ((1ull << lane) - 1ull));
            if (lane == 0)
                wave_cnt[w] = __popcll(m);
            __syncthreads();
            int off = total;
            for (int q = 0; q < w; ++q)
                off += wave_cnt[q];
            if constexpr (WIN) {
                const int rank = off + before;
                if (f && rank >= lo && rank - lo < cap)
                    slots[rank - lo] = (S)t;
            } else {
                if (f)
                    slots[off + before] = (S)t;
            }
            int sum = 0;
            for (int q = 0; q < NW; ++q)
                sum += wave_cnt[q];
            __syncthreads();
            total += sum;
        }
    }
    return total;
}

// Work list of the grouped kernels. Without it the grid has one workgroup
// per (expert, block) for all E experts, and a workgroup whose expert got no
// slot still pays for the slot compaction before it leaves -- at batch 64 of
// 256 experts most of the grid. With it, every workgroup builds the same list
// of the routed experts in its LDS and walks the items (routed-expert rank,
// block) with a stride of the grid size. Used when E <= kWorklistMaxE.
constexpr int kWorklistMaxE = 1024;

// LDS bytes of the work list: E marks and the list of routed experts (at
// most E).
inline size_t worklist_lds(int E)
{
    return E <= kWorklistMaxE ? ((size_t)2 * (size_t)E + 3) / 4 * 16 : 0;
}

// act[0..n) = the experts with at least one slot routed to them (ids in
// [0, E)), in increasing order; mark is E ints of scratch. Returns n. All
// threads of the workgroup must call it.
template <int NW = kGroupWaves>
__device__ __forceinline__ int routed_experts(int n_slots, const int* ids, int E, int* mark, int* act, int* wave_cnt)
{
    constexpr int kChunk = NW * kWave;
    const int tid = threadIdx.x;
    for (int t = tid; t < E; t += kChunk)
        mark[t] = 0;
    __syncthreads();
    for (int base = 0; base < n_slots; base += 4 * kChunk) {
        int v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {             // four ids per thread in flight at once
            const int t = base + c * kChunk + tid;
            v[c] = t < n_slots ? ids[t] : -1;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if ((unsigned)v[c] < (unsigned)E)
                mark[v[c]] = 1;                   // equal values: any order of the stores
    }
    __syncthreads();
    return compact_slots<NW>(E, mark, act, wave_cnt, [](int v) { return v != 0; });
}

// routed_experts, and the window count of the items: 1 when n_slots <= kSlotCap;
// otherwise the slots of each expert are counted with LDS atomic adds into mark
// (exact in any order) and the count is ceil(largest count / kSlotCap). All
// threads of the workgroup must call it.
template <int NW = kGroupWaves>
__device__ __forceinline__ int routed_experts_windows(int n_slots, const int* ids, int E, int* mark, int* act,
                                                      int* wave_cnt, int& nwin)
{
    constexpr int kChunk = NW * kWave;
    const int tid = threadIdx.x;
    const bool counted = n_slots > kSlotCap;      // else no expert can have more than one window
    for (int t = tid; t < E; t += kChunk)
        mark[t] = 0;
    __syncthreads();
    for (int base = 0; base < n_slots; base += 4 * kChunk) {
        int v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int t = base + c * kChunk + tid;
            v[c] = t < n_slots ? ids[t] : -1;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if ((unsigned)v[c] < (unsigned)E) {
                if (counted)
                    atomicAdd(&mark[v[c]], 1);
                else
                    mark[v[c]] = 1;
            }
    }
    __syncthreads();
    nwin = 1;
    if (!counted)
        return compact_slots<NW>(E, mark, act, wave_cnt, [](int v) { return v != 0; });
    int m = 0;
    for (int t = tid; t < E; t += kChunk)
        m = mark[t] > m ? mark[t] : m;
    for (int off = kWave / 2; off > 0; off >>= 1) {
        const int o = __shfl_xor(m, off);
        m = o > m ? o : m;
    }
    if ((tid & (kWave - 1)) == 0)
        wave_cnt[tid / kWave] = m;
    __syncthreads();
    int mx = 0;
    for (int q = 0; q < NW; ++q)
        mx = wave_cnt[q] > mx ? wave_cnt[q] : mx;
    __syncthreads();                              // wave_cnt is reused by the compaction
    nwin = mx > kSlotCap ? (mx + kSlotCap - 1) / kSlotCap : 1;
    return compact_slots<NW>(E, mark, act, wave_cnt, [](int v) { return v != 0; });
}

}  // namespace moed
