// C ABI of libmoedecode: argument checks, launch-shape choice, two launches.
// Everything here runs on the host; all arithmetic of the layer runs in the
// kernels of gate_up.hip and down.hip. No call keeps state between calls: the
// launch shape comes from the built-in table or from the caller's
// moed_tuning, passed with the call.
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <set>
#include <tuple>

#include "moedecode.h"
#include "launch.h"

static_assert(sizeof(moed::Tuning) <= sizeof(moed_tuning), "moed_tuning too small for the launch table");
static_assert(sizeof(moed::Tuning) % sizeof(int) == 0, "moed::Tuning holds ints only");

namespace {

thread_local int g_last_hip = 0;
constexpr uint32_t kTuningMagic = 0x6D6F6564u;   // "moed": marks an initialised moed_tuning

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline bool dtype_ok(int d) { return d == MOED_BF16 || d == MOED_F32; }

inline bool wformat_ok(int f) { return f == MOED_MXFP8 || f == MOED_MXFP4; }

int check_shape(int B, int E, int k, int H, int I)
{
    if (B < 0 || E < 1 || k < 1 || k > E)
        return MOED_ERR_SHAPE;
    if (H < 32 || I < 32 || (H % 32) != 0 || (I % 32) != 0)
        return MOED_ERR_SHAPE;
    const long long BK_I = (long long)B * k * I, B_H = (long long)B * H;
    if (BK_I >= (1LL << 31) || B_H >= (1LL << 31) || (long long)k * (I / 16) >= (1LL << 22))
        return MOED_ERR_SHAPE;
    return MOED_OK;
}

int hip_status(hipError_t e)
{
    if (e == hipSuccess)
        return MOED_OK;
    g_last_hip = (int)e;
    return MOED_ERR_HIP;
}

// The launch table of one call: the built-in choice (picked by sweeps on
// MI355X), or the caller's moed_tuning. Returns false for a moed_tuning that
// moed_tuning_init() did not fill.
bool pick(const moed_tuning* user, moed::Tuning* t)
{
    *t = moed::Tuning();
    if (!user)
        return true;
    if ((uint32_t)user->words[0] != kTuningMagic)
        return false;
    memcpy(static_cast<void*>(t), &user->words[1], sizeof(moed::Tuning));
    return true;
}

// Expert-grouped gate/up (each routed row read once per 16-slot tile) against
// the per-slot kernel (each row read once per slot), measured with uniform
// routing, k = 8, E = 128 and 256: the grouped kernel wins from about 0.75
// slots per expert at H = 2048 and 4096 (it loses at 0.5: 41 vs 30 us, 133 vs
// 122 us), and at H = 7168 from two tokens on (0.25 slots per expert: 256 vs
// 327 us), once its items (expert, 64 neurons) fill the 512 workgroup slots
// of the chip (one token: 47 vs 41 us). Hence the rule: grouped when
// 4*B*k >= 3*E, or when H >= 6144 and min(B*k, E)*ceil(I/64) >= 512 (H between
// 4096 and 6144 unmeasured). Its slot list (16-bit entries; past about 16000
// of them, windows of 4096) fits in 64 KiB of LDS with the x tiles (the wide
// loads add 32-64 KiB, within the 160 KiB of a workgroup) for B*k up to 65535.
bool use_grouped(const moed::Tuning& t, int B, int E, int k, int H, int I, int wfmt)
{
    (void)wfmt;                                   // both weight formats have a grouped kernel
    if ((long)B * k > 65535 || moed::gate_up_grouped_lds(B, k, E, false) > 65536 || t.gu_group == 0)
        return false;
    if (t.gu_group == 1)
        return true;
    const long long slots = (long long)B * k;
    const long long items = (slots < E ? slots : E) * ((I + 63) / 64);
    return 4 * slots >= 3LL * E || (H >= 6144 && items >= 512);
}

hipError_t gate_up_launch(const moed::GateUpArgs& p, bool a_bf16, const moed::Tuning& t, hipStream_t s)
{
    if (use_grouped(t, p.B, p.E, p.k, p.H, p.I, p.wfmt))
        return moed::launch_gate_up_grouped(p, a_bf16, t, s);
    return moed::launch_gate_up(p, a_bf16, t, s);
}

// Expert-major down: used inside moe_decode (which owns a workspace for the
// per-slot partials) once tokens share experts, about two or more slots per
// expert on average (measured crossovers at 1.5-2 slots per expert).
// The expert-major down's wide loads: rows of whole 256-byte steps and scale
// blocks (I a multiple of 512, the scale array at an 8-byte aligned base: its
// blocks are read as 8-byte pieces), both weight formats, unless dn_wide = 0;
// otherwise the 128-byte slices, which give the same floats.
bool down_wide(const moed::Tuning& t, int I, const uint8_t* wd_s)
{
    return I % 512 == 0 && t.dn_wide != 0 && ((uintptr_t)wd_s & 7u) == 0;
}

int pick_down_tiles(const moed::Tuning& t, int B, int E, int k, bool a_bf16, bool wide)
{
    if (t.dn_group == 0 || (t.dn_group == 2 && (long)B * k < 2L * E))
        return 0;
    return moed::down_grouped_tiles(B, k, E, a_bf16, t.dn_tiles, t.dn_rt, wide);
}

hipError_t down_launch(const moed::DownArgs& p, bool a_bf16, bool out_bf16, const moed::Tuning& t, float* y,
                       hipStream_t s)
{
    if (y) {
        const bool wide = down_wide(t, p.I, p.wd_s);
        if (int mt = pick_down_tiles(t, p.B, p.E, p.k, a_bf16, wide)) {
            moed::DownArgs q = p;
            q.split = t.dn_split;
            return moed::launch_down_grouped(q, a_bf16, out_bf16, y, mt, t.dn_rt, wide, t.dn_grid, s);
        }
    }
    return moed::launch_down(p, a_bf16, out_bf16, t, s);
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Opt-in input check (MOED_CHECK=1 in the environment, read on every call):
// a check kernel on the caller's stream, then a synchronisation and a read of
// its flag word, which lives in a file-scope device array (one per device,
// allocated with the code object). Nothing is allocated.
bool check_enabled()
{
    const char* v = getenv("MOED_CHECK");
    return v && v[0] == '1' && v[1] == '\0';
}

// grouped: the call takes the expert-grouped gate/up (its block scales are
// folded into the BF16 conversion); expert_down: the expert-major down (the
// same for the down scales).
int run_check(const moed::CheckArgs& c, bool grouped, bool expert_down, hipStream_t s)
{
    uint32_t* flag = nullptr;
    hipError_t err = moed::check_flag(&flag);
    uint32_t host = 0;
    if (err == hipSuccess)
        err = moed::launch_check(c, flag, s);
    if (err == hipSuccess)
        err = hipStreamSynchronize(s);
    if (err == hipSuccess)
        err = hipMemcpy(&host, flag, sizeof(host), hipMemcpyDeviceToHost);
    if (err != hipSuccess) {
        g_last_hip = (int)err;
        return MOED_ERR_HIP;
    }
    if (host & (moed::kCheckBadId | moed::kCheckNaN))
        return MOED_ERR_SHAPE;
    if ((grouped && (host & moed::kCheckScaleGateUp)) || (expert_down && (host & moed::kCheckScaleDown)))
        return MOED_ERR_SCALE;
    return MOED_OK;
}

moed::CheckArgs check_args(const int32_t* ids, const uint8_t* wg_q, const uint8_t* wg_s, const uint8_t* wu_q,
                           const uint8_t* wu_s, const uint8_t* wd_q, const uint8_t* wd_s, int B, int E, int k,
                           int H, int I, int wfmt)
{
    moed::CheckArgs c;
    c.ids = ids;
    c.wg_q = wg_q; c.wg_s = wg_s; c.wu_q = wu_q; c.wu_s = wu_s; c.wd_q = wd_q; c.wd_s = wd_s;
    c.B = B; c.E = E; c.k = k; c.H = H; c.I = I; c.wfmt = wfmt;
    return c;
}

moed::GateUpArgs gate_up_args(const void* x, const int32_t* ids, const uint8_t* wg_q,
                              const uint8_t* wg_s, const uint8_t* wu_q, const uint8_t* wu_s,
                              int wfmt, void* a, int B, int E, int k, int H, int I)
{
    moed::GateUpArgs p;
    p.x = static_cast<const uint16_t*>(x);
    p.ids = ids;
    p.wg_q = wg_q; p.wg_s = wg_s; p.wu_q = wu_q; p.wu_s = wu_s;
    p.a = a;
    p.B = B; p.E = E; p.k = k; p.H = H; p.I = I;
    p.wfmt = wfmt;
    return p;
}

moed::DownArgs down_args(const void* a, const int32_t* ids, const float* w, const uint8_t* wd_q,
                         const uint8_t* wd_s, int wfmt, void* out, int B, int E, int k, int H, int I)
{
    moed::DownArgs p;
    p.a = a; p.ids = ids; p.w = w; p.wd_q = wd_q; p.wd_s = wd_s; p.out = out;
    p.B = B; p.E = E; p.k = k; p.H = H; p.I = I;
    p.inv_cpr = 1.0f / (float)(I / 16);
    p.wfmt = wfmt;
    p.split = 0;
    return p;
}

// Both steps of the layer on `s`, arguments already checked; `workspace`
// holds the intermediate, then (256-byte aligned) the per-slot partials.
int layer(const void* x, const int32_t* topk_ids, const float* topk_w, const uint8_t* wg_q, const uint8_t* wg_s,
          const uint8_t* wu_q, const uint8_t* wu_s, const uint8_t* wd_q, const uint8_t* wd_s, int weight_format,
          void* out, int out_dtype, int inter_dtype, int B, int E, int k, int H, int I, void* workspace,
          const moed::Tuning& t, hipStream_t s)
{
    const bool a_bf16 = inter_dtype == MOED_BF16;
    if (check_enabled()) {
        const bool expert_down = pick_down_tiles(t, B, E, k, a_bf16, down_wide(t, I, wd_s)) != 0;
        if (int st = run_check(check_args(topk_ids, wg_q, wg_s, wu_q, wu_s, wd_q, wd_s, B, E, k, H, I, weight_format),
                               use_grouped(t, B, E, k, H, I, weight_format), expert_down, s))
            return st;
    }
    int st = hip_status(gate_up_launch(
        gate_up_args(x, topk_ids, wg_q, wg_s, wu_q, wu_s, weight_format, workspace, B, E, k, H, I), a_bf16, t, s));
    if (st)
        return st;
    const size_t inter = (size_t)B * (size_t)k * (size_t)I * (a_bf16 ? 2u : 4u);
    float* partials = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + align256(inter));
    return hip_status(down_launch(
        down_args(workspace, topk_ids, topk_w, wd_q, wd_s, weight_format, out, B, E, k, H, I), a_bf16,
        out_dtype == MOED_BF16, t, partials, s));
}

// Scratch of moe_decode_noalloc(): the workspace (intermediate, then the
// per-slot partials) in a file-scope device array, one per device, held until
// the process ends. In host code `scratch` names a host-side stand-in, not the
// device memory: host code only ever uses the address hipGetSymbolAddress
// gives for the current device, taken once per device on its first call.
constexpr size_t kScratchBytes = (size_t)32 << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

hipError_t scratch_address(void** out)
{
    static std::mutex mu;
    static void* addr[moed::kMaxDevices] = {};
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return err;
    if (dev < 0 || dev >= moed::kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess)
            return err;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

size_t moed_workspace_bytes(int B, int k, int H, int I, int inter_dtype)
{
    if (B < 0 || k < 1 || H < 1 || I < 1 || !dtype_ok(inter_dtype))
        return 0;
    const size_t inter = (size_t)B * (size_t)k * (size_t)I * (inter_dtype == MOED_F32 ? 4u : 2u);
    const size_t partials = (size_t)B * (size_t)k * (size_t)H * 4u;
    return B == 0 ? 0 : align256(inter) + partials;
}

int moe_decode_gate_up_tuned(const void* x, const int32_t* topk_ids, const uint8_t* wg_q, const uint8_t* wg_s,
                             const uint8_t* wu_q, const uint8_t* wu_s, int weight_format, void* a, int inter_dtype,
                             int B, int E, int k, int H, int I, void* stream, const moed_tuning* tuning)
{
    if (int st = check_shape(B, E, k, H, I))
        return st;
    if (!dtype_ok(inter_dtype) || !wformat_ok(weight_format))
        return MOED_ERR_DTYPE;
    moed::Tuning t;
    if (!pick(tuning, &t))
        return MOED_ERR_TUNING;
    if (B == 0)
        return MOED_OK;
    if (!x || !topk_ids || !wg_q || !wg_s || !wu_q || !wu_s || !a)
        return MOED_ERR_NULL;
    if (!aligned16(x) || !aligned16(wg_q) || !aligned16(wu_q) || !aligned16(a))
        return MOED_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (check_enabled()) {
        if (int st = run_check(check_args(topk_ids, wg_q, wg_s, wu_q, wu_s, nullptr, nullptr, B, E, k, H, I,
                                          weight_format),
                               use_grouped(t, B, E, k, H, I, weight_format), false, s))
            return st;
    }
    return hip_status(gate_up_launch(gate_up_args(x, topk_ids, wg_q, wg_s, wu_q, wu_s, weight_format, a,
                                                  B, E, k, H, I),
                                     inter_dtype == MOED_BF16, t, s));
}

int moe_decode_gate_up(const void* x, const int32_t* topk_ids, const uint8_t* wg_q, const uint8_t* wg_s,
                       const uint8_t* wu_q, const uint8_t* wu_s, int weight_format, void* a, int inter_dtype,
                       int B, int E, int k, int H, int I, void* stream)
{
    return moe_decode_gate_up_tuned(x, topk_ids, wg_q, wg_s, wu_q, wu_s, weight_format, a, inter_dtype, B, E, k, H,
                                    I, stream, nullptr);
}

int moe_decode_down_tuned(const void* a, int inter_dtype, const int32_t* topk_ids, const float* topk_w,
                          const uint8_t* wd_q, const uint8_t* wd_s, int weight_format, void* out, int out_dtype,
                          int B, int E, int k, int H, int I, float* partials, size_t partials_bytes, void* stream,
                          const moed_tuning* tuning)
{
    if (int st = check_shape(B, E, k, H, I))
        return st;
    if (!dtype_ok(inter_dtype) || !dtype_ok(out_dtype) || !wformat_ok(weight_format))
        return MOED_ERR_DTYPE;
    moed::Tuning t;
    if (!pick(tuning, &t))
        return MOED_ERR_TUNING;
    if (B == 0)
        return MOED_OK;
    if (!a || !topk_ids || !topk_w || !wd_q || !wd_s || !out)
        return MOED_ERR_NULL;
    if (partials && partials_bytes < (size_t)B * (size_t)k * (size_t)H * 4u)
        return MOED_ERR_WORKSPACE;
    if (!aligned16(a) || !aligned16(wd_q) || (partials && !aligned16(partials)))
        return MOED_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool a_bf16 = inter_dtype == MOED_BF16;
    if (check_enabled()) {
        const bool expert_down =
            partials && pick_down_tiles(t, B, E, k, a_bf16, down_wide(t, I, wd_s)) != 0;
        if (int st = run_check(check_args(topk_ids, nullptr, nullptr, nullptr, nullptr, wd_q, wd_s, B, E, k, H, I,
                                          weight_format),
                               false, expert_down, s))
            return st;
    }
    return hip_status(down_launch(down_args(a, topk_ids, topk_w, wd_q, wd_s, weight_format, out, B, E, k, H, I),
                                  a_bf16, out_dtype == MOED_BF16, t, partials, s));
}

int moe_decode_down(const void* a, int inter_dtype, const int32_t* topk_ids, const float* topk_w,
                    const uint8_t* wd_q, const uint8_t* wd_s, int weight_format, void* out, int out_dtype,
                    int B, int E, int k, int H, int I, float* partials, size_t partials_bytes, void* stream)
{
    return moe_decode_down_tuned(a, inter_dtype, topk_ids, topk_w, wd_q, wd_s, weight_format, out, out_dtype, B, E,
                                 k, H, I, partials, partials_bytes, stream, nullptr);
}

int moe_decode_tuned(const void* x, const int32_t* topk_ids, const float* topk_w, const uint8_t* wg_q,
                     const uint8_t* wg_s, const uint8_t* wu_q, const uint8_t* wu_s, const uint8_t* wd_q,
                     const uint8_t* wd_s, int weight_format, void* out, int out_dtype, int inter_dtype, int B, int E,
                     int k, int H, int I, void* workspace, size_t workspace_bytes, void* stream,
                     const moed_tuning* tuning)
{
    if (int st = check_shape(B, E, k, H, I))
        return st;
    if (!dtype_ok(inter_dtype) || !dtype_ok(out_dtype) || !wformat_ok(weight_format))
        return MOED_ERR_DTYPE;
    moed::Tuning t;
    if (!pick(tuning, &t))
        return MOED_ERR_TUNING;
    if (B == 0)
        return MOED_OK;
    if (!x || !topk_ids || !topk_w || !wg_q || !wg_s || !wu_q || !wu_s || !wd_q || !wd_s || !out || !workspace)
        return MOED_ERR_NULL;
    if (workspace_bytes < moed_workspace_bytes(B, k, H, I, inter_dtype))
        return MOED_ERR_WORKSPACE;
    if (!aligned16(x) || !aligned16(wg_q) || !aligned16(wu_q) || !aligned16(wd_q) || !aligned16(workspace))
        return MOED_ERR_ALIGN;
    return layer(x, topk_ids, topk_w, wg_q, wg_s, wu_q, wu_s, wd_q, wd_s, weight_format, out, out_dtype, inter_dtype,
                 B, E, k, H, I, workspace, t, static_cast<hipStream_t>(stream));
}

int moe_decode(const void* x, const int32_t* topk_ids, const float* topk_w, const uint8_t* wg_q,
               const uint8_t* wg_s, const uint8_t* wu_q, const uint8_t* wu_s, const uint8_t* wd_q,
               const uint8_t* wd_s, int weight_format, void* out, int out_dtype, int inter_dtype, int B, int E, int k,
               int H, int I, void* workspace, size_t workspace_bytes, void* stream)
{
    return moe_decode_tuned(x, topk_ids, topk_w, wg_q, wg_s, wu_q, wu_s, wd_q, wd_s, weight_format, out, out_dtype,
                            inter_dtype, B, E, k, H, I, workspace, workspace_bytes, stream, nullptr);
}

int moe_decode_noalloc(const void* x, const int32_t* topk_ids, const float* topk_w, const uint8_t* wg_q,
                       const uint8_t* wg_s, const uint8_t* wu_q, const uint8_t* wu_s, const uint8_t* wd_q,
                       const uint8_t* wd_s, int weight_format, void* out, int out_dtype, int inter_dtype, int B,
                       int E, int k, int H, int I, void* stream)
{
    if (int st = check_shape(B, E, k, H, I))
        return st;
    if (!dtype_ok(inter_dtype) || !dtype_ok(out_dtype) || !wformat_ok(weight_format))
        return MOED_ERR_DTYPE;
    if (B == 0)
        return MOED_OK;
    if (!x || !topk_ids || !topk_w || !wg_q || !wg_s || !wu_q || !wu_s || !wd_q || !wd_s || !out)
        return MOED_ERR_NULL;
    if (moed_workspace_bytes(B, k, H, I, inter_dtype) > kScratchBytes)
        return MOED_ERR_WORKSPACE;
    if (!aligned16(x) || !aligned16(wg_q) || !aligned16(wu_q) || !aligned16(wd_q))
        return MOED_ERR_ALIGN;
    void* ws = nullptr;
    if (int st = hip_status(scratch_address(&ws)))
        return st;
    return layer(x, topk_ids, topk_w, wg_q, wg_s, wu_q, wu_s, wd_q, wd_s, weight_format, out, out_dtype, inter_dtype,
                 B, E, k, H, I, ws, moed::Tuning(), static_cast<hipStream_t>(stream));
}

int moe_route(const float* logits, int B, int E, int k, int n_shared, float routed_scale, int32_t* topk_ids,
              float* topk_w, void* stream)
{
    if (B < 0 || E < 1 || E > moed::kRouteMaxE || k < 1 || k > E || k > moed::kRouteMaxK || n_shared < 0)
        return MOED_ERR_SHAPE;
    if ((long long)B * (k + n_shared) >= (1LL << 31) || (long long)B * E >= (1LL << 31))
        return MOED_ERR_SHAPE;
    if (B == 0)
        return MOED_OK;
    if (!logits || !topk_ids || !topk_w)
        return MOED_ERR_NULL;
    return hip_status(moed::launch_route(logits, B, E, k, n_shared, routed_scale, topk_ids, topk_w,
                                         static_cast<hipStream_t>(stream)));
}

int moed_selftest_decode(const uint8_t* codes, const uint8_t* scales, float* out, int n, int path,
                         void* stream)
{
    if (n < 0 || path < 0 || path > 5)
        return MOED_ERR_SHAPE;
    if (n == 0)
        return MOED_OK;
    if (!codes || !scales || !out)
        return MOED_ERR_NULL;
    return hip_status(moed::launch_selftest_decode(codes, scales, out, n, path, static_cast<hipStream_t>(stream)));
}

int moed_bench_read(const void* src, size_t bytes, void* sink, size_t sink_bytes, void* stream)
{
    if (bytes == 0)
        return MOED_OK;
    if (!src || !sink)
        return MOED_ERR_NULL;
    if (bytes % 16 != 0 || sink_bytes < 4096)
        return MOED_ERR_SHAPE;
    if (!aligned16(src))
        return MOED_ERR_ALIGN;
    return hip_status(moed::launch_bench_read(src, bytes, sink, static_cast<hipStream_t>(stream)));
}

int moed_bench_read_cfg(const void* src, size_t bytes, void* sink, size_t sink_bytes, int unroll,
                        int waves_per_group, int groups, void* stream)
{
    if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8 && unroll != 16)
        return MOED_ERR_SHAPE;
    if (waves_per_group < 1 || waves_per_group > 16 || groups < 0)
        return MOED_ERR_SHAPE;
    if (bytes == 0)
        return MOED_OK;
    if (!src || !sink)
        return MOED_ERR_NULL;
    if (bytes % 16 != 0 || sink_bytes < 4096)
        return MOED_ERR_SHAPE;
    if (!aligned16(src))
        return MOED_ERR_ALIGN;
    return hip_status(moed::launch_bench_read_cfg(src, bytes, sink, unroll, waves_per_group, groups,
                                                  static_cast<hipStream_t>(stream)));
}

int moed_bench_copy(const void* src, void* dst, size_t bytes, void* stream)
{
    if (bytes == 0)
        return MOED_OK;
    if (!src || !dst)
        return MOED_ERR_NULL;
    if (bytes % 16 != 0)
        return MOED_ERR_SHAPE;
    if (!aligned16(src) || !aligned16(dst))
        return MOED_ERR_ALIGN;
    return hip_status(moed::launch_bench_copy(src, dst, bytes, static_cast<hipStream_t>(stream)));
}

const char* moed_status_string(int status)
{
    switch (status) {
    case MOED_OK: return "MOED_OK";
    case MOED_ERR_NULL: return "MOED_ERR_NULL: a required pointer is NULL";
    case MOED_ERR_SHAPE: return "MOED_ERR_SHAPE: invalid or unsupported sizes";
    case MOED_ERR_DTYPE: return "MOED_ERR_DTYPE: unknown dtype";
    case MOED_ERR_WORKSPACE: return "MOED_ERR_WORKSPACE: workspace too small";
    case MOED_ERR_ALIGN: return "MOED_ERR_ALIGN: pointer not 16-byte aligned";
    case MOED_ERR_HIP: return "MOED_ERR_HIP: HIP launch failed";
    case MOED_ERR_SCALE: return "MOED_ERR_SCALE: a routed block scale outside the range the large-batch kernels decode exactly";
    case MOED_ERR_TUNING: return "MOED_ERR_TUNING: moed_tuning not filled by moed_tuning_init";
    default: return "unknown moed_status";
    }
}

int moed_last_hip_error(void) { return g_last_hip; }

int moed_tuning_init(moed_tuning* out, const char* spec)
{
    if (!out)
        return MOED_ERR_NULL;
    moed::Tuning t;
    if (spec && strlen(spec) >= 512)
        return MOED_ERR_SHAPE;
    char buf[512] = {0};
    if (spec)
        strncpy(buf, spec, sizeof buf - 1);
    char* save = nullptr;
    for (char* tok = strtok_r(buf, ",", &save); tok; tok = strtok_r(nullptr, ",", &save)) {
        char* eq = strchr(tok, '=');
        if (!eq)
            return MOED_ERR_SHAPE;
        *eq = 0;
        char* end = nullptr;
        const long v = strtol(eq + 1, &end, 10);
        if (!end || *end)
            return MOED_ERR_SHAPE;
        if (!strcmp(tok, "gu_wpb") && v >= 1 && v <= 4) t.gu_wpb = (int)v;
        else if (!strcmp(tok, "dn_wpb") && v >= 1 && v <= 8) t.dn_wpb = (int)v;
        else if (!strcmp(tok, "dn_stage") && (v == 0 || v == 1)) t.dn_stage = (int)v;
        else if (!strcmp(tok, "dn_group") && v >= 0 && v <= 2) t.dn_group = (int)v;
        else if (!strcmp(tok, "dn_tiles") && v >= 0 && v <= 4) t.dn_tiles = (int)v;
        else if (!strcmp(tok, "dn_rt") && v >= 1 && v <= 2) t.dn_rt = (int)v;
        else if (!strcmp(tok, "dn_wide") && (v == 0 || v == 1)) t.dn_wide = (int)v;
        else if (!strcmp(tok, "gu_wide") && v >= 0 && v <= 1) t.gu_wide = (int)v;
        else if (!strcmp(tok, "gu_order") && v >= 0 && v <= 2) t.gu_order = (int)v;
        else if (!strcmp(tok, "gu_pair") && (v == 0 || v == 1)) t.gu_pair = (int)v;
        else if (!strcmp(tok, "gu_umax") && v >= 1 && v <= 8) t.gu_umax = (int)v;
        else if (!strcmp(tok, "gu_group") && v >= 0 && v <= 2) t.gu_group = (int)v;
        else if (!strcmp(tok, "dn_umax") && v >= 1 && v <= 8) t.dn_umax = (int)v;
        else if (!strcmp(tok, "dn_lanegroups") && (v == 0 || v == 1)) t.dn_lanegroups = (int)v;
        else if (!strcmp(tok, "dn_onepass") && (v == 0 || v == 1)) t.dn_onepass = (int)v;
        else if (!strcmp(tok, "dn_pair") && (v == 0 || v == 1)) t.dn_pair = (int)v;
        else if (!strcmp(tok, "dn_split") && (v == 0 || v == 1)) t.dn_split = (int)v;
        else if (!strcmp(tok, "gu_exact") && (v == 0 || v == 1)) t.gu_exact = (int)v;
        else if (!strcmp(tok, "gu_waves") && (v == 0 || v == 4 || v == 8)) t.gu_waves = (int)v;
        else if (!strcmp(tok, "gu_grid") && v >= 0 && v <= 65536) t.gu_grid = (int)v;
        else if (!strcmp(tok, "dn_grid") && v >= 0 && v <= 65536) t.dn_grid = (int)v;
        else return MOED_ERR_SHAPE;
    }
    memset(out, 0, sizeof(*out));
    out->words[0] = (int32_t)kTuningMagic;
    memcpy(&out->words[1], &t, sizeof(t));
    return MOED_OK;
}

}  // extern "C"
