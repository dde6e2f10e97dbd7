"""GPU parity: the HIP path (through the C-ABI) against the float64 CPU oracle.

Gate (the tolerance the layer is specified to): with float32 outputs,
max |gpu - oracle| <= 2e-3 * rms(oracle) over the compared outputs. BF16
outputs must be the round-to-nearest-even of the float32 result, bit for bit,
and within that bound plus half a bf16 ulp of the oracle value.

The five decode workloads run in the launch configuration the benchmark
times, and every output of every token is compared with the oracle; the two
large ones also on the pure output-centric kernel pair, plus properties that
hold at any size (determinism, finiteness, batch = concatenation of tokens).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from output_centric_expert_amd import moedecode as md
from output_centric_expert_amd import synth

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    md.load()                                   # raises if the HIP library is missing
    oracle.build(force=False)
    yield
    md.set_default_tuning(None)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def layer(shape, seed=None, **kw):
    return synth.make_layer(shape, seed=seed, device="cuda", **kw)


def small(B, E, k, H, I, seed=0, zipf=0.0):
    return layer(synth.LayerShape(f"s{B}_{E}_{k}_{H}_{I}", B, E, k, H, I, zipf), seed=seed)


def run(L, out_dtype=torch.float32, inter_dtype=torch.float32, ids=None, w=None, x=None):
    xd, idd, wd = md.layer_device_inputs(L)
    if ids is not None:
        idd = torch.as_tensor(ids, dtype=torch.int32).cuda().contiguous()
    if w is not None:
        wd = torch.as_tensor(w, dtype=torch.float32).cuda().contiguous()
    if x is not None:
        xd = x
    out = md.moe_decode(xd, idd, wd, L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s,
                        out_dtype=out_dtype, inter_dtype=inter_dtype)
    torch.cuda.synchronize()
    return out


def oracle_tokens(L, tokens, ids=None, w=None, wformat="mxfp8"):
    """Oracle output (and intermediate) for a subset of tokens, from the same weight bytes."""
    ids = L.ids if ids is None else np.asarray(ids, np.int32)
    w = L.w if w is None else np.asarray(w, np.float32)
    ids_t = ids[tokens]
    sel = sorted({int(e) for e in ids_t.ravel() if 0 <= e < L.shape.E})
    remap = np.full(L.shape.E, -1, np.int64)
    remap[sel] = np.arange(len(sel))
    ids_c = np.where((ids_t >= 0) & (ids_t < L.shape.E), remap[np.clip(ids_t, 0, L.shape.E - 1)], -1)
    idx = torch.tensor(sel if sel else [0], device=L.wg_q.device)
    pick = lambda t: t.index_select(0, idx).cpu()
    return oracle.moe_decode(np.ascontiguousarray(L.x[tokens]), np.ascontiguousarray(ids_c.astype(np.int32)),
                             np.ascontiguousarray(w[tokens]), pick(L.wg_q), pick(L.wg_s), pick(L.wu_q),
                             pick(L.wu_s), pick(L.wd_q), pick(L.wd_s), return_inter=True, wformat=wformat)


def check_f32(gpu_out, ref, label, tol=TOL):
    g = gpu_out.double().cpu().numpy() if torch.is_tensor(gpu_out) else gpu_out
    rms = math.sqrt(float(np.mean(ref ** 2)))
    err = float(np.max(np.abs(g - ref)))
    say(f"[{label}] max|err| = {err:.3e}  rms = {rms:.3e}  ratio = {err / rms:.3e}")
    assert np.isfinite(g).all()
    assert err <= tol * rms, f"{label}: max|err|/rms = {err / rms:.3e} > {tol}"
    return err / rms


def bf16_ulp(v):
    v = np.abs(v)
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -126)))
    return np.exp2(e - 7)


def check_bf16(gpu_bf16, gpu_f32, ref, label):
    rne = gpu_f32.cpu().to(torch.bfloat16)                     # library RNE of our f32 result
    assert torch.equal(gpu_bf16.cpu().view(torch.int16), rne.view(torch.int16)), f"{label}: bf16 != RNE(f32)"
    g = gpu_bf16.double().cpu().numpy()
    rms = math.sqrt(float(np.mean(ref ** 2)))
    assert np.all(np.abs(g - ref) <= TOL * rms + 0.5 * bf16_ulp(ref)), label


# --------------------------------------------------------------------------------------
# decode self-test: every E4M3 code, both in-register routes, bit for bit
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("path", [0, 1, 2])
def test_decode_all_codes_bit_exact(path):
    scales = [127, 100, 120, 126, 128, 134, 147]
    codes = np.tile(np.arange(256, dtype=np.uint8), len(scales))
    sc = np.repeat(np.array(scales, np.uint8), 256)
    got = md.moed_selftest_decode(torch.from_numpy(codes).cuda(), torch.from_numpy(sc).cuda(), path).cpu().numpy()
    for t in range(codes.size):
        ref = oracle.e4m3_value(int(codes[t])) * oracle.ue8m0_value(int(sc[t]))
        if math.isnan(ref):
            assert math.isnan(got[t]), (path, hex(codes[t]), sc[t])
        else:
            r32 = np.float32(ref)
            assert float(r32) == ref                     # exactly representable
            assert got[t] == r32 and np.signbit(got[t]) == np.signbit(r32), (path, hex(codes[t]), sc[t], got[t], ref)


def test_decode_nan_scale():
    codes = torch.tensor([0x38, 0x00, 0x81], dtype=torch.uint8).cuda()
    sc = torch.full((3,), 255, dtype=torch.uint8).cuda()
    for path in (0, 1, 2):
        assert torch.isnan(md.moed_selftest_decode(codes, sc, path)).all()


# --------------------------------------------------------------------------------------
# the five decode workloads
# --------------------------------------------------------------------------------------

FULL = ["tiny_B1_E8_k2_H256_I128", "wide_B1_E128_k8_H2048_I768", "batch_B8_E128_k8_H2048_I768"]
LARGE = ["batch_B32_E128_k8_H4096_I1536", "skewed_B64_E256_k8_H7168_I2048"]


@pytest.mark.parametrize("name", FULL)
def test_workload_full_parity(name):
    say(f"workload {name}: full parity")
    L = layer(name)
    ref, a_ref = oracle_tokens(L, list(range(L.shape.B)))
    out32 = run(L, torch.float32)
    check_f32(out32, ref, name)
    out16 = run(L, torch.bfloat16)
    check_bf16(out16, out32, ref, name)
    # the gate/up step alone against the oracle's intermediate
    x, ids, _ = md.layer_device_inputs(L)
    a = md.inter_to_bki(md.moe_decode_gate_up(x, ids, L.wg_q, L.wg_s, L.wu_q, L.wu_s))
    torch.cuda.synchronize()
    check_f32(a.reshape(L.shape.B, -1), a_ref.reshape(L.shape.B, -1), name + " a")


@pytest.mark.parametrize("name", LARGE)
def test_workload_large_full_parity(name):
    """The two large workloads, every output of every token against the oracle (run on all
    tokens, all host threads), on the default kernel pair (expert-grouped gate/up, expert-major
    down) and on the pure output-centric pair (per-slot gate/up, per-output down); plus
    determinism, the bf16 store, the intermediate, and batch = concatenation of tokens."""
    say(f"workload {name}: full parity, both kernel pairs")
    L = layer(name)
    B = L.shape.B
    out32 = run(L, torch.float32)
    out32b = run(L, torch.float32)
    assert torch.equal(out32, out32b), "not deterministic"
    assert torch.isfinite(out32).all()
    say(f"workload {name}: oracle on all {B} tokens")
    ref, a_ref = oracle_tokens(L, list(range(B)))
    check_f32(out32, ref, name + " default pair")
    out16 = run(L, torch.bfloat16)
    check_bf16(out16, out32, ref, name + " default pair")
    x, ids, w = md.layer_device_inputs(L)
    a = md.inter_to_bki(md.moe_decode_gate_up(x, ids, L.wg_q, L.wg_s, L.wu_q, L.wu_s))
    torch.cuda.synchronize()
    check_f32(a.reshape(B, -1), a_ref.reshape(B, -1), name + " default a")
    with md.tuned("gu_group=0,dn_group=0"):
        oc32 = run(L, torch.float32)
        check_f32(oc32, ref, name + " output-centric pair")
        oc16 = run(L, torch.bfloat16)
        check_bf16(oc16, oc32, ref, name + " output-centric pair")
        a0 = md.inter_to_bki(md.moe_decode_gate_up(x, ids, L.wg_q, L.wg_s, L.wu_q, L.wu_s))
        torch.cuda.synchronize()
        check_f32(a0.reshape(B, -1), a_ref.reshape(B, -1), name + " output-centric a")
    # batch = concatenation of single-token calls, bit for bit, on each kernel pair
    # (the per-slot/per-output and the grouped kernels accumulate in different orders)
    for spec in ("gu_group=0,dn_group=0", "gu_group=1,dn_group=1"):
        with md.tuned(spec):
            full = run(L, torch.float32)
            for b in (0, B // 3, B - 1):
                one = md.moe_decode(x[b:b + 1].contiguous(), ids[b:b + 1].contiguous(), w[b:b + 1].contiguous(),
                                    L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s, out_dtype=torch.float32)
                torch.cuda.synchronize()
                assert torch.equal(one[0], full[b]), spec


@pytest.mark.parametrize("name", FULL)
def test_bf16_intermediate_variant_reported(name):
    """The FP32-accumulate path that stores BF16 intermediates: error reported, not gated."""
    L = layer(name)
    ref, _ = oracle_tokens(L, list(range(L.shape.B)))
    out = run(L, torch.float32, inter_dtype=torch.bfloat16)
    g = out.double().cpu().numpy()
    rms = math.sqrt(float(np.mean(ref ** 2)))
    ratio = float(np.max(np.abs(g - ref))) / rms
    say(f"[{name}] bf16-intermediate max|err|/rms = {ratio:.3e}")
    assert np.isfinite(g).all() and ratio < 5e-2


# --------------------------------------------------------------------------------------
# ragged shapes, multi-pass rows, tuning variants
# --------------------------------------------------------------------------------------

SHAPES = [
    (1, 4, 2, 32, 32),        # one MX block per row
    (3, 6, 3, 96, 160),       # rows shorter than a wave; k*I/16 not a multiple of 64
    (2, 5, 5, 2080, 96),      # k = E; 130 chunks per row: a ragged second chunk per lane
    (2, 3, 2, 8224, 64),      # 514 chunks per row: more than 8 per lane -> two passes
    (2, 8, 4, 128, 2080),     # down: k*I/16 = 520 -> two passes
    (5, 16, 1, 64, 1056),     # k = 1
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}_E{}_k{}_H{}_I{}".format(*s))
def test_ragged_shapes(shape):
    B, E, k, H, I = shape
    L = small(B, E, k, H, I, seed=sum(shape))
    ref, a_ref = oracle_tokens(L, list(range(B)))
    check_f32(run(L), ref, f"ragged {shape}")
    x, ids, _ = md.layer_device_inputs(L)
    a = md.inter_to_bki(md.moe_decode_gate_up(x, ids, L.wg_q, L.wg_s, L.wu_q, L.wu_s))
    torch.cuda.synchronize()
    check_f32(a.reshape(B, -1), a_ref.reshape(B, -1), f"ragged a {shape}")
    # the down step alone on the gate/up step's buffer gives the layer
    a_ws = md.moe_decode_gate_up(x, ids, L.wg_q, L.wg_s, L.wu_q, L.wu_s)
    _, idd, wd = md.layer_device_inputs(L)
    out = md.moe_decode_down(a_ws, idd, wd, L.wd_q, L.wd_s, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_f32(out, ref, f"ragged steps {shape}")


@pytest.mark.parametrize("spec", ["gu_wpb=1,dn_wpb=1", "gu_wpb=2,dn_wpb=2", "gu_umax=1,dn_umax=1",
                                  "gu_umax=3,dn_umax=5", "gu_group=1", "gu_group=0", "dn_stage=0",
                                  "dn_group=1", "gu_group=1,dn_group=1", "dn_group=0", "dn_stage=0,dn_wpb=3",
                                  "dn_wpb=5", "dn_lanegroups=0", "dn_lanegroups=1,dn_umax=1",
                                  "dn_onepass=0", "dn_onepass=0,dn_umax=2,dn_wpb=3", "dn_onepass=0,dn_wpb=5",
                                  "gu_exact=0", "gu_exact=0,gu_umax=1,gu_wpb=3", "gu_exact=0,dn_onepass=0",
                                  "gu_grid=0,dn_grid=0,gu_group=1,dn_group=1", "gu_grid=3,dn_grid=5,gu_group=1,dn_group=1",
                                  "dn_group=1,dn_wide=0", "dn_group=1,dn_wide=1,dn_tiles=3", "gu_order=0", "gu_order=2"])
def test_tuning_variants_keep_parity(spec):
    # B=1; tokens sharing experts (B*k >= E); B*k < E at B > 1 (two outputs per down wavefront)
    for shape in [(1, 128, 8, 2048, 768), (3, 6, 3, 96, 160), (2, 3, 2, 8224, 64), (4, 40, 4, 1024, 256)]:
        L = small(*shape, seed=3)
        ref, _ = oracle_tokens(L, list(range(shape[0])))
        md.set_default_tuning(spec)
        try:
            check_f32(run(L), ref, f"{spec} {shape}")
        finally:
            md.set_default_tuning(None)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_unaligned_out_in_the_expert_major_down(out_dtype):
    """Tokens sharing experts (B*k >= 2E: expert-major down and the combine launch): an `out`
    that starts one element past an aligned address gives the same bits as an aligned one."""
    L = small(8, 6, 3, 256, 128, seed=17)
    x, ids, w = md.layer_device_inputs(L)
    B, H = 8, 256
    ref = md.moe_decode(x, ids, w, L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s, out_dtype=out_dtype)
    buf = torch.full((B * H + 1,), float("nan"), dtype=out_dtype, device="cuda")
    off = buf[1:].view(B, H)
    md.moe_decode(x, ids, w, L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s, out=off, out_dtype=out_dtype)
    torch.cuda.synchronize()
    bits = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
    assert torch.equal(off.view(bits), ref.view(bits))
    assert torch.isnan(buf[0])                  # nothing written before out


@pytest.mark.parametrize("seed", range(8))
def test_random_small_shapes(seed):
    shape = synth.random_small_shape(np.random.default_rng(500 + seed), max_E=12, max_dim=320)
    L = layer(shape, seed=seed)
    ref, _ = oracle_tokens(L, list(range(shape.B)))
    check_f32(run(L), ref, shape.name)


# --------------------------------------------------------------------------------------
# routing edge cases and invariants
# --------------------------------------------------------------------------------------

def test_duplicate_ids():
    L = small(2, 6, 3, 256, 128, seed=11)
    ids = L.ids.copy(); ids[:, 1] = ids[:, 0]
    ref, _ = oracle_tokens(L, [0, 1], ids=ids)
    check_f32(run(L, ids=ids), ref, "duplicate ids")


def test_out_of_range_ids_give_nan_rows_only():
    L = small(3, 6, 2, 256, 128, seed=12)
    ids = L.ids.copy(); ids[1, 1] = 6; ids[2, 0] = -3
    out = run(L, ids=ids).cpu()
    assert torch.isnan(out[1]).all() and torch.isnan(out[2]).all()
    ref, _ = oracle_tokens(L, [0])
    check_f32(out[0:1], ref, "valid token next to invalid ones")


def test_zero_routing_weights_give_zero():
    L = small(2, 6, 3, 256, 128, seed=13)
    out = run(L, w=np.zeros((2, 3), np.float32))
    assert torch.all(out == 0)


def test_power_of_two_weight_scaling_is_exact():
    L = small(2, 6, 3, 256, 128, seed=14)
    o1 = run(L)
    o2 = run(L, w=L.w * np.float32(2.0))
    assert torch.equal(o2, 2 * o1)


def test_slot_permutation_invariance():
    L = small(4, 16, 4, 512, 256, seed=15)
    base = run(L)
    perm = np.stack([np.random.default_rng(b).permutation(4) for b in range(4)])
    ids = np.take_along_axis(L.ids, perm, 1); w = np.take_along_axis(L.w, perm, 1)
    other = run(L, ids=ids, w=w)
    ref, _ = oracle_tokens(L, [0, 1, 2, 3])
    check_f32(other, ref, "permuted slots")
    rms = math.sqrt(float(np.mean(ref ** 2)))
    assert float((other - base).abs().max()) <= 1e-5 * rms


def test_empty_batch_launches_nothing():
    L = small(1, 4, 2, 64, 64, seed=16)
    x, ids, w = md.layer_device_inputs(L)
    out = md.moe_decode(x[:0], ids[:0], w[:0], L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s,
                        out_dtype=torch.float32)
    assert out.shape == (0, 64)


def test_deterministic_repeats():
    L = layer("batch_B8_E128_k8_H2048_I768")
    first = run(L)
    for _ in range(5):
        assert torch.equal(run(L), first)


def test_bench_kernels():
    src = torch.randint(0, 255, (1 << 20,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    md.moed_bench_copy(src, dst)
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    md.moed_bench_read(src, sink)
    # the launch-shape read probe: one-pass and looping grids, a ragged last chunk
    for unroll, wpg, groups, nbytes in ((1, 4, 0, 1 << 20), (16, 16, 3, 1 << 20), (4, 8, 0, (1 << 20) - 48),
                                        (2, 1, 1, 4096)):
        md.moed_bench_read_cfg(src, sink, nbytes, unroll, wpg, groups)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


# --------------------------------------------------------------------------------------
# expert-grouped gate/up (MFMA tiles of 16 neurons x 16 slots) and the
# tile-of-16-outputs x 16-tokens down kernel
# --------------------------------------------------------------------------------------

GROUPED = [
    (40, 3, 2, 96, 160),      # ~27 slots per expert: two slot tiles, ragged rows
    (24, 6, 4, 2080, 64),     # K steps not a multiple of the 4-step batch (65 steps)
    (3, 40, 5, 256, 96),      # mostly single-slot experts, many empty workgroups
    (64, 8, 8, 512, 288),     # every expert touched by many tokens
]


@pytest.mark.parametrize("shape", GROUPED, ids=lambda s: "B{}_E{}_k{}_H{}_I{}".format(*s))
def test_grouped_gate_up(shape):
    B = shape[0]
    L = small(*shape, seed=sum(shape) + 1)
    ref, a_ref = oracle_tokens(L, list(range(B)))
    md.set_default_tuning("gu_group=1,dn_group=1")
    try:
        check_f32(run(L), ref, f"grouped {shape}")
        check_bf16(run(L, torch.bfloat16), run(L), ref, f"grouped bf16 {shape}")
        x, ids, _ = md.layer_device_inputs(L)
        a = md.inter_to_bki(md.moe_decode_gate_up(x, ids, L.wg_q, L.wg_s, L.wu_q, L.wu_s))
        torch.cuda.synchronize()
        check_f32(a.reshape(B, -1), a_ref.reshape(B, -1), f"grouped a {shape}")
        a16 = md.inter_to_bki(md.moe_decode_gate_up(x, ids, L.wg_q, L.wg_s, L.wu_q, L.wu_s,
                                                    inter_dtype=torch.bfloat16))
        torch.cuda.synchronize()
        assert torch.isfinite(a16.float()).all()
        # bit-exact agreement between repeated runs
        assert torch.equal(run(L), run(L))
    finally:
        md.set_default_tuning(None)


def test_grouped_duplicates_and_invalid_ids():
    L = small(20, 5, 3, 128, 96, seed=77)
    ids = L.ids.copy()
    ids[:, 1] = ids[:, 0]                 # duplicate slot in every token
    ids[3, 2] = 5                         # out of range
    ids[7, 0] = -1
    md.set_default_tuning("gu_group=1,dn_group=1")
    try:
        out = run(L, ids=ids).cpu()
    finally:
        md.set_default_tuning(None)
    assert torch.isnan(out[3]).all() and torch.isnan(out[7]).all()
    good = [b for b in range(20) if b not in (3, 7)]
    ref, _ = oracle_tokens(L, good, ids=ids)
    check_f32(out[good], ref, "grouped duplicates")


# --------------------------------------------------------------------------------------
# HIP graph capture: replays equal the eager result, with eager work between replays
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("name,wformat", [("wide_B1_E128_k8_H2048_I768", "mxfp8"),
                                          ("batch_B8_E128_k8_H2048_I768", "mxfp4"),
                                          ("batch_B32_E128_k8_H4096_I1536", "mxfp8")])
def test_graph_replays_match_eager(name, wformat):
    L = synth.make_layer(name, device="cuda", wformat=wformat)
    x, ids, w = md.layer_device_inputs(L)
    sh = L.shape
    logits = torch.from_numpy(synth.make_router_logits(sh.B, sh.E, L.seed, sh.zipf_s).astype(np.float32)).cuda()
    ws = torch.empty(md.moed_workspace_bytes(sh.B, sh.k, sh.H, sh.I), dtype=torch.uint8, device="cuda")
    rid = torch.empty_like(ids)
    rw = torch.empty_like(w)
    outs = [torch.empty((sh.B, sh.H), dtype=torch.float32, device="cuda") for _ in range(2)]

    def step(o_given, o_routed):
        md.moe_decode(x, ids, w, L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s, out=o_given, workspace=ws,
                      wformat=wformat)
        md.moe_route(logits, sh.k, ids=rid, w=rw)
        md.moe_decode(x, rid, rw, L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s, out=o_routed, workspace=ws,
                      wformat=wformat)

    eager = [torch.empty_like(o) for o in outs]
    step(*eager)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(*outs)
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        rid.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {rep}"
        other = md.moe_decode(x, ids, w, L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s,
                              out_dtype=torch.bfloat16, wformat=wformat)      # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(other.float()).all()


# --------------------------------------------------------------------------------------
# expert-major down (per-slot partials in the workspace, then a slot-order sum)
# --------------------------------------------------------------------------------------

EXPERT_MAJOR = [
    (80, 2, 2, 96, 160),      # 80 slots per expert: several passes; H % 64 = 32; a leftover MX block
    (64, 4, 2, 2080, 288),    # wavefronts past H in the last row block; 2 K groups + 1 leftover block
    (33, 8, 8, 256, 64),      # k = E: every token on every expert; no full K group
    (6, 40, 5, 512, 128),     # mostly single-slot experts, many empty workgroups
]


@pytest.mark.parametrize("tiles,rt", [(0, 1), (0, 2), (1, 1), (1, 2), (2, 2), (3, 1), (3, 2)])
@pytest.mark.parametrize("shape", EXPERT_MAJOR, ids=lambda s: "B{}_E{}_k{}_H{}_I{}".format(*s))
def test_expert_major_down(shape, tiles, rt):
    B, E, k, H, I = shape
    L = small(*shape, seed=sum(shape) + 5)
    ref, _ = oracle_tokens(L, list(range(B)))
    md.set_default_tuning(f"dn_group=1,dn_tiles={tiles},dn_rt={rt}")
    try:
        out = run(L)
        check_f32(out, ref, f"expert-major tiles={tiles} rt={rt} {shape}")
        check_bf16(run(L, torch.bfloat16), out, ref, f"expert-major bf16 {shape}")
        assert torch.equal(run(L), out)
        # the down step alone with caller-owned partials: the same kernels, the same result;
        # the output is the float32 slot-order sum of the partials
        x, ids, w = md.layer_device_inputs(L)
        a_ws = md.moe_decode_gate_up(x, ids, L.wg_q, L.wg_s, L.wu_q, L.wu_s)
        y = torch.full((B * k * H,), float("nan"), dtype=torch.float32, device="cuda")
        out2 = md.moe_decode_down(a_ws, ids, w, L.wd_q, L.wd_s, out_dtype=torch.float32, partials=y)
        torch.cuda.synchronize()
        assert torch.equal(out2, out)
        yv = y.view(B, k, H)
        acc = torch.zeros((B, H), dtype=torch.float32, device="cuda")
        for j in range(k):
            acc = acc + yv[:, j]
        assert torch.equal(acc, out)
        # bf16 intermediates (the B operand is then the bf16 value itself): close to the
        # per-output kernel on the same intermediate
        o16 = run(L, inter_dtype=torch.bfloat16)
        md.set_default_tuning("dn_group=0")
        p16 = run(L, inter_dtype=torch.bfloat16)
        rms = math.sqrt(float(np.mean(ref ** 2)))
        assert float((o16 - p16).abs().max()) <= 1e-4 * rms
    finally:
        md.set_default_tuning(None)


def test_expert_major_down_without_partials_is_per_output():
    """moe_decode_down without partials keeps the per-output kernel: equal to dn_group=0."""
    L = small(40, 3, 2, 96, 160, seed=9)
    x, ids, w = md.layer_device_inputs(L)
    a_ws = md.moe_decode_gate_up(x, ids, L.wg_q, L.wg_s, L.wu_q, L.wu_s)
    md.set_default_tuning("dn_group=1")
    try:
        o1 = md.moe_decode_down(a_ws, ids, w, L.wd_q, L.wd_s, out_dtype=torch.float32)
        md.set_default_tuning("dn_group=0")
        o0 = md.moe_decode_down(a_ws, ids, w, L.wd_q, L.wd_s, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(o0, o1)
    finally:
        md.set_default_tuning(None)


def test_long_slot_list_keeps_three_tiles():
    """B*k = 8192 slots: the expert-major down holds at most 4096 16-bit slot entries in LDS at a
    time (8 KB), so three tiles of float32 a per pass still fit; the same bits as asking for two
    or three."""
    L = small(1024, 8, 8, 64, 64, seed=31)
    toks = [0, 1, 511, 1023]
    out = run(L)
    ref, _ = oracle_tokens(L, toks)
    check_f32(out[toks], ref, "B=1024")
    for form in ("dn_tiles=2", "dn_tiles=3"):
        md.set_default_tuning(form)
        try:
            assert torch.equal(run(L), out), form
        finally:
            md.set_default_tuning(None)


def test_slot_windows():
    """E = 2, k = 2, B = 9000: 18000 slots, past what the grouped gate/up holds in one list, and
    each expert has about 9000 of them, more than the 4096 one item holds, so both grouped kernels
    take each expert's slots in three windows (five without the work list, the last two empty).
    One out-of-range id at token 4500. The intermediate is the same bits with and without the
    work list and for 4 and 8 wavefronts; the layer output is the same bits with and without the
    down's work list, NaN on token 4500 and within tolerance of the oracle on tokens of all three
    windows. A second case puts 4200 out-of-range ids in the batch: the gate/up's invalid-slot
    pass also goes in windows and marks every one of them."""
    B, E, k, H, I = 9000, 2, 2, 512, 512
    L = small(B, E, k, H, I, seed=51)
    ids = L.ids.copy()
    ids[4500, 0] = E
    x, _, w = md.layer_device_inputs(L)
    idd = torch.as_tensor(ids, dtype=torch.int32).cuda().contiguous()
    got = {}
    for form in ("gu_group=1,gu_waves=4", "gu_group=1,gu_waves=8", "gu_group=1,gu_grid=0",
                 "gu_group=1,gu_waves=8,gu_grid=3"):
        say(f"slot windows {form}")
        got[form] = md.moe_decode_gate_up(x, idd, L.wg_q, L.wg_s, L.wu_q, L.wu_s, tuning=form)
    torch.cuda.synchronize()
    ref_a = got["gu_group=1,gu_waves=4"]
    for form, a in got.items():
        assert torch.equal(a.view(torch.int32), ref_a.view(torch.int32)), form
    assert torch.isnan(ref_a[4500, 0]).all()
    outs = {}
    for form in ("gu_group=1,dn_group=1", "gu_group=1,dn_group=1,dn_grid=0"):
        say(f"slot windows {form}")
        outs[form] = md.moe_decode(x, idd, w, L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s,
                                   out_dtype=torch.float32, tuning=form)
    torch.cuda.synchronize()
    out = outs["gu_group=1,dn_group=1"]
    for form, o in outs.items():
        assert torch.equal(o.view(torch.int32), out.view(torch.int32)), form
    assert torch.isnan(out[4500]).all()
    good = [0, 1, 2047, 4095, 4096, 4499, 4501, 8191, 8192, B - 1]
    assert not torch.isnan(out[good]).any()
    ref, _ = oracle_tokens(L, good, ids=ids)
    check_f32(out[good], ref, "slot windows")

    ids2 = L.ids.copy()
    ids2[:4200, 1] = -1
    idd2 = torch.as_tensor(ids2, dtype=torch.int32).cuda().contiguous()
    a2 = md.moe_decode_gate_up(x, idd2, L.wg_q, L.wg_s, L.wu_q, L.wu_s, tuning="gu_group=1")
    torch.cuda.synchronize()
    bad = torch.zeros(B, k, dtype=torch.bool)
    bad[:4200, 1] = True
    nan_rows = torch.isnan(a2.cpu()).all(dim=2)
    assert torch.equal(nan_rows, bad)
    assert not torch.isnan(a2.cpu()[~bad]).any()


@pytest.mark.parametrize("wformat", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("inter", ["f32", "bf16"])
def test_slot_windows_batch_invariance(wformat, inter):
    """Windowed and whole-list forms give the same bits: B = 9000, E = 2, k = 2 takes both grouped
    kernels in windows of 4096 slots; the first and the last 1024 tokens alone (2048 slots, one
    list) must give the same output bits for those tokens, in both weight formats and with a
    float32 or BF16 intermediate."""
    B, E, k, H, I = 9000, 2, 2, 512, 512
    L = synth.make_layer(synth.LayerShape("win", B, E, k, H, I), seed=52, device="cuda", wformat=wformat)
    x, ids, w = md.layer_device_inputs(L)
    dt = torch.float32 if inter == "f32" else torch.bfloat16
    args = (L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s)
    say(f"windows batch invariance {wformat} {inter}")
    full = md.moe_decode(x, ids, w, *args, out_dtype=torch.float32, inter_dtype=dt, wformat=wformat)
    for lo, hi in ((0, 1024), (B - 1024, B)):
        part = md.moe_decode(x[lo:hi].contiguous(), ids[lo:hi].contiguous(), w[lo:hi].contiguous(), *args,
                             out_dtype=torch.float32, inter_dtype=dt, wformat=wformat)
        torch.cuda.synchronize()
        assert torch.equal(part.view(torch.int32), full[lo:hi].view(torch.int32)), (wformat, inter, lo)
    toks = [0, 4500, B - 1]
    ref, _ = oracle_tokens(L, toks, wformat=wformat)
    check_f32(full[toks], ref, f"windows {wformat} {inter}", tol=TOL if inter == "f32" else 5e-2)   # BF16 a: the reported variant's bound


def test_slot_list_beyond_lds_falls_back():
    """B*k = 65600 slots: past what 16-bit slot entries can name, so neither grouped kernel is
    used and the layer keeps the per-slot gate/up and the per-output down."""
    L = small(8200, 8, 8, 64, 64, seed=33)
    toks = [0, 1, 4100, 8199]
    out = run(L)
    md.set_default_tuning("gu_group=0,dn_group=0")
    try:
        assert torch.equal(run(L), out)
    finally:
        md.set_default_tuning(None)
    ref, _ = oracle_tokens(L, toks)
    check_f32(out[toks], ref, "B=8200 fallback")


def test_partials_untouched_below_threshold():
    """Below B*k >= 2E moe_decode_down keeps the per-output form and never writes the partials."""
    L = small(2, 16, 4, 256, 128, seed=32)                # B*k = 8 < 2E
    x, ids, w = md.layer_device_inputs(L)
    a_ws = md.moe_decode_gate_up(x, ids, L.wg_q, L.wg_s, L.wu_q, L.wu_s)
    y = torch.full((2 * 4 * 256,), 7.0, dtype=torch.float32, device="cuda")
    out = md.moe_decode_down(a_ws, ids, w, L.wd_q, L.wd_s, out_dtype=torch.float32, partials=y)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
    ref, _ = oracle_tokens(L, [0, 1])
    check_f32(out, ref, "below threshold with partials")


def test_check_mode(monkeypatch):
    """MOED_CHECK=1: ids outside [0, E) and NaN codes or scales in a routed expert's rows are
    reported as MOED_ERR_SHAPE before anything else is launched; valid inputs give the same
    result as without the check; NaNs in experts nobody is routed to are not an error."""
    L = small(3, 6, 2, 256, 128, seed=41)
    base = run(L)
    monkeypatch.setenv("MOED_CHECK", "1")
    assert torch.equal(run(L), base)

    def expect_shape_error(fn):
        with pytest.raises(md.MoedError) as ei:
            fn()
        assert ei.value.status == md.MOED_ERR_SHAPE

    ids = L.ids.copy()
    ids[1, 1] = 6
    expect_shape_error(lambda: run(L, ids=ids))
    routed = sorted(set(L.ids.ravel().tolist()))
    unrouted = [e for e in range(6) if e not in routed]
    e = routed[0]
    for t, idx, bad in ((L.wd_q, (e, 5, 7), 0x7F), (L.wg_q, (e, 3, 100), 0xFF), (L.wu_s, (e, 2, 1), 0xFF)):
        saved = t[idx].item()
        t[idx] = bad
        try:
            expect_shape_error(lambda: run(L))
        finally:
            t[idx] = saved
    assert torch.equal(run(L), base)
    if unrouted:
        u = unrouted[0]
        saved = L.wg_s[u, 0, 0].item()
        L.wg_s[u, 0, 0] = 0xFF
        try:
            assert torch.equal(run(L), base)
        finally:
            L.wg_s[u, 0, 0] = saved
    # the step entry points check the matrices they use
    x, idd, wd = md.layer_device_inputs(L)
    bad_ids = torch.as_tensor(ids, dtype=torch.int32).cuda()
    expect_shape_error(lambda: md.moe_decode_gate_up(x, bad_ids, L.wg_q, L.wg_s, L.wu_q, L.wu_s))
    a_ws = md.moe_decode_gate_up(x, idd, L.wg_q, L.wg_s, L.wu_q, L.wu_s)
    saved = L.wd_s[e, 0, 0].item()
    L.wd_s[e, 0, 0] = 0xFF
    try:
        expect_shape_error(lambda: md.moe_decode_down(a_ws, idd, wd, L.wd_q, L.wd_s, out_dtype=torch.float32))
        md.moe_decode_gate_up(x, idd, L.wg_q, L.wg_s, L.wu_q, L.wu_s)     # gate/up does not read Wd
    finally:
        L.wd_s[e, 0, 0] = saved
    torch.cuda.synchronize()



def test_input_check_scale_range(monkeypatch):
    """MOED_CHECK=1 also reports routed block scales outside the range the large-batch kernels
    decode exactly (MXFP8 codes 10..245), as MOED_ERR_SCALE, and only for calls that take those
    kernels: the expert-grouped gate/up for gate/up scales, the expert-major down for down scales."""
    L = small(40, 4, 2, 256, 64, seed=43)            # 4*B*k >= 3*E and B*k >= 2E: both grouped
    monkeypatch.setenv("MOED_CHECK", "1")
    base = run(L)
    routed = sorted(set(L.ids.ravel().tolist()))
    e = routed[0]

    def status(fn):
        try:
            fn()
            torch.cuda.synchronize()
            return md.MOED_OK
        except md.MoedError as err:
            return err.status

    x, idd, wd = md.layer_device_inputs(L)
    for t, idx, code, grouped_spec, plain_spec in (
            (L.wg_s, (e, 1, 2), 5, "gu_group=1", "gu_group=0"),
            (L.wu_s, (e, 0, 0), 250, "gu_group=1", "gu_group=0"),
            (L.wd_s, (e, 3, 1), 9, "dn_group=1", "dn_group=0")):
        saved = t[idx].item()
        t[idx] = code
        try:
            assert status(lambda: run(L)) == md.MOED_ERR_SCALE
            with md.tuned(grouped_spec):
                assert status(lambda: run(L)) == md.MOED_ERR_SCALE
            with md.tuned(plain_spec):
                assert status(lambda: run(L)) == md.MOED_OK
            if t is L.wd_s:
                a_ws = md.moe_decode_gate_up(x, idd, L.wg_q, L.wg_s, L.wu_q, L.wu_s)
                y = torch.empty(40 * 2 * 256, dtype=torch.float32, device="cuda")
                assert status(lambda: md.moe_decode_down(a_ws, idd, wd, L.wd_q, L.wd_s, partials=y)) == \
                    md.MOED_ERR_SCALE
                assert status(lambda: md.moe_decode_down(a_ws, idd, wd, L.wd_q, L.wd_s)) == md.MOED_OK
            else:
                assert status(lambda: md.moe_decode_gate_up(x, idd, L.wg_q, L.wg_s, L.wu_q, L.wu_s)) == \
                    md.MOED_ERR_SCALE
        finally:
            t[idx] = saved
    # the edges of the exact range are accepted
    for code in (10, 245):
        saved = L.wg_s[e, 0, 0].item()
        L.wg_s[e, 0, 0] = code
        try:
            assert status(lambda: run(L)) == md.MOED_OK
        finally:
            L.wg_s[e, 0, 0] = saved
    assert torch.equal(run(L), base)

WIDE = [
    (40, 3, 2, 1024, 160),    # ~27 slots per expert (2 tiles); waves past I
    (72, 2, 2, 512, 96),      # 72 slots per expert: a 4-tile pass, then a 1-tile pass; one scale block
    (48, 2, 2, 1024, 192),    # 48 slots per expert: a 3-tile pass (an odd tile count for 8 wavefronts)
    (24, 6, 4, 2560, 64),     # 5 MXFP8 step pairs / 5 MXFP4 steps
    (20, 4, 3, 1536, 128),    # 3 step pairs / 3 steps
    (16, 8, 8, 7168, 64),     # 14 step pairs of 7168-value rows
    (24, 6, 4, 2080, 64),     # H not a multiple of 512: the 128-byte slices either way
]


@pytest.mark.parametrize("wformat", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("shape", WIDE, ids=lambda s: "B{}_E{}_k{}_H{}_I{}".format(*s))
def test_grouped_wide_loads(shape, wformat):
    """The MFMA path's wide weight loads (256-byte runs per row, moved to the operand layout
    through LDS, scales fetched in 16-byte blocks and handed out by ds_bpermute) feed every
    MFMA the codes and scales the 128-byte tile slices do, in the same order, with workgroups
    of 4 wavefronts (items of 64 neurons) or 8 (items of 128, the two halves loading
    alternate x tiles), and with the built-in choice between them: the intermediate is the
    same floats (float32 and bf16), and the layer within tolerance of the oracle."""
    B, E, k, H, I = shape
    L = synth.make_layer(synth.LayerShape("wide", B, E, k, H, I), seed=sum(shape) + 21, device="cuda",
                         wformat=wformat)
    x, ids, _ = md.layer_device_inputs(L)
    got = {}
    forms = ["gu_wide=0", "gu_wide=1,gu_waves=4", "gu_wide=1,gu_waves=8", "gu_wide=1"]
    try:
        for form in forms:
            md.set_default_tuning(f"gu_group=1,{form}")
            for dt in (torch.float32, torch.bfloat16):
                got[form, dt] = md.moe_decode_gate_up(x, ids, L.wg_q, L.wg_s, L.wu_q, L.wu_s,
                                                      inter_dtype=dt, wformat=wformat)
            torch.cuda.synchronize()
        say(f"wide loads {shape} {wformat}: comparing")
        for form in forms[1:]:
            for dt in (torch.float32, torch.bfloat16):
                assert torch.equal(got[form, dt], got[forms[0], dt]), f"{shape} {wformat} {form} {dt}"
        md.set_default_tuning("gu_group=1,gu_wide=1")
        ref, _ = oracle_tokens(L, [0, B - 1], wformat=wformat)
        xd, idd, wd = md.layer_device_inputs(L)
        out = md.moe_decode(xd, idd, wd, L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s,
                            out_dtype=torch.float32, wformat=wformat)
        torch.cuda.synchronize()
        check_f32(out[[0, B - 1]], ref, f"wide {shape} {wformat}")
    finally:
        md.set_default_tuning(None)


@pytest.mark.parametrize("wformat", ["mxfp8", "mxfp4"])
def test_grouped_eight_waves_with_invalid_ids(wformat):
    """The 8-wavefront gate/up (items of 128 neurons, its own choice here since B*k >= 32*E) with a
    duplicated and two out-of-range ids, with the work list at the built-in cap and at a cap of 3
    workgroups, and with one workgroup per item of all E experts (gu_grid=0): the intermediate is
    bit-identical to the 4-wavefront form,
    NaN over all I neurons of exactly the invalid slots (its invalid-slot pass covers blocks of 128
    neurons, the last one ragged at I = 160); the layer is NaN on those tokens and within tolerance
    of the oracle on the others."""
    B, E, k, H, I = 48, 3, 2, 1024, 160
    L = synth.make_layer(synth.LayerShape("w8", B, E, k, H, I), seed=91, device="cuda", wformat=wformat)
    ids = L.ids.copy()
    ids[5, 1] = ids[5, 0]
    ids[9, 0] = 3
    ids[30, 1] = -2
    x, _, w = md.layer_device_inputs(L)
    idd = torch.as_tensor(ids, dtype=torch.int32).cuda().contiguous()
    got = {}
    for form in ("gu_group=1,gu_waves=4", "gu_group=1,gu_waves=8", "gu_group=1",
                 "gu_group=1,gu_waves=8,gu_grid=0", "gu_group=1,gu_waves=8,gu_grid=3"):
        say(f"eight waves {wformat} {form}")
        got[form] = md.moe_decode_gate_up(x, idd, L.wg_q, L.wg_s, L.wu_q, L.wu_s, wformat=wformat, tuning=form)
    torch.cuda.synchronize()
    ref = got["gu_group=1,gu_waves=4"]
    for form, a in got.items():
        assert torch.equal(a.view(torch.int32), ref.view(torch.int32)), f"{wformat} {form}"
    bad = torch.zeros(B, k, dtype=torch.bool)
    bad[9, 0] = True
    bad[30, 1] = True
    nan_rows = torch.isnan(ref.cpu()).all(dim=2)
    assert torch.equal(nan_rows, bad)
    assert not torch.isnan(ref.cpu()[~bad]).any()
    out = md.moe_decode(x, idd, w, L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s, out_dtype=torch.float32,
                        wformat=wformat, tuning="gu_group=1,dn_group=1")
    torch.cuda.synchronize()
    assert torch.isnan(out[9]).all() and torch.isnan(out[30]).all()
    good = [0, 5, 17, B - 1]
    ref_out, _ = oracle_tokens(L, good, ids=ids, wformat=wformat)
    check_f32(out[good], ref_out, f"eight waves {wformat}")


# (B, E, k, H, I): which straight-line kernels each shape takes --
#   one-pass down: k = G*JB slots in one group, a row of at most 64/G chunks
#   exact-fit gate/up: a row of exactly 64*U chunks
@pytest.mark.parametrize("wformat", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("shape", [(1, 128, 8, 2048, 768),     # G=1 JB=8 (mxfp8), G=2 JB=4 (mxfp4); U=2 / U=1
                                   (1, 8, 2, 256, 128),        # lane groups, one slot each
                                   (3, 12, 4, 1024, 1024),     # G=1 JB=4 at B=3 (rows kernel for B>1 under mxfp8)
                                   (2, 9, 1, 4096, 544),       # k=1; U=4 / U=2
                                   (5, 64, 8, 2048, 256),      # four lane groups at B=5
                                   (1, 6, 6, 1024, 640),       # k=6: not a power-of-two group (generic kernels)
                                   (1, 64, 8, 2048, 256),      # single token, four lane groups of two slots
                                   (1, 32, 8, 1024, 1024),     # single token, four copy loads per thread
                                   (16, 128, 8, 2048, 768),    # B*k = E: blocks form (G=1 JB=8 / G=2 JB=4)
                                   (10, 64, 8, 1024, 1536),    # mxfp4 G=1 JB=8 (not the blocks form), mxfp8 generic
                                   (6, 16, 4, 512, 256),       # blocks form with four lane groups of one slot
                                   (8, 32, 4, 1056, 256)])     # B*k = E but H not a multiple of 64: generic
def test_straight_line_kernels_match_generic(shape, wformat):
    """The one-pass down (and its blocks form where tokens share experts) and the exact-fit gate/up
    kernels compute the same floats as the generic staged / per-slot kernels they replace (same
    products, FMA order and reduction), so the intermediate and both output dtypes agree bit for
    bit; both also meet the oracle gate. The ids include an invalid one when B > 1 (its token's
    outputs NaN on both sides)."""
    B, E, k, H, I = shape
    L = synth.make_layer(synth.LayerShape("sl", B, E, k, H, I), seed=sum(shape) + 5, device="cuda", wformat=wformat)
    ids = L.ids.copy()
    if B > 1:
        ids[B - 1, 0] = E                     # out of range: that token's outputs are NaN
    x, _, wd = md.layer_device_inputs(L)
    idd = torch.as_tensor(ids, dtype=torch.int32).cuda().contiguous()
    got = {}
    for spec in ["gu_exact=0,dn_onepass=0", None]:
        md.set_default_tuning(spec)
        try:
            say(f"straight-line {shape} {wformat} spec={spec}")
            a = md.moe_decode_gate_up(x, idd, L.wg_q, L.wg_s, L.wu_q, L.wu_s, wformat=wformat)
            outs = [md.moe_decode(x, idd, wd, L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s,
                                  out_dtype=dt, wformat=wformat) for dt in (torch.float32, torch.bfloat16)]
            torch.cuda.synchronize()
            got[spec] = [a.clone()] + [o.clone() for o in outs]
        finally:
            md.set_default_tuning(None)
    for t0, t1, what in zip(got["gu_exact=0,dn_onepass=0"], got[None], ["a", "out f32", "out bf16"]):
        nan0, nan1 = torch.isnan(t0.float()), torch.isnan(t1.float())
        assert torch.equal(nan0, nan1), f"{shape} {wformat}: {what} NaN positions differ"
        bits = torch.int32 if t0.dtype == torch.float32 else torch.int16
        assert torch.equal(t0.view(bits)[~nan0], t1.view(bits)[~nan1]), \
            f"{shape} {wformat}: {what} differs between the straight-line and the generic kernels"
    good = list(range(B - 1)) if B > 1 else [0]
    ref, _ = oracle_tokens(L, good, ids=ids, wformat=wformat)
    check_f32(got[None][1][good], ref, f"straight-line {shape} {wformat}")
    if B > 1:
        assert torch.isnan(got[None][1][B - 1]).all()


@pytest.mark.parametrize("wformat", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("shape", [(64, 40, 8, 512, 256, 1.1),    # skewed: a few hot experts, many empty ones
                                   (24, 16, 4, 1024, 384, 0.0),   # every expert routed
                                   (48, 300, 8, 256, 128, 1.1)])  # E beyond one item per routed expert
def test_grouped_work_list_matches_full_grid(shape, wformat):
    """The grouped gate/up and the expert-major down give the same bits whether the grid has one
    workgroup per item of all E experts (gu_grid=dn_grid=0) or a few workgroups walk the routed experts'
    items (the work list, at the built-in grid cap and at a cap of 5); an invalid id on the last
    token gives NaN there on every form."""
    B, E, k, H, I, zipf = shape
    L = synth.make_layer(synth.LayerShape("wl", B, E, k, H, I, zipf), seed=B + E, device="cuda", wformat=wformat)
    ids = L.ids.copy()
    ids[B - 1, 1] = -3
    x, _, wd = md.layer_device_inputs(L)
    idd = torch.as_tensor(ids, dtype=torch.int32).cuda().contiguous()
    got = []
    for spec in ["gu_grid=0,dn_grid=0,gu_group=1,dn_group=1", "gu_group=1,dn_group=1",
                 "gu_grid=5,dn_grid=3,gu_group=1,dn_group=1"]:
        md.set_default_tuning(spec)
        try:
            say(f"work list {shape} {wformat} {spec}")
            out = md.moe_decode(x, idd, wd, L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s,
                                out_dtype=torch.float32, wformat=wformat)
            torch.cuda.synchronize()
            got.append(out.clone())
        finally:
            md.set_default_tuning(None)
    for g in got[1:]:
        assert torch.equal(torch.isnan(g), torch.isnan(got[0]))
        assert torch.equal(g[:B - 1].view(torch.int32), got[0][:B - 1].view(torch.int32)), f"{shape} {wformat}"
    assert torch.isnan(got[0][B - 1]).all()
    ref, _ = oracle_tokens(L, [0, B // 2, B - 2], ids=ids, wformat=wformat)
    check_f32(got[1][[0, B // 2, B - 2]], ref, f"work list {shape} {wformat}")


@pytest.mark.parametrize("wformat", ["mxfp8", "mxfp4"])
def test_grouped_kernels_with_unaligned_scale_arrays(wformat):
    """The wide loads read each row's scale bytes in 8-byte pieces, so they need 8-byte aligned
    scale arrays; scale arrays at odd addresses take the 128-byte slices instead, which give the
    same floats: the layer output is bit-identical with aligned and unaligned scale arrays."""
    B, E, k, H, I = 40, 3, 2, 1024, 512
    L = synth.make_layer(synth.LayerShape("unal", B, E, k, H, I), seed=77, device="cuda", wformat=wformat)
    x, ids, w = md.layer_device_inputs(L)

    def shifted(t):                                   # the same bytes at an address 1 past a 16-byte boundary
        buf = torch.empty(t.numel() + 16, dtype=torch.uint8, device="cuda")
        v = buf[1:1 + t.numel()].view(t.shape)
        v.copy_(t)
        assert v.data_ptr() % 8 == 1
        return v

    scales = {"wg_s": shifted(L.wg_s), "wu_s": shifted(L.wu_s), "wd_s": shifted(L.wd_s)}
    outs = []
    with md.tuned("gu_group=1,dn_group=1"):
        for gs, us, ds in ((L.wg_s, L.wu_s, L.wd_s), (scales["wg_s"], scales["wu_s"], scales["wd_s"])):
            outs.append(md.moe_decode(x, ids, w, L.wg_q, gs, L.wu_q, us, L.wd_q, ds, out_dtype=torch.float32,
                                      wformat=wformat))
        torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
    ref, _ = oracle_tokens(L, [0, B - 1], wformat=wformat)
    check_f32(outs[1][[0, B - 1]], ref, f"unaligned scales {wformat}")


# (B, E, k, H, I) for the expert-major down's wide weight loads
DOWN_WIDE = [
    (40, 3, 2, 96, 1024),     # ~27 slots per expert (2 tiles); waves past H
    (72, 2, 2, 64, 512),      # 72 slots per expert: passes of 2 + 2 + 1 tiles (float32 a); one scale block
    (24, 6, 4, 2080, 1536),   # 3 MXFP8 step pairs / 3 MXFP4 steps; waves past H in the last block
    (20, 4, 3, 128, 2560),    # 5 step pairs / 5 steps
    (16, 8, 8, 64, 7168),     # 14 step pairs per row
    (24, 6, 4, 2080, 544),    # I not a multiple of 512: the 128-byte slices either way
    (40, 1, 1, 64, 512),      # 40 slots: 3 tiles in one pass of two halves, the last half partly empty
    (64, 1, 1, 128, 1024),    # 64 slots: 4 tiles in one pass of two halves
]


@pytest.mark.parametrize("rt", [2, 1])
@pytest.mark.parametrize("wformat", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("shape", DOWN_WIDE, ids=lambda s: "B{}_E{}_k{}_H{}_I{}".format(*s))
def test_expert_major_down_wide_loads(shape, wformat, rt):
    """The expert-major down's wide weight loads (256-byte runs per row, moved to the operand
    layout through LDS, scales fetched in 16-byte blocks and handed out by ds_bpermute) feed
    every MFMA the codes and scales the 128-byte slices do, in the same order, with passes of 2
    float32 tiles or (the default) of up to 4 in two halves: the layer output is the same floats
    for float32 and bf16 intermediates (an invalid id on the last token gives NaN there on all),
    and within tolerance of the oracle."""
    B, E, k, H, I = shape
    L = synth.make_layer(synth.LayerShape("dwide", B, E, k, H, I), seed=sum(shape) + 41, device="cuda",
                         wformat=wformat)
    ids = L.ids.copy()
    ids[B - 1, 0] = E + 2
    x, _, wd = md.layer_device_inputs(L)
    idd = torch.as_tensor(ids, dtype=torch.int32).cuda().contiguous()
    got = {}
    variants = ("dn_wide=0", "dn_wide=1,dn_split=0", "dn_wide=1")
    try:
        for v in variants:
            md.set_default_tuning(f"dn_group=1,dn_rt={rt},{v}")
            say(f"down wide loads {shape} {wformat} rt={rt} {v}")
            for dt in (torch.float32, torch.bfloat16):
                got[v, dt] = md.moe_decode(x, idd, wd, L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s,
                                           out_dtype=torch.float32, inter_dtype=dt, wformat=wformat)
            torch.cuda.synchronize()
    finally:
        md.set_default_tuning(None)
    for dt in (torch.float32, torch.bfloat16):
        o0 = got[variants[0], dt]
        for v in variants[1:]:
            o1 = got[v, dt]
            assert torch.equal(torch.isnan(o0), torch.isnan(o1))
            assert torch.equal(o0[:B - 1].view(torch.int32), o1[:B - 1].view(torch.int32)), f"{shape} {wformat} {dt} {v}"
            assert torch.isnan(o1[B - 1]).all()
    toks = sorted({0, B // 2, B - 2})
    ref, _ = oracle_tokens(L, toks, ids=ids, wformat=wformat)
    check_f32(got["dn_wide=1", torch.float32][toks], ref, f"down wide {shape} {wformat}")
