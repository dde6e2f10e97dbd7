"""GPU parity of the MXFP4 weight variant (FP4 E2M1 codes two per byte, one UE8M0
scale per 32 values) through the C-ABI, against the float64 CPU oracle run on
the same packed bytes.

Same gate as the MXFP8 path: with float32 outputs, max |gpu - oracle| <=
2e-3 * rms(oracle); BF16 outputs are the RNE of the float32 result bit for bit.
The decode self-test checks all 16 E2M1 codes in both nibble positions and all
four byte selects, on both in-register routes, bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from output_centric_expert_amd import moedecode as md
from output_centric_expert_amd import synth
from test_gpu_parity import check_bf16, check_f32, say

pytestmark = pytest.mark.gpu
WF = "mxfp4"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    md.load()
    oracle.build(force=False)
    yield
    md.set_default_tuning(None)


def layer(shape, seed=None):
    return synth.make_layer(shape, seed=seed, device="cuda", wformat=WF)


def small(B, E, k, H, I, seed=0, zipf=0.0):
    return layer(synth.LayerShape(f"f4_{B}_{E}_{k}_{H}_{I}", B, E, k, H, I, zipf), seed=seed)


def run(L, out_dtype=torch.float32, inter_dtype=torch.float32, ids=None):
    x, idd, w = md.layer_device_inputs(L)
    if ids is not None:
        idd = torch.as_tensor(ids, dtype=torch.int32).cuda().contiguous()
    out = md.moe_decode(x, idd, w, L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s,
                        out_dtype=out_dtype, inter_dtype=inter_dtype, wformat=WF)
    torch.cuda.synchronize()
    return out


def oracle_tokens(L, tokens, ids=None):
    """Oracle output and intermediate for some tokens (only their experts copied to the host)."""
    ids = L.ids if ids is None else np.asarray(ids, np.int32)
    ids_t = ids[tokens]
    sel = sorted({int(e) for e in ids_t.ravel() if 0 <= e < L.shape.E})
    remap = np.full(L.shape.E, -1, np.int64)
    remap[sel] = np.arange(len(sel))
    ids_c = np.where((ids_t >= 0) & (ids_t < L.shape.E), remap[np.clip(ids_t, 0, L.shape.E - 1)], -1)
    idx = torch.tensor(sel if sel else [0], device=L.wg_q.device)
    pick = lambda t: t.index_select(0, idx).cpu()
    return oracle.moe_decode(np.ascontiguousarray(L.x[tokens]), np.ascontiguousarray(ids_c.astype(np.int32)),
                             np.ascontiguousarray(L.w[tokens]), pick(L.wg_q), pick(L.wg_s), pick(L.wu_q),
                             pick(L.wu_s), pick(L.wd_q), pick(L.wd_s), return_inter=True, wformat=WF)


# --------------------------------------------------------------------------------------
# decode self-test
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("path", [3, 4, 5])
def test_e2m1_decode_all_codes_bit_exact(path):
    scales = [127, 100, 120, 126, 128, 134, 147, 2]   # every product a normal float32
    # 16 codes x 8 nibble positions per scale (t % 8 picks the nibble inside the packed dword)
    codes = np.tile(np.repeat(np.arange(16, dtype=np.uint8), 8), len(scales))
    sc = np.repeat(np.array(scales, np.uint8), 16 * 8)
    got = md.moed_selftest_decode(torch.from_numpy(codes).cuda(), torch.from_numpy(sc).cuda(), path).cpu().numpy()
    for t in range(codes.size):
        ref = oracle.e2m1_value(int(codes[t])) * oracle.ue8m0_value(int(sc[t]))
        r32 = np.float32(ref)
        assert float(r32) == ref
        assert got[t] == r32 and np.signbit(got[t]) == np.signbit(r32), (path, t % 8, hex(codes[t]), sc[t], got[t], ref)


def test_e2m1_decode_nan_scale():
    codes = torch.tensor([0x2, 0x0, 0xF, 0x9], dtype=torch.uint8).cuda()
    sc = torch.full((4,), 255, dtype=torch.uint8).cuda()
    for path in (3, 4, 5):
        assert torch.isnan(md.moed_selftest_decode(codes, sc, path)).all()


# --------------------------------------------------------------------------------------
# workloads, ragged shapes, variants
# --------------------------------------------------------------------------------------

FULL = ["tiny_B1_E8_k2_H256_I128", "wide_B1_E128_k8_H2048_I768", "batch_B8_E128_k8_H2048_I768"]
LARGE = ["batch_B32_E128_k8_H4096_I1536", "skewed_B64_E256_k8_H7168_I2048"]


@pytest.mark.parametrize("name", FULL)
def test_fp4_workload_full_parity(name):
    say(f"mxfp4 workload {name}: full parity")
    L = layer(name)
    ref, a_ref = oracle_tokens(L, list(range(L.shape.B)))
    out32 = run(L)
    check_f32(out32, ref, "mxfp4 " + name)
    check_bf16(run(L, torch.bfloat16), out32, ref, "mxfp4 " + name)
    x, ids, _ = md.layer_device_inputs(L)
    a = md.inter_to_bki(md.moe_decode_gate_up(x, ids, L.wg_q, L.wg_s, L.wu_q, L.wu_s, wformat=WF))
    torch.cuda.synchronize()
    check_f32(a.reshape(L.shape.B, -1), a_ref.reshape(L.shape.B, -1), "mxfp4 a " + name)
    # the down step alone on that intermediate
    a_ws = md.moe_decode_gate_up(x, ids, L.wg_q, L.wg_s, L.wu_q, L.wu_s, wformat=WF)
    _, idd, wd = md.layer_device_inputs(L)
    out = md.moe_decode_down(a_ws, idd, wd, L.wd_q, L.wd_s, out_dtype=torch.float32, wformat=WF)
    torch.cuda.synchronize()
    assert torch.equal(out, out32)


@pytest.mark.parametrize("name", LARGE)
def test_fp4_workload_large_full_parity(name):
    """Every output of every token against the oracle, on the default and on the pure
    output-centric kernel pair; determinism and batch = concatenation of tokens."""
    say(f"mxfp4 workload {name}: full parity, both kernel pairs")
    L = layer(name)
    B = L.shape.B
    out = run(L)
    assert torch.isfinite(out).all()
    assert torch.equal(run(L), out), "not deterministic"
    ref, _ = oracle_tokens(L, list(range(B)))
    check_f32(out, ref, "mxfp4 " + name)
    with md.tuned("gu_group=0,dn_group=0"):
        check_f32(run(L), ref, "mxfp4 output-centric pair " + name)
    # batch = concatenation of single-token calls, bit for bit, on each kernel pair
    # (the per-slot/per-output and the expert-grouped kernels accumulate in different orders)
    x, ids, w = md.layer_device_inputs(L)
    for spec in ("gu_group=0,dn_group=0", "gu_group=1,dn_group=1"):
        with md.tuned(spec):
            full = run(L)
            for b in (0, B - 1):
                one = md.moe_decode(x[b:b + 1].contiguous(), ids[b:b + 1].contiguous(), w[b:b + 1].contiguous(),
                                    L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s, out_dtype=torch.float32,
                                    wformat=WF)
                torch.cuda.synchronize()
                assert torch.equal(one[0], full[b]), spec


@pytest.mark.parametrize("shape", [(3, 12, 4, 2048, 256), (2, 9, 1, 4096, 544), (4, 16, 8, 2048, 768),
                                   (3, 7, 2, 8192, 96)],
                         ids=lambda s: "B{}_E{}_k{}_H{}_I{}".format(*s))
def test_fp4_exact_fit_neuron_block_order(shape):
    """B > 1 with MXFP4 rows of exactly 64*U chunks: the exact-fit gate/up with two neurons per
    wavefront (the default here), with one (gu_pair=0), and in neuron-block order (gu_order=2)
    computes the same floats, and matches the oracle."""
    B = shape[0]
    L = small(*shape, seed=sum(shape) + 21)
    x, ids, _ = md.layer_device_inputs(L)
    got = {}
    for spec in ("gu_order=0", "gu_order=0,gu_pair=0", "gu_order=2"):
        with md.tuned(f"gu_group=0,{spec}"):
            got[spec] = md.moe_decode_gate_up(x, ids, L.wg_q, L.wg_s, L.wu_q, L.wu_s, wformat=WF)
            torch.cuda.synchronize()
    assert torch.equal(got["gu_order=0"], got["gu_order=0,gu_pair=0"])
    assert torch.equal(got["gu_order=0"], got["gu_order=2"])
    _, a_ref = oracle_tokens(L, list(range(B)))
    check_f32(md.inter_to_bki(got["gu_order=0"]).reshape(B, -1), a_ref.reshape(B, -1), f"mxfp4 pairs a {shape}")
    with md.tuned("gu_group=0,gu_order=2"):
        out = run(L)
    ref, _ = oracle_tokens(L, list(range(B)))
    check_f32(out, ref, f"mxfp4 gu_order=2 {shape}")


@pytest.mark.parametrize("shape", [(8, 128, 8, 2048, 768), (4, 40, 4, 1024, 256), (2, 16, 2, 256, 64),
                                   (3, 20, 4, 96, 160), (6, 64, 8, 512, 1024), (16, 64, 2, 2048, 256)],
                         ids=lambda s: "B{}_E{}_k{}_H{}_I{}".format(*s))
def test_fp4_down_two_outputs_per_wavefront(shape):
    """MXFP4: the one-pass down with two neighbouring outputs per wavefront (default at B > 1;
    workgroups of 4 wavefronts, or of 8 once B*H/16 >= 2048 as in the last shape) gives the same
    floats as with one (dn_pair=0), in float32 and bf16 output, and matches the oracle."""
    B = shape[0]
    L = small(*shape, seed=sum(shape) + 7)
    got = {}
    for spec in ("dn_pair=1", "dn_pair=0"):
        with md.tuned(spec):
            got[spec] = (run(L), run(L, out_dtype=torch.bfloat16))
    for t1, t0 in zip(got["dn_pair=1"], got["dn_pair=0"]):
        assert torch.equal(t1.view(torch.int16 if t1.dtype == torch.bfloat16 else torch.int32),
                           t0.view(torch.int16 if t0.dtype == torch.bfloat16 else torch.int32)), shape
    ref, _ = oracle_tokens(L, list(range(B)))
    check_f32(got["dn_pair=1"][0], ref, f"mxfp4 down pairs {shape}")


SHAPES = [
    (1, 4, 2, 32, 32),        # one MX block per row: a single 16-byte chunk
    (3, 6, 3, 96, 160),       # rows much shorter than a wave
    (2, 5, 5, 4160, 96),      # gate/up rows of 130 chunks: a ragged second chunk per lane
    (2, 3, 2, 16448, 64),     # 514 chunks per gate/up row: more than 8 per lane -> two passes
    (2, 8, 4, 128, 4160),     # down rows of 130 chunks; k*I*4 = 66560 > 64 KiB: unstaged down
    (5, 16, 1, 64, 1056),     # k = 1
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}_E{}_k{}_H{}_I{}".format(*s))
def test_fp4_ragged_shapes(shape):
    B = shape[0]
    L = small(*shape, seed=sum(shape) + 11)
    ref, a_ref = oracle_tokens(L, list(range(B)))
    check_f32(run(L), ref, f"mxfp4 ragged {shape}")
    x, ids, _ = md.layer_device_inputs(L)
    a = md.inter_to_bki(md.moe_decode_gate_up(x, ids, L.wg_q, L.wg_s, L.wu_q, L.wu_s, wformat=WF))
    torch.cuda.synchronize()
    check_f32(a.reshape(B, -1), a_ref.reshape(B, -1), f"mxfp4 ragged a {shape}")
    check_f32(run(L, inter_dtype=torch.bfloat16), ref, f"mxfp4 ragged bf16-a {shape}", tol=5e-2)


@pytest.mark.parametrize("spec", ["gu_umax=1,dn_umax=1", "dn_stage=0", "dn_stage=0,dn_umax=8", "gu_wpb=1,dn_wpb=3",
                                  "gu_group=1", "dn_group=1", "dn_lanegroups=0", "dn_umax=2", "gu_exact=0,gu_umax=1",
                                  "dn_onepass=0", "dn_onepass=0,dn_lanegroups=0", "gu_exact=0", "gu_order=2",
                                  "gu_pair=0", "dn_pair=0"])
def test_fp4_tuning_variants_keep_parity(spec):
    for shape in [(1, 128, 8, 2048, 768), (3, 6, 3, 96, 160), (2, 3, 2, 16448, 64), (4, 40, 4, 2048, 256)]:
        L = small(*shape, seed=3)
        ref, _ = oracle_tokens(L, list(range(shape[0])))
        md.set_default_tuning(spec)
        try:
            check_f32(run(L), ref, f"mxfp4 {spec} {shape}")
        finally:
            md.set_default_tuning(None)


def test_fp4_duplicate_and_invalid_ids():
    L = small(4, 6, 3, 128, 96, seed=41)
    ids = L.ids.copy()
    ids[0, 1] = ids[0, 0]                 # duplicate slot
    ids[2, 2] = 6                         # out of range
    ids[3, 0] = -5
    out = run(L, ids=ids).cpu()
    assert torch.isnan(out[2]).all() and torch.isnan(out[3]).all()
    assert torch.isfinite(out[[0, 1]]).all()
    ref, _ = oracle_tokens(L, [0, 1], ids=ids)
    check_f32(out[[0, 1]], ref, "mxfp4 ids")


@pytest.mark.parametrize("seed", range(4))
def test_fp4_random_small_shapes(seed):
    rng = np.random.default_rng(500 + seed)
    sh = synth.random_small_shape(rng, max_E=8, max_dim=256)
    L = layer(sh, seed=seed)
    ref, _ = oracle_tokens(L, list(range(sh.B)))
    check_f32(run(L), ref, f"mxfp4 random {sh.name}")


GROUPED = [
    (40, 3, 2, 96, 160),      # ~27 slots per expert: two slot tiles, ragged rows
    (24, 6, 4, 2080, 64),     # K steps not a multiple of the 4-step group (65 steps)
    (3, 40, 5, 256, 96),      # mostly single-slot experts
    (64, 8, 8, 512, 288),     # every expert touched by many tokens
]


@pytest.mark.parametrize("shape", GROUPED, ids=lambda s: "B{}_E{}_k{}_H{}_I{}".format(*s))
def test_fp4_grouped_gate_up(shape):
    B = shape[0]
    L = small(*shape, seed=sum(shape) + 21)
    ref, a_ref = oracle_tokens(L, list(range(B)))
    md.set_default_tuning("gu_group=1")
    try:
        out = run(L)
        check_f32(out, ref, f"mxfp4 grouped {shape}")
        check_bf16(run(L, torch.bfloat16), out, ref, f"mxfp4 grouped bf16 {shape}")
        x, ids, _ = md.layer_device_inputs(L)
        a = md.inter_to_bki(md.moe_decode_gate_up(x, ids, L.wg_q, L.wg_s, L.wu_q, L.wu_s, wformat=WF))
        torch.cuda.synchronize()
        check_f32(a.reshape(B, -1), a_ref.reshape(B, -1), f"mxfp4 grouped a {shape}")
        assert torch.equal(run(L), out)
    finally:
        md.set_default_tuning(None)


@pytest.mark.parametrize("shape", [(80, 2, 2, 96, 160), (64, 4, 2, 2080, 288)],
                         ids=lambda s: "B{}_E{}_k{}_H{}_I{}".format(*s))
def test_fp4_expert_major_down(shape):
    """The expert-major down on MXFP4 rows: more slots per expert than one pass takes, H % 64 = 32,
    a leftover MX block; through moe_decode and through moe_decode_down with partials."""
    B, E, k, H, I = shape
    L = small(*shape, seed=sum(shape) + 31)
    ref, _ = oracle_tokens(L, list(range(B)))
    for tiles, rt in ((0, 1), (0, 2), (1, 2)):
        md.set_default_tuning(f"dn_group=1,dn_tiles={tiles},dn_rt={rt}")
        try:
            out = run(L)
            check_f32(out, ref, f"mxfp4 expert-major tiles={tiles} rt={rt} {shape}")
            x, ids, w = md.layer_device_inputs(L)
            a_ws = md.moe_decode_gate_up(x, ids, L.wg_q, L.wg_s, L.wu_q, L.wu_s, wformat=WF)
            y = torch.full((B * k * H,), float("nan"), dtype=torch.float32, device="cuda")
            out2 = md.moe_decode_down(a_ws, ids, w, L.wd_q, L.wd_s, out_dtype=torch.float32, wformat=WF,
                                      partials=y)
            torch.cuda.synchronize()
            assert torch.equal(out2, out)
            # bf16 intermediate (the B operand is the bf16 value itself): close to the per-output
            # kernel on the same intermediate
            o16 = run(L, inter_dtype=torch.bfloat16)
            md.set_default_tuning("dn_group=0")
            p16 = run(L, inter_dtype=torch.bfloat16)
            rms = float(np.sqrt(np.mean(ref ** 2)))
            assert float((o16 - p16).abs().max()) <= 1e-4 * rms
        finally:
            md.set_default_tuning(None)
