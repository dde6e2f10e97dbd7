"""Host-side checks of the C-ABI library: it loads, exports every function the
header declares, and rejects bad arguments before launching anything (so these
run without a GPU)."""
import ctypes
import os
import re

import pytest

from output_centric_expert_amd import moedecode as md

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moedecode.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(md.LIB_PATH):
        from output_centric_expert_amd import build
        build.build_library()
    return md.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_expected_functions():
    assert header_functions() == sorted(md.EXPORTS)


def test_library_exports_every_header_function(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {md.LIB_PATH}").read()
    for name in header_functions():
        assert re.search(rf"\bT {name}\b", out), name


def test_status_strings(lib):
    for s in range(9):
        assert md.moed_status_string(s).startswith("MOED_")
    assert "unknown" in md.moed_status_string(99)
    assert md.moed_last_hip_error() == 0


def test_workspace_bytes(lib):
    # the intermediate rounded up to 256 bytes, then B*k*H float32 partials
    assert lib.moed_workspace_bytes(1, 8, 2048, 768, md.MOED_F32) == 8 * 768 * 4 + 8 * 2048 * 4
    assert lib.moed_workspace_bytes(64, 8, 7168, 2048, md.MOED_BF16) == 64 * 8 * 2048 * 2 + 64 * 8 * 7168 * 4
    assert lib.moed_workspace_bytes(1, 2, 256, 48, md.MOED_BF16) == 256 + 2 * 256 * 4     # 192 -> 256
    assert lib.moed_workspace_bytes(0, 8, 2048, 768, md.MOED_F32) == 0
    assert lib.moed_workspace_bytes(1, 8, 2048, 768, 7) == 0
    assert lib.moed_workspace_bytes(1, 8, 0, 768, md.MOED_F32) == 0


P = ctypes.c_void_p
A = P(4096)          # a fake, 16-byte-aligned non-null address: never dereferenced
MIS = P(4100)        # misaligned


def call_decode(lib, x=A, ids=A, w=A, wq=A, ws=A, out=A, od=0, idt=1, B=1, E=8, k=2, H=256, I=128,
                wsp=A, wsb=1 << 20, wf=0):
    return lib.moe_decode(x, ids, w, wq, ws, wq, ws, wq, ws, wf, out, od, idt, B, E, k, H, I, wsp, wsb, None)


def test_decode_rejects_before_launch(lib):
    assert call_decode(lib, x=None) == md.MOED_ERR_NULL
    assert call_decode(lib, ws=None) == md.MOED_ERR_NULL
    assert call_decode(lib, wsp=None) == md.MOED_ERR_NULL
    assert call_decode(lib, k=0) == md.MOED_ERR_SHAPE
    assert call_decode(lib, k=9) == md.MOED_ERR_SHAPE          # k > E
    assert call_decode(lib, H=250) == md.MOED_ERR_SHAPE        # not a multiple of 32
    assert call_decode(lib, I=16) == md.MOED_ERR_SHAPE
    assert call_decode(lib, B=-1) == md.MOED_ERR_SHAPE
    assert call_decode(lib, E=0, k=0) == md.MOED_ERR_SHAPE
    assert call_decode(lib, B=1 << 20, H=4096) == md.MOED_ERR_SHAPE   # B*H >= 2^31
    assert call_decode(lib, od=2) == md.MOED_ERR_DTYPE
    assert call_decode(lib, idt=-1) == md.MOED_ERR_DTYPE
    assert call_decode(lib, wf=2) == md.MOED_ERR_DTYPE          # unknown weight format
    assert call_decode(lib, wf=-1) == md.MOED_ERR_DTYPE
    assert call_decode(lib, wf=1, x=None) == md.MOED_ERR_NULL   # MXFP4 goes through the same checks
    assert call_decode(lib, wsb=1 * 2 * 128 * 4 - 1) == md.MOED_ERR_WORKSPACE
    assert call_decode(lib, wsb=1 * 2 * 128 * 4 + 1 * 2 * 256 * 4 - 1) == md.MOED_ERR_WORKSPACE   # no room for the partials
    assert call_decode(lib, x=MIS) == md.MOED_ERR_ALIGN
    assert call_decode(lib, wq=MIS) == md.MOED_ERR_ALIGN
    assert call_decode(lib, wsp=MIS) == md.MOED_ERR_ALIGN
    # B = 0 is a valid empty call: nothing launched, even with NULL pointers
    assert call_decode(lib, B=0, x=None, out=None, wsp=None, wsb=0) == md.MOED_OK


def test_step_entry_points_reject_before_launch(lib):
    gu = lambda **kw: lib.moe_decode_gate_up(kw.get("x", A), A, A, A, A, A, kw.get("wf", 0), kw.get("a", A),
                                             kw.get("idt", 1), kw.get("B", 1), 8, kw.get("k", 2), 256, 128, None)
    assert gu(x=None) == md.MOED_ERR_NULL
    assert gu(a=MIS) == md.MOED_ERR_ALIGN
    assert gu(idt=5) == md.MOED_ERR_DTYPE
    assert gu(wf=3) == md.MOED_ERR_DTYPE
    assert gu(k=0) == md.MOED_ERR_SHAPE
    assert gu(B=0, x=None) == md.MOED_OK
    dn = lambda **kw: lib.moe_decode_down(kw.get("a", A), 1, A, A, kw.get("wq", A), A, kw.get("wf", 0),
                                          kw.get("out", A), kw.get("od", 0), 1, 8, 2, 256, 128,
                                          kw.get("y", None), kw.get("yb", 0), None)
    assert dn(out=None) == md.MOED_ERR_NULL
    assert dn(y=A, yb=2 * 256 * 4 - 4) == md.MOED_ERR_WORKSPACE       # partials below B*k*H floats
    assert dn(y=MIS, yb=2 * 256 * 4) == md.MOED_ERR_ALIGN
    assert dn(wq=MIS) == md.MOED_ERR_ALIGN
    assert dn(od=3) == md.MOED_ERR_DTYPE
    assert dn(wf=7) == md.MOED_ERR_DTYPE
    assert lib.moed_selftest_decode(A, A, A, 4, 6, None) == md.MOED_ERR_SHAPE
    assert lib.moed_selftest_decode(A, A, A, 4, -1, None) == md.MOED_ERR_SHAPE
    assert lib.moed_selftest_decode(None, A, A, 4, 0, None) == md.MOED_ERR_NULL
    assert lib.moed_selftest_decode(None, None, None, 0, 0, None) == md.MOED_OK


def test_route_rejects_before_launch(lib):
    rt = lambda **kw: lib.moe_route(kw.get("lg", A), kw.get("B", 2), kw.get("E", 128), kw.get("k", 8),
                                    kw.get("ns", 0), 1.0, kw.get("ids", A), kw.get("w", A), None)
    assert rt(lg=None) == md.MOED_ERR_NULL
    assert rt(ids=None) == md.MOED_ERR_NULL
    assert rt(k=0) == md.MOED_ERR_SHAPE
    assert rt(k=129) == md.MOED_ERR_SHAPE            # k > E
    assert rt(E=4096, k=8) == md.MOED_ERR_SHAPE      # E above the router's 2048
    assert rt(E=256, k=65) == md.MOED_ERR_SHAPE      # k above 64
    assert rt(ns=-1) == md.MOED_ERR_SHAPE
    assert rt(B=-1) == md.MOED_ERR_SHAPE
    assert rt(B=0, lg=None, ids=None, w=None) == md.MOED_OK


def _init(lib, spec):
    t = md.MoedTuning()
    return lib.moed_tuning_init(ctypes.byref(t), spec)


def test_tuning_spec_parser(lib):
    """moed_tuning_init: the built-in table plus key=value overrides, filled into the caller's struct."""
    assert _init(lib, b"gu_wpb=2,dn_wpb=1,gu_umax=3") == md.MOED_OK
    assert _init(lib, b"gu_wpb=9") == md.MOED_ERR_SHAPE
    assert _init(lib, b"gu_group=1,dn_stage=0") == md.MOED_OK
    assert _init(lib, b"gu_group=3") == md.MOED_ERR_SHAPE
    assert _init(lib, b"dn_group=1") == md.MOED_OK
    assert _init(lib, b"dn_group=-1") == md.MOED_ERR_SHAPE
    assert _init(lib, b"dn_group=1,dn_tiles=4") == md.MOED_OK
    assert _init(lib, b"dn_tiles=0") == md.MOED_OK
    assert _init(lib, b"dn_tiles=5") == md.MOED_ERR_SHAPE
    assert _init(lib, b"dn_rt=1") == md.MOED_OK
    assert _init(lib, b"gu_wide=0") == md.MOED_OK
    assert _init(lib, b"gu_wide=1") == md.MOED_OK
    assert _init(lib, b"gu_wide=2") == md.MOED_ERR_SHAPE
    assert _init(lib, b"dn_rt=0") == md.MOED_ERR_SHAPE
    assert _init(lib, b"dn_rt=3") == md.MOED_ERR_SHAPE
    assert _init(lib, b"dn_lanegroups=0") == md.MOED_OK
    assert _init(lib, b"dn_lanegroups=2") == md.MOED_ERR_SHAPE
    for gone in (b"gu_dot=1", b"gu_npw=1", b"nt=2", b"dn_order=1", b"dn_rows=0", b"gu_rowslots=2"):   # removed knobs
        assert _init(lib, gone) == md.MOED_ERR_SHAPE
    assert _init(lib, b"dn_onepass=0") == md.MOED_OK
    assert _init(lib, b"dn_onepass=2") == md.MOED_ERR_SHAPE
    assert _init(lib, b"dn_wide=0") == md.MOED_OK
    assert _init(lib, b"dn_wide=1") == md.MOED_OK
    assert _init(lib, b"dn_wide=2") == md.MOED_ERR_SHAPE
    assert _init(lib, b"gu_pair=0") == md.MOED_OK
    assert _init(lib, b"gu_pair=2") == md.MOED_ERR_SHAPE
    assert _init(lib, b"dn_pair=0") == md.MOED_OK
    assert _init(lib, b"dn_pair=2") == md.MOED_ERR_SHAPE
    assert _init(lib, b"dn_split=0") == md.MOED_OK
    assert _init(lib, b"dn_split=2") == md.MOED_ERR_SHAPE
    assert _init(lib, b"gu_order=0") == md.MOED_OK
    assert _init(lib, b"gu_order=2") == md.MOED_OK
    assert _init(lib, b"gu_order=3") == md.MOED_ERR_SHAPE
    assert _init(lib, b"gu_exact=0") == md.MOED_OK
    assert _init(lib, b"gu_exact=2") == md.MOED_ERR_SHAPE
    assert _init(lib, b"gu_waves=0") == md.MOED_OK
    assert _init(lib, b"gu_waves=4") == md.MOED_OK
    assert _init(lib, b"gu_waves=8") == md.MOED_OK
    assert _init(lib, b"gu_waves=2") == md.MOED_ERR_SHAPE
    assert _init(lib, b"gu_grid=0,dn_grid=65536") == md.MOED_OK
    assert _init(lib, b"dn_grid=-1") == md.MOED_ERR_SHAPE
    assert _init(lib, b"grp_grid=1") == md.MOED_ERR_SHAPE
    assert _init(lib, b"bogus=1") == md.MOED_ERR_SHAPE
    assert _init(lib, b"gu_wpb") == md.MOED_ERR_SHAPE
    assert _init(lib, None) == md.MOED_OK


def test_tuning_struct_is_per_call(lib):
    """A moed_tuning is the caller's value: filled only by moed_tuning_init, checked by the *_tuned
    calls before anything else is looked at (MOED_ERR_TUNING for one it did not fill), and NULL
    means the built-in table. Nothing is launched here (argument errors come first)."""
    assert lib.moed_tuning_init(None, b"gu_group=0") == md.MOED_ERR_NULL
    t = md.MoedTuning()
    assert lib.moed_tuning_init(ctypes.byref(t), None) == md.MOED_OK
    u = md.MoedTuning()
    assert lib.moed_tuning_init(ctypes.byref(u), b"") == md.MOED_OK
    assert bytes(t) == bytes(u)                       # NULL and "" both give the built-in table
    v = md.MoedTuning()
    assert lib.moed_tuning_init(ctypes.byref(v), b"gu_group=0") == md.MOED_OK
    assert bytes(v) != bytes(t)
    bad = md.MoedTuning()                             # never initialised
    Z = ctypes.c_size_t
    # B = 0 launches nothing, but the tuning is checked first
    args = [None] * 9 + [0, None, 0, 0, 0, 8, 2, 256, 128, None, Z(0), None]
    assert lib.moe_decode_tuned(*args, ctypes.byref(bad)) == md.MOED_ERR_TUNING
    assert lib.moe_decode_tuned(*args, ctypes.byref(t)) == md.MOED_OK
    assert lib.moe_decode_tuned(*args, None) == md.MOED_OK
    gu = [None] * 6 + [0, None, 1, 0, 8, 2, 256, 128, None]
    assert lib.moe_decode_gate_up_tuned(*gu, ctypes.byref(bad)) == md.MOED_ERR_TUNING
    assert lib.moe_decode_gate_up_tuned(*gu, ctypes.byref(v)) == md.MOED_OK
    dn = [None, 1, None, None, None, None, 0, None, 1, 0, 8, 2, 256, 128, None, Z(0), None]
    assert lib.moe_decode_down_tuned(*dn, ctypes.byref(bad)) == md.MOED_ERR_TUNING
    assert lib.moe_decode_down_tuned(*dn, None) == md.MOED_OK
    # a shape error is still reported for a good tuning
    args_bad_shape = [None] * 9 + [0, None, 0, 0, 1, 8, 2, 100, 128, None, Z(0), None]
    assert lib.moe_decode_tuned(*args_bad_shape, ctypes.byref(t)) == md.MOED_ERR_SHAPE


def test_no_process_wide_tuning_state(lib):
    """The library exports no setter of process-wide launch state."""
    out = os.popen(f"nm -D --defined-only {md.LIB_PATH}").read()
    assert "moed_set_tuning" not in out


def test_inter_layout_roundtrip():
    """inter_to_bki inverts the documented chunk-interleaved index formula."""
    import torch
    B, k, I = 2, 3, 96
    for dt, q, per in ((torch.float32, 4, 4), (torch.bfloat16, 2, 8)):
        flat = torch.empty(B * k * I, dtype=torch.float32)
        for bj in range(B * k):
            for i in range(I):
                o, r = i // 16, i % per
                qq = (i // per) % q
                flat[((bj * q + qq) * (I // 16) + o) * per + r] = bj * 1000 + i
        plain = md.inter_to_bki(flat.to(dt).reshape(B, k, I)).float()
        want = torch.tensor([[[bj * 1000 + i for i in range(I)] for bj in range(b * k, b * k + k)] for b in range(B)],
                            dtype=torch.float32).to(dt).float()
        assert torch.equal(plain, want)


def test_bench_kernels_reject_before_launch(lib):
    assert lib.moed_bench_read(None, 64, A, 4096, None) == md.MOED_ERR_NULL
    assert lib.moed_bench_read(A, 60, A, 4096, None) == md.MOED_ERR_SHAPE
    assert lib.moed_bench_read(A, 64, A, 1024, None) == md.MOED_ERR_SHAPE   # sink too small
    assert lib.moed_bench_read(MIS, 64, A, 4096, None) == md.MOED_ERR_ALIGN
    assert lib.moed_bench_read(None, 0, None, 0, None) == md.MOED_OK
    rc = lib.moed_bench_read_cfg
    assert rc(None, 64, A, 4096, 1, 4, 0, None) == md.MOED_ERR_NULL
    assert rc(A, 64, A, 4096, 3, 4, 0, None) == md.MOED_ERR_SHAPE      # unroll not 1/2/4/8/16
    assert rc(A, 64, A, 4096, 2, 17, 0, None) == md.MOED_ERR_SHAPE     # more than 16 waves per group
    assert rc(A, 64, A, 4096, 2, 0, 0, None) == md.MOED_ERR_SHAPE
    assert rc(A, 64, A, 4096, 2, 4, -1, None) == md.MOED_ERR_SHAPE
    assert rc(A, 60, A, 4096, 2, 4, 0, None) == md.MOED_ERR_SHAPE
    assert rc(A, 64, A, 1024, 2, 4, 0, None) == md.MOED_ERR_SHAPE
    assert rc(MIS, 64, A, 4096, 2, 4, 0, None) == md.MOED_ERR_ALIGN
    assert rc(None, 0, None, 0, 16, 16, 1024, None) == md.MOED_OK
    assert lib.moed_bench_copy(A, None, 64, None) == md.MOED_ERR_NULL
    assert lib.moed_bench_copy(A, A, 65, None) == md.MOED_ERR_SHAPE
    assert lib.moed_bench_copy(A, MIS, 64, None) == md.MOED_ERR_ALIGN
