"""moe_decode_noalloc: the layer with the library's device scratch array instead of a
workspace (for callers that cannot allocate). Through the C-ABI it must give the same bits as
moe_decode on consecutive calls whose sizes shrink (the array keeps the previous call's
contents), match the oracle, and reject sizes beyond its 32 MiB before launching anything."""
import ctypes
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _oracle(L, toks):
    sel = sorted({int(e) for e in L.ids[toks].ravel()})
    remap = np.full(L.shape.E, -1, np.int64)
    remap[sel] = np.arange(len(sel))
    idx = torch.tensor(sel, device=L.wg_q.device)
    pick = lambda t: t.index_select(0, idx).cpu()
    return oracle.moe_decode(np.ascontiguousarray(L.x[toks]), np.ascontiguousarray(remap[L.ids[toks]].astype(np.int32)),
                             np.ascontiguousarray(L.w[toks]), pick(L.wg_q), pick(L.wg_s), pick(L.wu_q),
                             pick(L.wu_s), pick(L.wd_q), pick(L.wd_s), wformat=L.wformat)


@pytest.mark.parametrize("wformat,names", [
    ("mxfp8", ["batch_B32_E128_k8_H4096_I1536", "wide_B1_E128_k8_H2048_I768", "tiny_B1_E8_k2_H256_I128"]),
    ("mxfp4", ["batch_B8_E128_k8_H2048_I768", "tiny_B1_E8_k2_H256_I128"])])
def test_no_alloc_matches_moe_decode(wformat, names):
    assert torch.cuda.is_available()
    md.load()
    for name in names:                     # each call smaller than the one before
        say(f"no-alloc entry point: {name} {wformat}")
        L = synth.make_layer(name, device="cuda", wformat=wformat)
        x, ids, w = md.layer_device_inputs(L)
        args = (x, ids, w, L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s)
        for od in (torch.float32, torch.bfloat16):
            for idt in (torch.float32, torch.bfloat16):
                ref = md.moe_decode(*args, out_dtype=od, inter_dtype=idt, wformat=wformat)
                got = torch.full_like(ref, float("nan"))
                md.moe_decode_noalloc(*args, got, inter_dtype=idt, wformat=wformat)
                torch.cuda.synchronize()
                assert torch.equal(got.view(torch.int16 if od == torch.bfloat16 else torch.int32),
                                   ref.view(torch.int16 if od == torch.bfloat16 else torch.int32)), (name, od, idt)
        got = torch.empty((L.shape.B, L.shape.H), dtype=torch.float32, device="cuda")
        md.moe_decode_noalloc(*args, got, wformat=wformat)
        torch.cuda.synchronize()
        toks = list(range(L.shape.B))
        r = _oracle(L, toks)
        err = float(np.abs(got.double().cpu().numpy() - r).max())
        rms = math.sqrt(float(np.mean(r ** 2)))
        say(f"  max|err|/rms = {err / rms:.3e}")
        assert err <= TOL * rms
        del L, x, ids, w, args
        torch.cuda.empty_cache()


def test_no_alloc_rejects_sizes_beyond_its_scratch():
    """B*k*H*4 bytes of partials alone beyond 32 MiB: MOED_ERR_WORKSPACE, before any launch
    (the small tensors passed are never read)."""
    lib = md.load()
    t = torch.zeros(64, dtype=torch.uint8, device="cuda")
    p = ctypes.c_void_p(t.data_ptr())
    B, E, k, H, I = 128, 8, 8, 8192, 1024
    st = lib.moe_decode_noalloc(p, p, p, p, p, p, p, p, p, 0, p, 1, 1, B, E, k, H, I, None)
    assert st == md.MOED_ERR_WORKSPACE
    assert lib.moed_workspace_bytes(B, k, H, I, 1) > 32 << 20
    # the largest decode workload fits
    assert lib.moed_workspace_bytes(64, 8, 7168, 2048, 1) <= 32 << 20
