"""CPU oracle for the MoE decode expert layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package; the product path (``output_centric_expert_amd``)
never does. It wraps ``moe_oracle.c`` (plain C, float64 throughout) through
ctypes and takes/returns numpy arrays on the host.

Parity pins: every function here is pinned in ``tests/test_oracle_pins.py``
against the format definitions, a library float8 decoder, a dense SwiGLU MLP,
the brute-force matrix form, and the routing invariants; the MXFP4 format in
``tests/test_oracle_fp4.py``.

Weight formats (``wformat``): "mxfp8" -- one E4M3 code per byte, rows of K
bytes; "mxfp4" -- E2M1 codes two per byte (element c in the low nibble of byte
c/2 when c is even, the high nibble when odd), rows of K/2 bytes. Both carry
one UE8M0 scale byte per 32 values along K.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle_moe.so")
SOURCE = os.path.join(_HERE, "moe_oracle.c")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (float64, OpenMP, no fast-math)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-Wextra", "-o", tmp, SOURCE, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oracle_e4m3_value.argtypes = [ctypes.c_uint]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_ue8m0_value.argtypes = [ctypes.c_uint]
        lib.oracle_ue8m0_value.restype = ctypes.c_double
        lib.oracle_bf16_value.argtypes = [ctypes.c_uint]
        lib.oracle_bf16_value.restype = ctypes.c_double
        lib.oracle_gate_up.argtypes = [P] * 6 + [I] * 5 + [P, I]
        lib.oracle_gate_up.restype = I
        lib.oracle_down.argtypes = [P] * 5 + [I] * 5 + [P, I]
        lib.oracle_down.restype = I
        lib.oracle_moe_decode.argtypes = [P] * 9 + [I] * 5 + [P, P, I]
        lib.oracle_moe_decode.restype = I
        lib.oracle_e2m1_value.argtypes = [ctypes.c_uint]
        lib.oracle_e2m1_value.restype = ctypes.c_double
        lib.oracle_gate_up_fmt.argtypes = [P] * 6 + [I] * 5 + [P, I, I]
        lib.oracle_gate_up_fmt.restype = I
        lib.oracle_down_fmt.argtypes = [P] * 5 + [I] * 5 + [P, I, I]
        lib.oracle_down_fmt.restype = I
        lib.oracle_moe_decode_fmt.argtypes = [P] * 9 + [I] * 5 + [P, P, I, I]
        lib.oracle_moe_decode_fmt.restype = I
        lib.oracle_route.argtypes = [P, I, I, I, I, ctypes.c_double, P, P]
        lib.oracle_route.restype = I
        lib.oracle_threads.argtypes = [I]
        lib.oracle_threads.restype = I
        _lib = lib
    return _lib


def _host(a, dtype):
    """numpy (or torch, any device) -> C-contiguous host numpy array of `dtype`."""
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def e4m3_value(code: int) -> float:
    return _load().oracle_e4m3_value(code)


def ue8m0_value(code: int) -> float:
    return _load().oracle_ue8m0_value(code)


def e2m1_value(code: int) -> float:
    return _load().oracle_e2m1_value(code)


_FMT = {"mxfp8": 0, "mxfp4": 1}


def _kbytes(K: int, wformat: str) -> int:
    """Bytes of codes per row of K values."""
    return K // 2 if wformat == "mxfp4" else K


def bf16_value(bits: int) -> float:
    return _load().oracle_bf16_value(bits)


def threads(n: int = 0) -> int:
    return _load().oracle_threads(n)


def _dims(B, E, k, H, I):
    return [ctypes.c_int(v) for v in (B, E, k, H, I)]


def gate_up(x, ids, wg_q, wg_s, wu_q, wu_s, E, nthreads=0, wformat="mxfp8"):
    """a[b, j, i] = SiLU(gate) * up in float64, shape [B, k, I]."""
    x = _host(x, np.uint16); ids = _host(ids, np.int32)
    wg_q = _host(wg_q, np.uint8); wg_s = _host(wg_s, np.uint8)
    wu_q = _host(wu_q, np.uint8); wu_s = _host(wu_s, np.uint8)
    B, H = x.shape; k = ids.shape[1]; I = wg_q.shape[1]
    HB = _kbytes(H, wformat)
    assert wg_q.shape == (E, I, HB) and wu_q.shape == (E, I, HB)
    assert wg_s.shape == (E, I, H // 32) and wu_s.shape == (E, I, H // 32)
    a = np.empty((B, k, I), np.float64)
    rc = _load().oracle_gate_up_fmt(_p(x), _p(ids), _p(wg_q), _p(wg_s), _p(wu_q), _p(wu_s),
                                    *_dims(B, E, k, H, I), _p(a), nthreads, _FMT[wformat])
    if rc:
        raise ValueError(f"oracle_gate_up failed ({rc})")
    return a


def down(a, ids, w, wd_q, wd_s, E, nthreads=0, wformat="mxfp8"):
    """out[b, h] = sum_j w[b, j] * (Wd^[e_j] @ a[b, j])[h] in float64, shape [B, H]."""
    a = _host(a, np.float64); ids = _host(ids, np.int32); w = _host(w, np.float32)
    wd_q = _host(wd_q, np.uint8); wd_s = _host(wd_s, np.uint8)
    B, k, I = a.shape; H = wd_q.shape[1]
    assert wd_q.shape == (E, H, _kbytes(I, wformat)) and wd_s.shape == (E, H, I // 32)
    assert ids.shape == (B, k) and w.shape == (B, k)
    out = np.empty((B, H), np.float64)
    rc = _load().oracle_down_fmt(_p(a), _p(ids), _p(w), _p(wd_q), _p(wd_s),
                                 *_dims(B, E, k, H, I), _p(out), nthreads, _FMT[wformat])
    if rc:
        raise ValueError(f"oracle_down failed ({rc})")
    return out


def moe_decode(x, ids, w, wg_q, wg_s, wu_q, wu_s, wd_q, wd_s, return_inter=False, nthreads=0,
               wformat="mxfp8"):
    """The whole layer in float64: out [B, H] (and a [B, k, I] when asked)."""
    x = _host(x, np.uint16); ids = _host(ids, np.int32); w = _host(w, np.float32)
    arrs = [_host(t, np.uint8) for t in (wg_q, wg_s, wu_q, wu_s, wd_q, wd_s)]
    B, H = x.shape; k = ids.shape[1]; E, I = arrs[0].shape[:2]
    HB, IB = _kbytes(H, wformat), _kbytes(I, wformat)
    assert arrs[0].shape == (E, I, HB) and arrs[2].shape == (E, I, HB)
    assert arrs[1].shape == (E, I, H // 32) and arrs[3].shape == (E, I, H // 32)
    assert arrs[4].shape == (E, H, IB) and arrs[5].shape == (E, H, I // 32)
    assert w.shape == (B, k)
    out = np.empty((B, H), np.float64)
    a = np.empty((B, k, I), np.float64) if return_inter else None
    rc = _load().oracle_moe_decode_fmt(_p(x), _p(ids), _p(w), *[_p(t) for t in arrs],
                                       *_dims(B, E, k, H, I), _p(out),
                                       _p(a) if a is not None else None, nthreads, _FMT[wformat])
    if rc:
        raise ValueError(f"oracle_moe_decode failed ({rc})")
    return (out, a) if return_inter else out


def route(logits, k, n_shared=0, routed_scale=1.0):
    """Router front-end in float64 from float32 logits [B, E]: (ids int32 [B, k+n_shared],
    w float32 [B, k+n_shared]); see oracle_route in moe_oracle.c."""
    logits = _host(logits, np.float32)
    B, E = logits.shape
    kt = k + n_shared
    ids = np.empty((B, kt), np.int32)
    w = np.empty((B, kt), np.float32)
    rc = _load().oracle_route(_p(logits), B, E, k, n_shared, float(routed_scale), _p(ids), _p(w))
    if rc:
        raise ValueError(f"oracle_route failed ({rc})")
    return ids, w


def moe_decode_layer(L, return_inter=False, nthreads=0):
    """Convenience: run the oracle on a ``synth.LayerInputs``."""
    return moe_decode(L.x, L.ids, L.w, L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s,
                      return_inter=return_inter, nthreads=nthreads,
                      wformat=getattr(L, "wformat", "mxfp8"))
