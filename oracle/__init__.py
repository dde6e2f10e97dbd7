"""CPU oracle for the MoE decode expert layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package; the product path (``output_centric_expert_amd``)
never does. It wraps ``moe_oracle.c`` (plain C, float64 throughout) through
ctypes and takes/returns numpy arrays on the host.

Parity pins: every function here is pinned in ``tests/test_oracle_pins.py``
against the format definitions, a library float8 decoder, a dense SwiGLU MLP,
the brute-force matrix form, and the routing invariants.
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


def bf16_value(bits: int) -> float:
    return _load().oracle_bf16_value(bits)


def threads(n: int = 0) -> int:
    return _load().oracle_threads(n)


def _dims(B, E, k, H, I):
    return [ctypes.c_int(v) for v in (B, E, k, H, I)]


def gate_up(x, ids, wg_q, wg_s, wu_q, wu_s, E, nthreads=0):
    """a[b, j, i] = SiLU(gate) * up in float64, shape [B, k, I]."""
    x = _host(x, np.uint16); ids = _host(ids, np.int32)
    wg_q = _host(wg_q, np.uint8); wg_s = _host(wg_s, np.uint8)
    wu_q = _host(wu_q, np.uint8); wu_s = _host(wu_s, np.uint8)
    B, H = x.shape; k = ids.shape[1]; I = wg_q.shape[1]
    assert wg_q.shape == (E, I, H) and wu_q.shape == (E, I, H)
    assert wg_s.shape == (E, I, H // 32) and wu_s.shape == (E, I, H // 32)
    a = np.empty((B, k, I), np.float64)
    rc = _load().oracle_gate_up(_p(x), _p(ids), _p(wg_q), _p(wg_s), _p(wu_q), _p(wu_s),
                                *_dims(B, E, k, H, I), _p(a), nthreads)
    if rc:
        raise ValueError(f"oracle_gate_up failed ({rc})")
    return a


def down(a, ids, w, wd_q, wd_s, E, nthreads=0):
    """out[b, h] = sum_j w[b, j] * (Wd^[e_j] @ a[b, j])[h] in float64, shape [B, H]."""
    a = _host(a, np.float64); ids = _host(ids, np.int32); w = _host(w, np.float32)
    wd_q = _host(wd_q, np.uint8); wd_s = _host(wd_s, np.uint8)
    B, k, I = a.shape; H = wd_q.shape[1]
    assert wd_q.shape == (E, H, I) and wd_s.shape == (E, H, I // 32)
    assert ids.shape == (B, k) and w.shape == (B, k)
    out = np.empty((B, H), np.float64)
    rc = _load().oracle_down(_p(a), _p(ids), _p(w), _p(wd_q), _p(wd_s),
                             *_dims(B, E, k, H, I), _p(out), nthreads)
    if rc:
        raise ValueError(f"oracle_down failed ({rc})")
    return out


def moe_decode(x, ids, w, wg_q, wg_s, wu_q, wu_s, wd_q, wd_s, return_inter=False, nthreads=0):
    """The whole layer in float64: out [B, H] (and a [B, k, I] when asked)."""
    x = _host(x, np.uint16); ids = _host(ids, np.int32); w = _host(w, np.float32)
    arrs = [_host(t, np.uint8) for t in (wg_q, wg_s, wu_q, wu_s, wd_q, wd_s)]
    B, H = x.shape; k = ids.shape[1]; E, I = arrs[0].shape[:2]
    assert arrs[0].shape == (E, I, H) and arrs[2].shape == (E, I, H)
    assert arrs[1].shape == (E, I, H // 32) and arrs[3].shape == (E, I, H // 32)
    assert arrs[4].shape == (E, H, I) and arrs[5].shape == (E, H, I // 32)
    assert w.shape == (B, k)
    out = np.empty((B, H), np.float64)
    a = np.empty((B, k, I), np.float64) if return_inter else None
    rc = _load().oracle_moe_decode(_p(x), _p(ids), _p(w), *[_p(t) for t in arrs],
                                   *_dims(B, E, k, H, I), _p(out),
                                   _p(a) if a is not None else None, nthreads)
    if rc:
        raise ValueError(f"oracle_moe_decode failed ({rc})")
    return (out, a) if return_inter else out


def moe_decode_layer(L, return_inter=False, nthreads=0):
    """Convenience: run the oracle on a ``synth.LayerInputs``."""
    return moe_decode(L.x, L.ids, L.w, L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s,
                      return_inter=return_inter, nthreads=nthreads)
