"""ctypes binding of libmoedecode (include/moedecode.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. Tensors are torch CUDA tensors (device memory on the current device);
the stream is torch's current stream unless one is given. There is no CPU
fallback -- if the shared library is missing or fails to load, importing the
functions raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoedecode.so")

(MOED_OK, MOED_ERR_NULL, MOED_ERR_SHAPE, MOED_ERR_DTYPE, MOED_ERR_WORKSPACE, MOED_ERR_ALIGN, MOED_ERR_HIP,
 MOED_ERR_SCALE, MOED_ERR_TUNING) = range(9)
MOED_BF16, MOED_F32 = 0, 1

EXPORTS = ("moed_workspace_bytes", "moe_decode", "moe_decode_gate_up", "moe_decode_down", "moe_route",
           "moed_selftest_decode", "moed_bench_read", "moed_bench_copy", "moed_status_string",
           "moed_last_hip_error", "moed_tuning_init", "moe_decode_tuned", "moe_decode_gate_up_tuned",
           "moe_decode_down_tuned", "moe_decode_noalloc", "moed_bench_read_cfg")


class MoedTuning(ctypes.Structure):
    """moed_tuning of the header: a launch-shape choice handed to one call."""
    _fields_ = [("words", ctypes.c_int32 * 48)]


class MoedError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        msg = lib.moed_status_string(status).decode()
        if status == MOED_ERR_HIP:
            msg += f" (hipError {lib.moed_last_hip_error()})"
        super().__init__(f"{where}: {msg}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libmoedecode.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} not built: run __graft_entry__.build() "
                              "(or python -m output_centric_expert_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        lib.moed_workspace_bytes.argtypes = [I, I, I, I, I]
        lib.moed_workspace_bytes.restype = Z
        lib.moe_decode.argtypes = [P] * 9 + [I, P] + [I] * 7 + [P, Z, P]
        lib.moe_decode.restype = I
        lib.moe_decode_gate_up.argtypes = [P] * 6 + [I, P] + [I] * 6 + [P]
        lib.moe_decode_gate_up.restype = I
        lib.moe_decode_down.argtypes = [P, I, P, P, P, P, I, P, I] + [I] * 5 + [P, Z, P]
        lib.moe_decode_down.restype = I
        lib.moe_decode_noalloc.argtypes = [P] * 9 + [I, P] + [I] * 7 + [P]
        lib.moe_decode_noalloc.restype = I
        TP = ctypes.POINTER(MoedTuning)
        lib.moed_tuning_init.argtypes = [TP, ctypes.c_char_p]
        lib.moed_tuning_init.restype = I
        lib.moe_decode_tuned.argtypes = lib.moe_decode.argtypes + [TP]
        lib.moe_decode_tuned.restype = I
        lib.moe_decode_gate_up_tuned.argtypes = lib.moe_decode_gate_up.argtypes + [TP]
        lib.moe_decode_gate_up_tuned.restype = I
        lib.moe_decode_down_tuned.argtypes = lib.moe_decode_down.argtypes + [TP]
        lib.moe_decode_down_tuned.restype = I
        lib.moe_route.argtypes = [P, I, I, I, I, ctypes.c_float, P, P, P]
        lib.moe_route.restype = I
        lib.moed_selftest_decode.argtypes = [P, P, P, I, I, P]
        lib.moed_selftest_decode.restype = I
        lib.moed_bench_read.argtypes = [P, Z, P, Z, P]
        lib.moed_bench_read.restype = I
        lib.moed_bench_read_cfg.argtypes = [P, Z, P, Z, I, I, I, P]
        lib.moed_bench_read_cfg.restype = I
        lib.moed_bench_copy.argtypes = [P, P, Z, P]
        lib.moed_bench_copy.restype = I
        lib.moed_status_string.argtypes = [I]
        lib.moed_status_string.restype = ctypes.c_char_p
        lib.moed_last_hip_error.argtypes = []
        lib.moed_last_hip_error.restype = I
        _lib = lib
    return _lib


_DT = {torch.bfloat16: MOED_BF16, torch.float32: MOED_F32}


def _ptr(t: torch.Tensor | None, name: str, dtype=None, shape=None, cuda=True):
    if t is None:
        return None
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if cuda and not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else ctypes.c_void_p(0)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(st: int, where: str):
    if st != MOED_OK:
        raise MoedError(st, where)


def moed_tuning_init(spec: str | None) -> MoedTuning:
    """A moed_tuning filled from the built-in table and `spec` ("key=value,...")."""
    t = MoedTuning()
    _check(load().moed_tuning_init(ctypes.byref(t), spec.encode() if spec else None), "moed_tuning_init")
    return t


_default = threading.local()


def set_default_tuning(spec: str | None):
    """Later calls made by this Python thread without a tuning argument pass a moed_tuning
    filled from `spec` (None: the built-in table). A convenience of the binding for tests and
    sweeps; the library itself keeps no state between calls."""
    _default.tuning = moed_tuning_init(spec) if spec else None


@contextlib.contextmanager
def tuned(spec: str | None):
    """set_default_tuning(spec) for the calls inside the block."""
    prev = getattr(_default, "tuning", None)
    set_default_tuning(spec)
    try:
        yield
    finally:
        _default.tuning = prev


def _tuning(tuning):
    """tuning argument -> (use the _tuned entry point?, pointer)."""
    if tuning is None:
        tuning = getattr(_default, "tuning", None)
    elif isinstance(tuning, str):
        tuning = moed_tuning_init(tuning)
    return (tuning is not None), (ctypes.byref(tuning) if tuning is not None else None)


def moed_workspace_bytes(B: int, k: int, H: int, I: int, inter_dtype=torch.float32) -> int:
    """Workspace of moe_decode: the intermediate (256-byte aligned), then B*k*H float32 partials."""
    return int(load().moed_workspace_bytes(B, k, H, I, _DT[inter_dtype]))


_WF = {"mxfp8": 0, "mxfp4": 1}          # moed_wformat


def _kb(K: int, wformat: str) -> int:
    """Code bytes per row of K values."""
    if wformat not in _WF:
        raise ValueError(f"unknown weight format {wformat!r}")
    return K // 2 if wformat == "mxfp4" else K


def moe_decode(x, topk_ids, topk_w, wg_q, wg_s, wu_q, wu_s, wd_q, wd_s, out=None,
               out_dtype=torch.bfloat16, inter_dtype=torch.float32, workspace=None, stream=None,
               wformat="mxfp8", tuning=None):
    """The whole layer: returns out [B, H] (out_dtype). wformat: "mxfp8" or "mxfp4"
    (codes [E, I, H/2] and [E, H, I/2], two per byte, low nibble first). tuning: None (the
    built-in table, or the one of an enclosing tuned() block), a spec string or a MoedTuning."""
    B, H = x.shape
    k = topk_ids.shape[1]
    E, I = wg_q.shape[0], wg_q.shape[1]
    HB, IB = _kb(H, wformat), _kb(I, wformat)
    if out is None:
        out = torch.empty((B, H), dtype=out_dtype, device=x.device)
    need = moed_workspace_bytes(B, k, H, I, inter_dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    use, tp = _tuning(tuning)
    lib = load()
    args = (
        _ptr(x, "x", torch.bfloat16, (B, H)), _ptr(topk_ids, "topk_ids", torch.int32, (B, k)),
        _ptr(topk_w, "topk_w", torch.float32, (B, k)),
        _ptr(wg_q, "wg_q", torch.uint8, (E, I, HB)), _ptr(wg_s, "wg_s", torch.uint8, (E, I, H // 32)),
        _ptr(wu_q, "wu_q", torch.uint8, (E, I, HB)), _ptr(wu_s, "wu_s", torch.uint8, (E, I, H // 32)),
        _ptr(wd_q, "wd_q", torch.uint8, (E, H, IB)), _ptr(wd_s, "wd_s", torch.uint8, (E, H, I // 32)),
        _WF[wformat], _ptr(out, "out", None, (B, H)), _DT[out.dtype], _DT[inter_dtype],
        B, E, k, H, I, _ptr(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream))
    st = lib.moe_decode_tuned(*args, tp) if use else lib.moe_decode(*args)
    _check(st, "moe_decode")
    return out


def moe_decode_noalloc(x, topk_ids, topk_w, wg_q, wg_s, wu_q, wu_s, wd_q, wd_s, out,
                       inter_dtype=torch.float32, stream=None, wformat="mxfp8"):
    """The whole layer into the caller's `out` [B, H] (bf16 or float32) with the library's
    device scratch array instead of a workspace: the call allocates nothing."""
    B, H = x.shape
    k = topk_ids.shape[1]
    E, I = wg_q.shape[0], wg_q.shape[1]
    HB, IB = _kb(H, wformat), _kb(I, wformat)
    st = load().moe_decode_noalloc(
        _ptr(x, "x", torch.bfloat16, (B, H)), _ptr(topk_ids, "topk_ids", torch.int32, (B, k)),
        _ptr(topk_w, "topk_w", torch.float32, (B, k)),
        _ptr(wg_q, "wg_q", torch.uint8, (E, I, HB)), _ptr(wg_s, "wg_s", torch.uint8, (E, I, H // 32)),
        _ptr(wu_q, "wu_q", torch.uint8, (E, I, HB)), _ptr(wu_s, "wu_s", torch.uint8, (E, I, H // 32)),
        _ptr(wd_q, "wd_q", torch.uint8, (E, H, IB)), _ptr(wd_s, "wd_s", torch.uint8, (E, H, I // 32)),
        _WF[wformat], _ptr(out, "out", None, (B, H)), _DT[out.dtype], _DT[inter_dtype],
        B, E, k, H, I, _stream(stream))
    _check(st, "moe_decode_noalloc")
    return out


def moe_decode_gate_up(x, topk_ids, wg_q, wg_s, wu_q, wu_s, a=None, inter_dtype=torch.float32,
                       stream=None, wformat="mxfp8", tuning=None):
    """Gate/up step alone: returns a = SiLU(gate) * up, shape [B, k, I] in the
    library's chunk-interleaved element order (inter_to_bki() gives plain order)."""
    B, H = x.shape
    k = topk_ids.shape[1]
    E, I = wg_q.shape[0], wg_q.shape[1]
    HB = _kb(H, wformat)
    if a is None:
        a = torch.empty((B, k, I), dtype=inter_dtype, device=x.device)
    use, tp = _tuning(tuning)
    lib = load()
    args = (
        _ptr(x, "x", torch.bfloat16, (B, H)), _ptr(topk_ids, "topk_ids", torch.int32, (B, k)),
        _ptr(wg_q, "wg_q", torch.uint8, (E, I, HB)), _ptr(wg_s, "wg_s", torch.uint8, (E, I, H // 32)),
        _ptr(wu_q, "wu_q", torch.uint8, (E, I, HB)), _ptr(wu_s, "wu_s", torch.uint8, (E, I, H // 32)),
        _WF[wformat], _ptr(a, "a", None, (B, k, I)), _DT[a.dtype], B, E, k, H, I, _stream(stream))
    st = lib.moe_decode_gate_up_tuned(*args, tp) if use else lib.moe_decode_gate_up(*args)
    _check(st, "moe_decode_gate_up")
    return a


def moe_decode_down(a, topk_ids, topk_w, wd_q, wd_s, out=None, out_dtype=torch.bfloat16, stream=None,
                    wformat="mxfp8", partials=None, tuning=None):
    """Down step alone: returns out [B, H] from a [B, k, I]. partials: None (one wavefront per
    output) or a float32 CUDA tensor of at least B*k*H elements, which lets batches whose
    tokens share experts take the expert-major form."""
    B, k, I = a.shape
    E, H = wd_q.shape[0], wd_q.shape[1]
    IB = _kb(I, wformat)
    if out is None:
        out = torch.empty((B, H), dtype=out_dtype, device=a.device)
    pp, pn = None, 0
    if partials is not None:
        pp = _ptr(partials, "partials", torch.float32)
        pn = partials.numel() * 4
    use, tp = _tuning(tuning)
    lib = load()
    args = (
        _ptr(a, "a", None, (B, k, I)), _DT[a.dtype], _ptr(topk_ids, "topk_ids", torch.int32, (B, k)),
        _ptr(topk_w, "topk_w", torch.float32, (B, k)),
        _ptr(wd_q, "wd_q", torch.uint8, (E, H, IB)), _ptr(wd_s, "wd_s", torch.uint8, (E, H, I // 32)),
        _WF[wformat], _ptr(out, "out", None, (B, H)), _DT[out.dtype], B, E, k, H, I, pp, pn,
        _stream(stream))
    st = lib.moe_decode_down_tuned(*args, tp) if use else lib.moe_decode_down(*args)
    _check(st, "moe_decode_down")
    return out


def moe_route(logits, k: int, n_shared: int = 0, routed_scale: float = 1.0, ids=None, w=None, stream=None):
    """Router front-end on the GPU: (topk_ids int32 [B, k+n_shared], topk_w float32 [B, k+n_shared])
    from float32 logits [B, E]; shared slots get ids E, E+1, ... and weight 1."""
    B, E = logits.shape
    kt = k + n_shared
    if ids is None:
        ids = torch.empty((B, kt), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((B, kt), dtype=torch.float32, device=logits.device)
    st = load().moe_route(_ptr(logits, "logits", torch.float32, (B, E)), B, E, k, n_shared, float(routed_scale),
                          _ptr(ids, "topk_ids", torch.int32, (B, kt)), _ptr(w, "topk_w", torch.float32, (B, kt)),
                          _stream(stream))
    _check(st, "moe_route")
    return ids, w


def moed_selftest_decode(codes, scales, path: int, out=None, stream=None):
    """Decode codes[t] * 2^(scales[t]-127) with the kernels' decoder; float32 result."""
    n = codes.numel()
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=codes.device)
    st = load().moed_selftest_decode(_ptr(codes, "codes", torch.uint8), _ptr(scales, "scales", torch.uint8),
                                     _ptr(out, "out", torch.float32), n, path, _stream(stream))
    _check(st, "moed_selftest_decode")
    return out


def moed_bench_read(src: torch.Tensor, sink: torch.Tensor, nbytes: int | None = None, stream=None):
    """Stream-read `nbytes` (default: all) of `src` with the contiguous read kernel."""
    n = src.numel() * src.element_size() if nbytes is None else nbytes
    _check(load().moed_bench_read(_ptr(src, "src"), n, _ptr(sink, "sink"), sink.numel() * sink.element_size(),
                                  _stream(stream)), "moed_bench_read")


def moed_bench_read_cfg(src: torch.Tensor, sink: torch.Tensor, nbytes: int, unroll: int, waves_per_group: int,
                        groups: int = 0, stream=None):
    """The read probe with a chosen launch shape (see the header)."""
    _check(load().moed_bench_read_cfg(_ptr(src, "src"), nbytes, _ptr(sink, "sink"), sink.numel() * sink.element_size(),
                                      unroll, waves_per_group, groups, _stream(stream)), "moed_bench_read_cfg")


def moed_bench_copy(src: torch.Tensor, dst: torch.Tensor, nbytes: int | None = None, stream=None):
    n = src.numel() * src.element_size() if nbytes is None else nbytes
    if n > dst.numel() * dst.element_size():
        raise ValueError("moed_bench_copy: dst too small")
    _check(load().moed_bench_copy(_ptr(src, "src"), _ptr(dst, "dst"), n, _stream(stream)), "moed_bench_copy")


def moed_status_string(status: int) -> str:
    return load().moed_status_string(status).decode()


def moed_last_hip_error() -> int:
    return load().moed_last_hip_error()


def inter_to_bki(a: torch.Tensor) -> torch.Tensor:
    """Reorder the library's chunk-interleaved intermediate (see the header) to plain [B, k, I]."""
    B, k, I = a.shape
    q, per = (2, 8) if a.dtype == torch.bfloat16 else (4, 4)
    return a.reshape(B * k, q, I // 16, per).permute(0, 2, 1, 3).reshape(B, k, I)


def layer_device_inputs(L, device="cuda"):
    """Host parts of a synth.LayerInputs -> device tensors (x bf16, ids int32, w f32)."""
    x = torch.from_numpy(L.x.view("int16")).view(torch.bfloat16).to(device)
    ids = torch.from_numpy(L.ids).to(device)
    w = torch.from_numpy(L.w).to(device)
    return x, ids, w
