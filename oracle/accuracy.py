"""Accuracy-study references -- TEST INFRASTRUCTURE ONLY (tests, benchmark).

The warp-decode post claims (section "Improved accuracy") that keeping
activations in BF16 with FP32 accumulators lands 1.4x closer to a full 32-bit
reference than the classical expert-centric path, which converts BF16
activations to MXFP8 and back. Two references and one emulation make that
claim measurable here:

* ``reference_dense``: the layer in float64 with the UNQUANTIZED weight draws
  (the values before MXFP8 encoding) and the bf16 activations ("reading A"
  of the full-precision reference).
* ``classical_emulation``: the classical path as the post describes its
  numerics: x quantized to MXFP8 (blocks of 32 along H) before gate/up,
  float32 accumulation, SwiGLU in float32, the intermediate quantized to
  MXFP8 (blocks of 32 along I) before down, float32 accumulation, every
  expert's output rounded to BF16 (the per-expert BF16 output buffer of the
  section "Buffer removal"), combined with the routing weights in float32 and
  rounded to BF16.

Parity status: e4m3_round, mx_quantize, bf16_round and reference_dense are
pinned (library rounding, the independent input encoder, the oracle).
classical_emulation is pinned against a second construction of the same
stages from already-pinned parts (the C oracle's float64 gate/up and down, per
slot, with mx_quantize and bf16_round between them): bit for bit where every
stage is exact, and output for output (at most one BF16 ulp apart, nearly all
identical) on random layers; a copy with any one stage taken out fails.

The MX quantizer here is written from the OCP Microscaling v1.0 rule
(shared exponent floor(log2 amax) - 8, clamped; elements rounded to nearest
even E4M3, saturating at 448) and shares no code with the input generator.
"""
from __future__ import annotations

import numpy as np


def _silu(t):
    return t / (1.0 + np.exp(-t))


def e4m3_round(v: np.ndarray) -> np.ndarray:
    """Round float64 values (|v| <= 448 after clamping) to the nearest-even E4M3 value."""
    v = np.clip(np.asarray(v, np.float64), -448.0, 448.0)
    a = np.abs(v)
    # exponent of the E4M3 bin: normals 2^-6..2^8 carry 3 fraction bits; below 2^-6 the
    # spacing is the subnormal step 2^-9
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    step = np.exp2(e - 3)
    return np.sign(v) * np.rint(a / step) * step


def mx_quantize(v: np.ndarray) -> np.ndarray:
    """MXFP8 round trip along the last axis (blocks of 32): returns the decoded float64 values."""
    v = np.asarray(v, np.float64)
    K = v.shape[-1]
    assert K % 32 == 0
    blk = v.reshape(*v.shape[:-1], K // 32, 32)
    amax = np.abs(blk).max(axis=-1, keepdims=True)
    with np.errstate(divide="ignore"):
        se = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8, -127)
    se = np.clip(se, -127, 127)
    scale = np.exp2(se)
    return (e4m3_round(blk / scale) * scale).reshape(v.shape)


def bf16_round(v: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (nearest even) and return float64."""
    v = np.asarray(v, np.float64)
    m, e = np.frexp(v)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def reference_dense(x: np.ndarray, ids: np.ndarray, w: np.ndarray, wg, wu, wd) -> np.ndarray:
    """float64 layer with dense (unquantized) weights. x: float64 [B,H] (bf16 values);
    wg/wu: [E,I,H], wd: [E,H,I] float arrays (only the routed experts are touched)."""
    B, k = ids.shape
    out = np.zeros((B, wd.shape[1]))
    for b in range(B):
        for j in range(k):
            e = int(ids[b, j])
            g = np.asarray(wg[e], np.float64) @ x[b]
            u = np.asarray(wu[e], np.float64) @ x[b]
            out[b] += float(w[b, j]) * (np.asarray(wd[e], np.float64) @ (_silu(g) * u))
    return out


# The classical path, stage by stage (the post, "Improved accuracy": activations
# converted BF16 -> MXFP8 -> back around each projection; "Buffer removal": a
# BF16 output buffer per routed expert, combined afterwards). Each stage is a
# function of its own so that a test can take one out and see the pins fail.

def _cls_quantize_x(x):
    """Stage 1: the token's activations to MXFP8 (blocks of 32 along H) and back."""
    return mx_quantize(x).astype(np.float32)


def _cls_gate_up(wg_e, wu_e, xq_b):
    """Stage 2: both projections with float32 accumulation, SwiGLU in float32."""
    g = np.asarray(wg_e, np.float32) @ xq_b
    u = np.asarray(wu_e, np.float32) @ xq_b
    return (g / (np.float32(1.0) + np.exp(-g)) * u).astype(np.float32)


def _cls_quantize_a(act):
    """Stage 3: the intermediate to MXFP8 (blocks of 32 along I) and back."""
    return mx_quantize(act[None, :])[0].astype(np.float32)


def _cls_down(wd_e, aq):
    """Stage 4: the down projection with float32 accumulation."""
    return np.asarray(wd_e, np.float32) @ aq


def _cls_expert_round(y):
    """Stage 5: the expert's output stored in its BF16 buffer."""
    return bf16_round(y).astype(np.float32)


def _cls_final_round(out):
    """Stage 7: the combined output stored as BF16."""
    return bf16_round(out)


def classical_emulation(x: np.ndarray, ids: np.ndarray, w: np.ndarray, wg_deq, wu_deq, wd_deq) -> np.ndarray:
    """The classical path's numerics on the MXFP8 weights (decoded values in wg_deq etc.).
    Stage 6, the combine, adds the routing-weighted BF16 expert outputs in float32."""
    B, k = ids.shape
    xq = _cls_quantize_x(x)
    out = np.zeros((B, wd_deq.shape[1]), np.float32)
    for b in range(B):
        for j in range(k):
            e = int(ids[b, j])
            aq = _cls_quantize_a(_cls_gate_up(wg_deq[e], wu_deq[e], xq[b]))
            out[b] += np.float32(w[b, j]) * _cls_expert_round(_cls_down(wd_deq[e], aq))
    return _cls_final_round(out)


def error_stats(got: np.ndarray, ref: np.ndarray) -> dict:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    rms_ref = float(np.sqrt(np.mean(ref ** 2)))
    cos = float(np.min(np.sum(got * ref, axis=1) /
                       (np.linalg.norm(got, axis=1) * np.linalg.norm(ref, axis=1))))
    return {"rms_err": float(np.sqrt(np.mean(d ** 2))), "max_abs": float(np.abs(d).max()),
            "rms_err_over_rms": float(np.sqrt(np.mean(d ** 2))) / rms_ref,
            "max_err_over_rms": float(np.abs(d).max()) / rms_ref, "min_cosine": cos}
