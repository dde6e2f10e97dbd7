"""Seeded synthetic inputs for the MoE decode expert layer.

This module only *makes inputs*: activations, router outputs and MXFP8-encoded
expert weights. It holds none of the layer's arithmetic (no decode, no dot
product, no SwiGLU, no routing-weight fold), so both the CPU oracle and the HIP
path can consume what it produces without sharing any of the method's code.

Recipe (the workload the warp-decode post measures is a Qwen-3-style MoE
decode layer, 8 of 128 experts, hidden 2048, batch up to 32 -- "Warp decode",
sections "Traditional MoE path", "Buffer removal", "Hardware efficiency"):

* x ~ N(0, 1) drawn in float64, rounded to bfloat16 (round-to-nearest-even).
* router logits ~ N(0, 1) [B, E] in float64; the skewed-routing workload adds a
  per-expert bias -s * ln(r_e) with r a seeded random permutation of 1..E
  (a log-Zipf(s) prior, so the hot experts sit at scattered indices).
  p = softmax(logits); ids = the k largest p (descending, ties to the lower
  index); w = p[ids] / sum(p[ids]) computed in float64, stored as float32.
* weights ~ N(0, 0.02) in float32, encoded to MXFP8 along the reduction axis:
  blocks of 32 contiguous elements share one UE8M0 scale byte, elements are
  OCP FP8 E4M3 codes (the block format named by the GC-MoE summary, section
  "How to use": FP8 E4M3 with a UE8M0 scale per 32 K values).
  Encoder rule (OCP Microscaling v1.0): shared exponent = floor(log2 amax) - 8
  (8 = the largest E4M3 exponent), clamped to [-127, 127]; an all-zero block
  gets exponent -127; elements = v * 2^-exponent clamped to +-448 and rounded
  to nearest-even E4M3. Scale code = exponent + 127.
* MXFP4 weights (wformat="mxfp4"; the FP4 E2M1 routed weights with K32 UE8M0
  scales of the same GC-MoE section): shared exponent = floor(log2 amax) - 2
  (2 = the largest E2M1 exponent, 6 = 1.5 * 2^2), elements clamped to +-6 and
  rounded to the nearest E2M1 value, ties to the even code; two codes per
  byte, element 2t in the low nibble of byte t and element 2t+1 in the high
  nibble.

Weights are drawn with torch on the requested device (so multi-GB inputs are
made in HBM in well under a second); x and routing are drawn with numpy on the
host, so they are identical on every machine. The weight bytes a GPU run uses
differ from a CPU run's for the same seed; every consumer reads the bytes it is
given, never a regenerated copy.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

BLOCK = 32            # elements per MX block (one UE8M0 scale each)
E4M3_MAX = 448.0      # largest finite OCP E4M3 magnitude
E4M3_EMAX = 8         # exponent of E4M3_MAX (448 = 1.75 * 2^8)
E2M1_MAX = 6.0        # largest OCP E2M1 magnitude
E2M1_EMAX = 2         # exponent of E2M1_MAX (6 = 1.5 * 2^2)
WFORMATS = ("mxfp8", "mxfp4")


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """One MoE decode layer: B tokens, E experts, top-k, hidden H, intermediate I."""
    name: str
    B: int
    E: int
    k: int
    H: int
    I: int
    zipf_s: float = 0.0      # > 0: skewed (log-Zipf) router prior

    def __post_init__(self):
        if self.H % BLOCK or self.I % BLOCK:
            raise ValueError("H and I must be multiples of 32 (one MX block)")
        if not 1 <= self.k <= self.E:
            raise ValueError("need 1 <= k <= E")

    @property
    def bytes_per_expert(self) -> int:
        """Codes + scales of one expert's gate, up and down matrices (MXFP8)."""
        return 3 * self.I * self.H * (BLOCK + 1) // BLOCK

    def weight_bytes_per_expert(self, wformat: str = "mxfp8") -> int:
        """Codes + scales of one expert's three matrices in the given format."""
        if wformat == "mxfp4":
            return 3 * self.I * self.H * (BLOCK // 2 + 1) // BLOCK
        return self.bytes_per_expert


# The five decode workloads, smallest first.
WORKLOADS = {
    "tiny_B1_E8_k2_H256_I128": LayerShape("tiny_B1_E8_k2_H256_I128", 1, 8, 2, 256, 128),
    "wide_B1_E128_k8_H2048_I768": LayerShape("wide_B1_E128_k8_H2048_I768", 1, 128, 8, 2048, 768),
    "batch_B8_E128_k8_H2048_I768": LayerShape("batch_B8_E128_k8_H2048_I768", 8, 128, 8, 2048, 768),
    "batch_B32_E128_k8_H4096_I1536": LayerShape("batch_B32_E128_k8_H4096_I1536", 32, 128, 8, 4096, 1536),
    "skewed_B64_E256_k8_H7168_I2048": LayerShape("skewed_B64_E256_k8_H7168_I2048", 64, 256, 8, 7168, 2048,
                                                 zipf_s=1.1),
}
WORKLOAD_ORDER = list(WORKLOADS)


def workload_seed(name: str) -> int:
    return 1000 + WORKLOAD_ORDER.index(name) + 1


# --------------------------------------------------------------------------------------
# host-side draws (numpy PCG64, identical everywhere)
# --------------------------------------------------------------------------------------

def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *key])))


def float64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float64 -> bfloat16 (nearest-even) and return the uint16 bit patterns.

    The float64 significand is rounded straight to bf16's 8 significant bits
    (one rounding, no double rounding through float32). Valid for the normal
    bf16 range, which N(0, 1) draws never leave.
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                     # v = m * 2^e, |m| in [0.5, 1)
    mr = np.rint(m * 256.0) / 256.0        # 8 significant bits, ties to even
    r = np.ldexp(mr, e).astype(np.float32)  # exact: fits in bf16 hence float32
    bits = r.view(np.uint32) >> 16
    return bits.astype(np.uint16)


def bf16_bits_to_float64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def make_activations(B: int, H: int, seed: int) -> np.ndarray:
    """x ~ N(0,1), as bfloat16 bit patterns [B, H] (uint16)."""
    return float64_to_bf16_bits(_rng(seed, 0).standard_normal((B, H)))


def make_router_logits(B: int, E: int, seed: int, zipf_s: float = 0.0,
                       contiguous_hot: bool = False) -> np.ndarray:
    """Router logits [B, E] in float64: N(0, 1), plus the log-Zipf prior when zipf_s > 0."""
    logits = _rng(seed, 1).standard_normal((B, E))
    if zipf_s > 0.0:
        rank = np.arange(1, E + 1) if contiguous_hot else _rng(seed, 2).permutation(E) + 1
        logits = logits - zipf_s * np.log(rank.astype(np.float64))[None, :]
    return logits


def make_routing(B: int, E: int, k: int, seed: int, zipf_s: float = 0.0,
                 contiguous_hot: bool = False):
    """Router output for B tokens: (ids int32 [B,k], w float32 [B,k], probs float64 [B,E])."""
    logits = make_router_logits(B, E, seed, zipf_s, contiguous_hot)
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(p, order, axis=1)
    w = sel / sel.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32), p


# --------------------------------------------------------------------------------------
# MXFP8 encoder (torch, any device)
# --------------------------------------------------------------------------------------

def encode_mxfp8(w: torch.Tensor):
    """Encode float32 [..., K] (K % 32 == 0) to (codes uint8 [..., K], scales uint8 [..., K/32])."""
    if w.dtype != torch.float32 or w.shape[-1] % BLOCK:
        raise ValueError("encode_mxfp8 wants float32 with a last dim that is a multiple of 32")
    K = w.shape[-1]
    blk = w.reshape(*w.shape[:-1], K // BLOCK, BLOCK)
    amax = blk.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)                       # amax = m * 2^ex, m in [0.5, 1)
    se = (ex.to(torch.int32) - 1) - E4M3_EMAX       # floor(log2 amax) - emax
    se = torch.where(amax > 0, se, torch.full_like(se, -127)).clamp_(-127, 127)
    mul = torch.exp2((-se).to(torch.float32))       # exact power of two
    scaled = (blk * mul.unsqueeze(-1)).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = scaled.to(torch.float8_e4m3fn).view(torch.uint8).reshape(w.shape)
    scales = (se + 127).to(torch.uint8)
    return codes.contiguous(), scales.contiguous()


_E2M1_MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)   # between the 8 magnitudes


def encode_mxfp4(w: torch.Tensor):
    """Encode float32 [..., K] (K % 32 == 0) to (packed codes uint8 [..., K/2], scales uint8 [..., K/32])."""
    if w.dtype != torch.float32 or w.shape[-1] % BLOCK:
        raise ValueError("encode_mxfp4 wants float32 with a last dim that is a multiple of 32")
    K = w.shape[-1]
    blk = w.reshape(*w.shape[:-1], K // BLOCK, BLOCK)
    amax = blk.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)
    se = (ex.to(torch.int32) - 1) - E2M1_EMAX       # floor(log2 amax) - emax
    se = torch.where(amax > 0, se, torch.full_like(se, -127)).clamp_(-127, 127)
    mul = torch.exp2((-se).to(torch.float32))
    scaled = blk * mul.unsqueeze(-1)
    mag = scaled.abs().clamp_(max=E2M1_MAX)
    mids = torch.tensor(_E2M1_MIDPOINTS, dtype=torch.float32, device=w.device)
    idx = torch.searchsorted(mids, mag.contiguous())   # number of midpoints below the value
    # a value exactly on a midpoint goes to the even code (mantissa bit 0)
    on_mid = (idx < len(_E2M1_MIDPOINTS)) & (mag == mids[idx.clamp(max=len(_E2M1_MIDPOINTS) - 1)])
    idx = torch.where(on_mid & (idx % 2 == 1), idx + 1, idx)
    codes = (idx | torch.where(scaled < 0, 8, 0)).to(torch.uint8).reshape(*w.shape[:-1], K)
    packed = codes[..., 0::2] | (codes[..., 1::2] << 4)
    scales = (se + 127).to(torch.uint8)
    return packed.contiguous(), scales.contiguous()


@dataclasses.dataclass
class LayerInputs:
    shape: LayerShape
    seed: int
    x: np.ndarray            # uint16 bf16 bits [B, H]  (host)
    ids: np.ndarray          # int32 [B, k]             (host)
    w: np.ndarray            # float32 [B, k]           (host)
    probs: np.ndarray        # float64 [B, E]           (host)
    wg_q: torch.Tensor       # uint8 [E, I, H]          (device)
    wg_s: torch.Tensor       # uint8 [E, I, H/32]
    wu_q: torch.Tensor       # uint8 [E, I, H]
    wu_s: torch.Tensor       # uint8 [E, I, H/32]
    wd_q: torch.Tensor       # uint8 [E, H, I]
    wd_s: torch.Tensor       # uint8 [E, H, I/32]
    dense: dict | None = None  # unquantized float32 draws, when asked for
    wformat: str = "mxfp8"     # "mxfp4": codes packed two per byte ([E, I, H/2], [E, H, I/2])

    @property
    def unique_experts(self) -> int:
        return int(np.unique(self.ids).size)

    @property
    def unique_weight_bytes(self) -> int:
        return self.unique_experts * self.shape.weight_bytes_per_expert(self.wformat)


def make_weights(E: int, N: int, K: int, seed: int, tensor_id: int, device,
                 keep_dense: bool = False, experts_per_draw: int = 8, wformat: str = "mxfp8"):
    """N(0, 0.02) weights [E, N, K] encoded to MXFP8 (or MXFP4), drawn on `device` in expert groups."""
    if wformat not in WFORMATS:
        raise ValueError(f"unknown weight format {wformat!r}")
    device = torch.device(device)
    encode = encode_mxfp4 if wformat == "mxfp4" else encode_mxfp8
    q = torch.empty((E, N, K // 2 if wformat == "mxfp4" else K), dtype=torch.uint8, device=device)
    s = torch.empty((E, N, K // BLOCK), dtype=torch.uint8, device=device)
    dense = torch.empty((E, N, K), dtype=torch.float32, device=device) if keep_dense else None
    gen = torch.Generator(device=device)
    for e0 in range(0, E, experts_per_draw):
        e1 = min(E, e0 + experts_per_draw)
        gen.manual_seed(int(seed) * 1_000_003 + tensor_id * 10_007 + e0)
        d = torch.randn((e1 - e0, N, K), generator=gen, dtype=torch.float32, device=device)
        d.mul_(0.02)
        q[e0:e1], s[e0:e1] = encode(d)
        if keep_dense:
            dense[e0:e1] = d
        del d
    return q, s, dense


def make_layer(shape: LayerShape | str, seed: int | None = None, device="cpu",
               keep_dense: bool = False, contiguous_hot: bool = False,
               wformat: str = "mxfp8") -> LayerInputs:
    """All inputs of one decode layer. Weights live on `device`, the rest on the host."""
    if isinstance(shape, str):
        shape = WORKLOADS[shape]
    if seed is None:
        seed = workload_seed(shape.name)
    B, E, k, H, I = shape.B, shape.E, shape.k, shape.H, shape.I
    x = make_activations(B, H, seed)
    ids, w, probs = make_routing(B, E, k, seed, shape.zipf_s, contiguous_hot)
    wg_q, wg_s, dg = make_weights(E, I, H, seed, 0, device, keep_dense, wformat=wformat)
    wu_q, wu_s, du = make_weights(E, I, H, seed, 1, device, keep_dense, wformat=wformat)
    wd_q, wd_s, dd = make_weights(E, H, I, seed, 2, device, keep_dense, wformat=wformat)
    dense = dict(gate=dg, up=du, down=dd) if keep_dense else None
    return LayerInputs(shape, seed, x, ids, w, probs, wg_q, wg_s, wu_q, wu_s, wd_q, wd_s, dense, wformat)


def random_small_shape(rng: np.random.Generator, max_E=8, max_dim=128) -> LayerShape:
    """A random tiny shape for brute-force and fuzz cases (dims are multiples of 32)."""
    E = int(rng.integers(1, max_E + 1))
    k = int(rng.integers(1, E + 1))
    B = int(rng.integers(1, 5))
    H = 32 * int(rng.integers(1, max_dim // 32 + 1))
    I = 32 * int(rng.integers(1, max_dim // 32 + 1))
    return LayerShape(f"rand_B{B}_E{E}_k{k}_H{H}_I{I}", B, E, k, H, I)
