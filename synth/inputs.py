"""Seeded generators for synthetic MoE-layer inputs (no layer arithmetic here)."""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

GROUP = 64          # quantisation group along the input dimension
PACK = 8            # 4-bit codes per uint32 word


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32)
    # finite inputs only: u + 0x8000 cannot wrap below 0xFF800000
    u = (u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen bf16 bits (uint16) to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Projection:
    """One 4-bit affine projection W[N][K]: packed codes plus per-group scale/bias."""
    q: np.ndarray       # uint32 [..., N, K/8]
    scale: np.ndarray   # uint16 (bf16 bits) [..., N, K/64]
    bias: np.ndarray    # uint16 (bf16 bits) [..., N, K/64]


@dataclass
class LayerInputs:
    T: int
    H: int
    I: int
    E: int
    top_k: int
    x: np.ndarray                       # uint16 [T, H]
    router_wt: np.ndarray               # uint16 [E, H]
    router_bias: Optional[np.ndarray]   # float32 [E] or None
    gate: Projection                    # [E, I, H/8]
    up: Projection                      # [E, I, H/8]
    down: Projection                    # [E, H, I/8]
    sh_gate: Projection                 # [I, H/8]
    sh_up: Projection                   # [I, H/8]
    sh_down: Projection                 # [H, I/8]
    meta: Dict[str, object] = field(default_factory=dict)


def make_projection(rng: np.random.Generator, lead: tuple, N: int, K: int) -> Projection:
    """Draw codes (random words), scales U(0.002, 0.02) in bf16 and bias = -8*scale."""
    if K % GROUP:
        raise ValueError("K must be a multiple of 64")
    q = rng.integers(0, 2**32, size=lead + (N, K // PACK), dtype=np.uint32)
    s = rng.uniform(0.002, 0.02, size=lead + (N, K // GROUP)).astype(np.float32)
    s16 = f32_to_bf16_bits(s)
    # -8 * s only changes sign and exponent, so it is exact in bf16
    b16 = f32_to_bf16_bits(-8.0 * bf16_bits_to_f32(s16))
    return Projection(q=q, scale=s16, bias=b16)


def zipf_bias(E: int, s: float) -> np.ndarray:
    """Per-expert additive logit bias -s*ln(rank), rank = expert index + 1 (float32)."""
    return (-s * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)


def ep_share_bias(E: int, n_gpus: int) -> np.ndarray:
    """Router bias that keeps every pick among experts [0, E / n_gpus): one GPU's share of the
    experts under expert parallelism over n_gpus GPUs (0 there, -32 elsewhere; the logits are
    about N(0, 1), so no other expert reaches the top-k)."""
    if E % n_gpus:
        raise ValueError("E must be a multiple of n_gpus")
    b = np.full(E, -32.0, np.float32)
    b[: E // n_gpus] = 0.0
    return b


def make_layer(seed: int, T: int, H: int, I: int, E: int = 256, top_k: int = 8,
               zipf_s: Optional[float] = None, with_x: bool = True,
               ep_share: Optional[int] = None) -> LayerInputs:
    """Draw one layer in a fixed order: x, router weight, gate, up, down, shared gate/up/down."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if with_x:
        x = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    else:
        x = np.zeros((T, H), np.uint16)
    wr = f32_to_bf16_bits((rng.standard_normal((E, H)) / np.sqrt(H)).astype(np.float32))
    gate = make_projection(rng, (E,), I, H)
    up = make_projection(rng, (E,), I, H)
    down = make_projection(rng, (E,), H, I)
    sh_gate = make_projection(rng, (), I, H)
    sh_up = make_projection(rng, (), I, H)
    sh_down = make_projection(rng, (), H, I)
    bias = zipf_bias(E, zipf_s) if zipf_s is not None else None
    if ep_share is not None:
        bias = ep_share_bias(E, ep_share)
    return LayerInputs(T=T, H=H, I=I, E=E, top_k=top_k, x=x, router_wt=wr, router_bias=bias,
                       gate=gate, up=up, down=down, sh_gate=sh_gate, sh_up=sh_up,
                       sh_down=sh_down, meta={"seed": seed, "zipf_s": zipf_s, "ep_share": ep_share})


# The workloads: shapes and routing recipes of the five synthetic layers.
WORKLOADS = {
    "tiny":        dict(T=32,   H=512,  I=128, seed_base=1000, zipf_s=None),
    "decode":      dict(T=1,    H=2048, I=512, seed_base=2000, zipf_s=None),
    "prefill512":  dict(T=512,  H=2048, I=512, seed_base=3000, zipf_s=None),
    "prefill2048_zipf": dict(T=2048, H=2048, I=512, seed_base=4000, zipf_s=1.1),
    "stack40":     dict(T=4096, H=2048, I=512, seed_base=5000, zipf_s=None, layers=40),
}
