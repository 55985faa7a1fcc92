"""The same synthetic layer, drawn directly in GPU memory with torch's seeded generator.

Used where many independently seeded layers are needed quickly (the benchmark
rotates weight sets so that consecutive steps never find their weights in the
last-level cache).  Same layouts and distributions as ``synth.inputs``; the
values differ from the numpy draws of the same seed.  No layer arithmetic here.
"""
from __future__ import annotations

import numpy as np
import torch

from .inputs import GROUP, PACK, LayerInputs, Projection, ep_share_bias, zipf_bias


def _bf16_bits(t: torch.Tensor) -> torch.Tensor:
    return t.to(torch.bfloat16).view(torch.int16)      # round to nearest even


def _proj(g: torch.Generator, lead, N, K, dev, affine: bool = False):
    q = torch.randint(-2 ** 31, 2 ** 31, lead + (N, K // PACK), generator=g, device=dev,
                      dtype=torch.int64).to(torch.int32)
    s = torch.empty(lead + (N, K // GROUP), device=dev, dtype=torch.float32).uniform_(
        0.002, 0.02, generator=g).to(torch.bfloat16)
    b = -8.0 * s.float()                                # exact: -8 only moves the exponent
    if affine:
        # the general affine case: every group's bias off -8 s by d ~ U(-2 s, 2 s)
        d = torch.empty_like(b).uniform_(-2.0, 2.0, generator=g) * s.float()
        b = b + d
    return q, s.view(torch.int16), b.to(torch.bfloat16).view(torch.int16)


def make_layer_device(seed: int, T: int, H: int, I: int, E: int = 256, zipf_s=None,
                      device="cuda", with_x: bool = True, affine: bool = False,
                      ep_share=None) -> dict:
    """Dict of device tensors: x, router_wt, router_bias and the six projections
    (affine=True: biases b != -8 s in every group; ep_share=n: the router bias keeps the
    picks among one GPU's E/n experts)."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    out = {}
    if with_x:
        out["x"] = _bf16_bits(torch.randn((T, H), generator=g, device=dev))
    out["router_wt"] = _bf16_bits(torch.randn((E, H), generator=g, device=dev) / float(np.sqrt(H)))
    out["router_bias"] = (None if zipf_s is None else
                          torch.from_numpy(zipf_bias(E, zipf_s)).to(dev))
    if ep_share is not None:
        out["router_bias"] = torch.from_numpy(ep_share_bias(E, ep_share)).to(dev)
    out["gate"] = _proj(g, (E,), I, H, dev, affine)
    out["up"] = _proj(g, (E,), I, H, dev, affine)
    out["down"] = _proj(g, (E,), H, I, dev, affine)
    out["sh_gate"] = _proj(g, (), I, H, dev, affine)
    out["sh_up"] = _proj(g, (), I, H, dev, affine)
    out["sh_down"] = _proj(g, (), H, I, dev, affine)
    return out


def to_host_inputs(d: dict, T: int, H: int, I: int, E: int = 256, top_k: int = 8,
                   x=None) -> LayerInputs:
    """Copy a device layer back to numpy (for the CPU oracle)."""
    def p(name):
        q, s, b = d[name]
        return Projection(q=q.cpu().numpy().view(np.uint32), scale=s.cpu().numpy().view(np.uint16),
                          bias=b.cpu().numpy().view(np.uint16))
    xx = d["x"] if x is None else x
    rb = d["router_bias"]
    return LayerInputs(T=T, H=H, I=I, E=E, top_k=top_k,
                       x=xx.cpu().numpy().view(np.uint16),
                       router_wt=d["router_wt"].cpu().numpy().view(np.uint16),
                       router_bias=None if rb is None else rb.cpu().numpy(),
                       gate=p("gate"), up=p("up"), down=p("down"), sh_gate=p("sh_gate"),
                       sh_up=p("sh_up"), sh_down=p("sh_down"))
