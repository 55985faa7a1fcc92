"""Helpers shared by the GPU tests: upload a synthetic layer and run the C ABI."""
from __future__ import annotations

import numpy as np
import torch

import bit_quantized_expert_top_amd as moe

TOL = 2e-2     # max |y - y_oracle| <= TOL * RMS(y_oracle)


def device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def shape_of(inp) -> moe.Shape:
    return moe.Shape(T=inp.T, H=inp.H, I=inp.I, E=inp.E, top_k=inp.top_k)


def upload(inp, dev=None) -> moe.DeviceLayer:
    dev = dev or device()
    proj = {n: (getattr(inp, n).q, getattr(inp, n).scale, getattr(inp, n).bias)
            for n in moe.DeviceLayer.NAMES}
    return moe.DeviceLayer(proj, inp.router_wt, inp.router_bias, device=dev)


def x_dev(inp, dev=None):
    return torch.from_numpy(inp.x).view(torch.int16).to(dev or device())


class LayerRun:
    """Buffers and results of one moe_layer call."""

    def __init__(self, inp, w: moe.DeviceLayer = None, dev=None, logits: bool = False):
        """logits=False runs the production routing (certified fast router); logits=True also
        computes every router logit in the fixed order and selects on those."""
        dev = dev or device()
        self.inp = inp
        self.shape = shape_of(inp)
        self.w = w or upload(inp, dev)
        self.x = x_dev(inp, dev)
        self.r = moe.Routing(self.shape, dev, with_logits=logits)
        self.ws = moe.workspace(self.shape, dev)
        rows = inp.T * inp.top_k + inp.T
        self.h = torch.zeros((rows, inp.I), dtype=torch.int16, device=dev)
        self.y = torch.zeros((inp.T, inp.H), dtype=torch.float32, device=dev)

    def route(self):
        moe.moe_route(self.shape, self.x, self.w, self.r, self.ws)
        return self

    def gemm(self):
        moe.moe_expert_gemm_q4(self.shape, self.x, self.w, self.r, self.h, self.ws)
        return self

    def down(self):
        moe.moe_down_combine(self.shape, self.h, self.w, self.r, self.y, self.ws)
        return self

    def layer(self):
        moe.moe_layer(self.shape, self.x, self.w, self.r, self.h, self.y, self.ws)
        return self

    def sync(self):
        torch.cuda.synchronize()
        return self

    def routing_np(self):
        r = self.r
        nb = int(r.num_blocks.cpu()[0])
        return dict(logits=None if r.logits is None else r.logits.cpu().numpy(),
                    ids=r.topk_ids.cpu().numpy(),
                    w=r.topk_w.cpu().numpy(), counts=r.counts.cpu().numpy(),
                    offsets=r.offsets.cpu().numpy(), row_token=r.row_token.cpu().numpy(),
                    tok_row=r.tok_row.cpu().numpy(), row_w=r.row_w.cpu().numpy(),
                    blocks=r.blocks.cpu().numpy()[:nb], num_blocks=nb)


def f16_np(t: torch.Tensor) -> np.ndarray:
    """int16 device tensor of fp16 bits -> float32 numpy."""
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.float16).astype(np.float32)




def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, tol: float = TOL):
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    err = float(np.max(np.abs(y_gpu.astype(np.float64) - y_ref)))
    assert np.all(np.isfinite(y_gpu)), "non-finite output"
    assert err <= tol * rms, f"max err {err:.4g} > {tol} * rms {rms:.4g} (ratio {err / rms:.4g})"
    return err / rms


_ORACLE_CACHE = {}


def oracle_tokens(inp, tokens, key=None):
    """oracle.Layer(inp).tokens(tokens), memoised under `key` (e.g. the seed and shape of a
    workload that several tests compare against)."""
    import oracle
    tokens = list(tokens)
    if key is not None:
        k = (key, tuple(tokens))
        if k not in _ORACLE_CACHE:
            _ORACLE_CACHE[k] = oracle.Layer(inp).tokens(tokens)
        return _ORACLE_CACHE[k]
    return oracle.Layer(inp).tokens(tokens)


def check_topk_weights(w_gpu: np.ndarray, w_ref: np.ndarray, ulps: float = 1.0):
    """Routing weights against the oracle's float64 values: within `ulps` units in the last
    place of the float32 value (the kernels evaluate the renormalised softmax in float64 from
    the fixed-order logits and round once), and every token's weights sum to 1 within 1e-6."""
    w_gpu = np.asarray(w_gpu, np.float32)
    ref32 = np.abs(w_ref).astype(np.float32)
    ulp = np.maximum(np.spacing(ref32), np.spacing(np.nextafter(ref32, np.float32(0))))
    err = np.abs(w_gpu.astype(np.float64) - w_ref)
    worst = float(np.max(err / ulp)) if err.size else 0.0
    assert worst <= ulps, f"routing weight off by {worst:.3g} ulp (limit {ulps})"
    assert np.all(np.abs(w_gpu.astype(np.float64).sum(axis=-1) - 1.0) <= 1e-6)
    return worst


def asymmetric_bias(inp, seed):
    """Biases b = bf16(-8 s + d) with d ~ U(-2s, 2s) in a random half of the groups
    (the rest keep b = -8 s), so the GEMMs' rank-G bias term is exercised."""
    from synth.inputs import bf16_bits_to_f32, f32_to_bf16_bits
    rng = np.random.default_rng(seed)
    for p in (inp.gate, inp.up, inp.down, inp.sh_gate, inp.sh_up, inp.sh_down):
        s = bf16_bits_to_f32(p.scale)
        d = rng.uniform(-2.0, 2.0, size=s.shape).astype(np.float32) * s
        d[rng.random(size=s.shape) < 0.5] = 0.0
        p.bias[...] = f32_to_bf16_bits(-8.0 * s + d)
