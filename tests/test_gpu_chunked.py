"""Chunked prefill (moe_layer_chunked): the layer over consecutive token chunks with a
workspace sized by the chunk.  Every token's routing and output depend on that token
alone, so the chunked layer must equal the single-call layer bit for bit; it is also
held to the oracle on every token."""
import numpy as np
import pytest
import torch

import bit_quantized_expert_top_amd as moe
import oracle
from moe_case import LayerRun, asymmetric_bias, check_y, device, shape_of
from synth import make_layer

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,H,I,chunk,zipf,seed", [
    (300, 512, 128, 128, None, 1300),      # three chunks, ragged last (44 tokens)
    (300, 512, 128, 1000, None, 1301),     # one chunk larger than T
    (2053, 2048, 512, 1024, 1.1, 4030),    # skewed routing, last chunk of 5 tokens
    (20, 768, 384, 7, None, 1302),         # chunks of 7, 7 and 6 tokens
])
def test_chunked_equals_single_call_and_oracle(T, H, I, chunk, zipf, seed):
    print(f"[chunked] T={T} H={H} I={I} chunk={chunk} zipf={zipf}", flush=True)
    dev = device()
    inp = make_layer(seed, T=T, H=H, I=I, zipf_s=zipf)
    run = LayerRun(inp).layer().sync()
    sh = shape_of(inp)
    ws = moe.workspace_chunked(sh, chunk, dev)
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device=dev)
    moe.moe_layer_chunked(sh, run.x, run.w, y, chunk, ws)
    torch.cuda.synchronize()
    assert torch.equal(y, run.y), "chunked layer differs from the single call"
    y_ref, _, _ = oracle.Layer(inp).tokens(range(T))
    ratio = check_y(y.cpu().numpy(), y_ref)
    print(f"  max err / rms = {ratio:.4g}", flush=True)


def test_chunked_workspace_reuse_across_calls():
    """Two chunked calls in a row on one workspace (the second with fewer tokens and a
    different chunk) each equal their single-call layers."""
    dev = device()
    for T, chunk, seed in ((500, 96, 1310), (130, 64, 1311)):
        inp = make_layer(seed, T=T, H=512, I=128)
        run = LayerRun(inp).layer().sync()
        sh = shape_of(inp)
        if T == 500:
            ws = moe.workspace_chunked(sh, chunk, dev)
        assert ws.numel() >= moe.moe_query_chunked(sh, chunk)
        y = torch.empty((T, 512), dtype=torch.float32, device=dev)
        moe.moe_layer_chunked(sh, run.x, run.w, y, chunk, ws)
        torch.cuda.synchronize()
        assert torch.equal(y, run.y), (T, chunk)


def test_chunked_asymmetric_bias():
    """Chunks over weights with b != -8 s in half of the groups: equal to the single call
    bit for bit, and to the oracle within the layer tolerance."""
    T, H, I, chunk, seed = 500, 1024, 256, 192, 1310
    print(f"[chunked-bias] T={T} H={H} I={I} chunk={chunk}", flush=True)
    dev = device()
    inp = make_layer(seed, T=T, H=H, I=I)
    asymmetric_bias(inp, seed)
    run = LayerRun(inp).layer().sync()
    sh = shape_of(inp)
    ws = moe.workspace_chunked(sh, chunk, dev)
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device=dev)
    moe.moe_layer_chunked(sh, run.x, run.w, y, chunk, ws)
    torch.cuda.synchronize()
    assert torch.equal(y, run.y), "chunked layer differs from the single call"
    y_ref, _, _ = oracle.Layer(inp).tokens(range(T))
    ratio = check_y(y.cpu().numpy(), y_ref)
    print(f"  max err / rms = {ratio:.4g}", flush=True)
