"""moe_decode_static (no workspace, the library's per-GPU scratch array) against moe_decode:
two calls in a row on the same weights, the second with fewer tokens and a smaller layer,
each bit-identical to moe_decode with a caller workspace."""
import numpy as np
import pytest
import torch

import bit_quantized_expert_top_amd as moe
from moe_case import device, shape_of, upload, x_dev
from synth import make_layer

pytestmark = pytest.mark.gpu


def _decode_both(inp):
    dev = device()
    w = upload(inp, dev)
    sh = shape_of(inp)
    T, k, H = inp.T, inp.top_k, inp.H
    x = x_dev(inp, dev)
    out = []
    for static in (False, True):
        ids = torch.full((T, k), -1, dtype=torch.int32, device=dev)
        tw = torch.full((T, k), float("nan"), dtype=torch.float32, device=dev)
        y = torch.full((T, H), float("nan"), dtype=torch.float32, device=dev)
        if static:
            moe.moe_decode_static(sh, x, w, ids, tw, y)
        else:
            moe.moe_decode(sh, x, w, ids, tw, y, moe.workspace(sh, dev))
        torch.cuda.synchronize()
        out.append((ids.cpu().numpy(), tw.cpu().numpy(), y.cpu().numpy()))
    return out


def test_decode_static_equals_decode_twice_shrinking():
    cases = [(dict(T=8, H=2048, I=2048), 2600),      # the largest call the scratch array holds
             (dict(T=3, H=768, I=384), 2601)]        # then a smaller one on the same array
    for kw, seed in cases:
        print(f"[decode-static] {kw} seed={seed}", flush=True)
        inp = make_layer(seed, **kw)
        (ids0, tw0, y0), (ids1, tw1, y1) = _decode_both(inp)
        np.testing.assert_array_equal(ids1, ids0)
        np.testing.assert_array_equal(tw1.view(np.uint32), tw0.view(np.uint32))
        np.testing.assert_array_equal(y1.view(np.uint32), y0.view(np.uint32))
        assert np.all(np.isfinite(y1))


def test_decode_static_refuses_more_than_eight_tokens():
    inp = make_layer(2602, T=1, H=512, I=128)
    dev = device()
    w = upload(inp, dev)
    sh = moe.Shape(T=9, H=512, I=128)
    x = torch.zeros((9, 512), dtype=torch.int16, device=dev)
    ids = torch.empty((9, 8), dtype=torch.int32, device=dev)
    tw = torch.empty((9, 8), dtype=torch.float32, device=dev)
    y = torch.empty((9, 512), dtype=torch.float32, device=dev)
    with pytest.raises(moe.MoeError):
        moe.moe_decode_static(sh, x, w, ids, tw, y)
