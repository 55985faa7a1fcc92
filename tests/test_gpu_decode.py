"""Batch-1 decode path against the oracle."""
import numpy as np
import pytest
import torch

import bit_quantized_expert_top_amd as moe
import oracle
from synth import make_layer
from moe_case import LayerRun, asymmetric_bias, check_topk_weights, check_y, device, shape_of, upload, x_dev
from synth.inputs import bf16_bits_to_f32

pytestmark = pytest.mark.gpu


def run_decode(inp, w=None):
    """moe_decode of all inp.T tokens; at T=1 the arrays are [top_k] and [H]."""
    dev = device()
    w = w or upload(inp, dev)
    sh = shape_of(inp)
    T = inp.T
    ids = torch.empty((T, inp.top_k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, inp.top_k), dtype=torch.float32, device=dev)
    y = torch.empty((T, inp.H), dtype=torch.float32, device=dev)
    ws = moe.workspace(sh, dev)
    moe.moe_decode(sh, x_dev(inp, dev), w, ids, tw, y, ws)
    torch.cuda.synchronize()
    out = ids.cpu().numpy(), tw.cpu().numpy(), y.cpu().numpy()
    return tuple(a[0] for a in out) if T == 1 else out


@pytest.mark.parametrize("seed", [2000, 2001, 2002, 2003])
def test_decode_matches_oracle(seed):
    print(f"[decode] seed={seed}", flush=True)
    inp = make_layer(seed, T=1, H=2048, I=512)
    ids, tw, y = run_decode(inp)
    y_ref, ids_ref, w_ref = oracle.Layer(inp).tokens([0])
    np.testing.assert_array_equal(ids, ids_ref[0])
    check_topk_weights(tw, w_ref[0])
    ratio = check_y(y[None, :], y_ref)
    print(f"  max err / rms = {ratio:.4g}", flush=True)


def test_decode_tiny_and_zipf():
    for kw, seed in ((dict(T=1, H=512, I=128), 1030), (dict(T=1, H=2048, I=512, zipf_s=1.1), 4010),
                     (dict(T=1, H=768, I=384), 1031), (dict(T=1, H=256, I=1024), 1032)):
        print(f"[decode] {kw} seed={seed}", flush=True)
        inp = make_layer(seed, **kw)
        ids, tw, y = run_decode(inp)
        y_ref, ids_ref, _ = oracle.Layer(inp).tokens([0])
        np.testing.assert_array_equal(ids, ids_ref[0])
        check_y(y[None, :], y_ref)


def test_decode_equals_prefill_path_at_t1():
    inp = make_layer(2005, T=1, H=2048, I=512)
    w = upload(inp)
    ids, tw, y = run_decode(inp, w)
    run = LayerRun(inp, w=w).layer().sync()
    np.testing.assert_array_equal(run.r.topk_ids.cpu().numpy()[0], ids)
    y2 = run.y.cpu().numpy()[0]
    assert np.max(np.abs(y2 - y)) <= 1e-2 * np.sqrt(np.mean(y ** 2))


def test_decode_stack_teacher_forced_and_graph():
    """Batch-1 decode through stacked layers (residual add + RMSNorm between them, the
    decode stack's structure on 4 layers).  Each layer is checked against the oracle on
    the GPU's own bf16 input (teacher forcing); the whole chain captured in one HIP graph
    replays bit for bit like the eager chain, with eager work between the replays."""
    H, I, L = 2048, 512, 4
    print(f"[decode-stack] H={H} I={I} layers={L}", flush=True)
    dev = device()
    layers = [make_layer(2100 + l, T=1, H=H, I=I, with_x=(l == 0)) for l in range(L)]
    x0 = layers[0].x.reshape(H).copy()
    ws_ = [upload(inp, dev) for inp in layers]
    sh = shape_of(layers[0])
    ws = moe.workspace(sh, dev)
    ids = torch.empty(8, dtype=torch.int32, device=dev)
    tw = torch.empty(8, dtype=torch.float32, device=dev)
    y = torch.empty(H, dtype=torch.float32, device=dev)
    r = torch.empty(H, dtype=torch.float32, device=dev)
    u = torch.empty(H, dtype=torch.int16, device=dev)
    x0_dev = torch.from_numpy(x0).view(torch.int16).to(dev)
    trace = []

    def chain(record):
        r.copy_(x0_dev.view(torch.bfloat16).float())
        u.copy_(x0_dev)
        for l in range(L):
            if record:
                trace.append(u.clone())
            moe.moe_decode(sh, u, ws_[l], ids, tw, y, ws)
            if record:
                trace.append((ids.clone(), y.clone()))
            moe.moe_rmsnorm_residual(1, H, 1e-6, r, y, u)

    chain(record=True)
    torch.cuda.synchronize()
    for l in range(L):
        inp = layers[l]
        inp.x = trace[2 * l].cpu().numpy().view(np.uint16).reshape(1, H).copy()
        ids_g, y_g = (t.cpu().numpy() for t in trace[2 * l + 1])
        y_ref, ids_ref, _ = oracle.Layer(inp).tokens([0])
        np.testing.assert_array_equal(ids_g, ids_ref[0])
        ratio = check_y(y_g[None, :], y_ref)
        print(f"  layer {l}: max err / rms = {ratio:.4g}", flush=True)
    r_eager, u_eager = r.clone(), u.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain(record=False)
    for rep in range(3):
        r.zero_()
        u.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(r, r_eager) and torch.equal(u, u_eager), rep


@pytest.mark.parametrize("T,seed,zipf", [(2, 2200, None), (3, 2201, None), (5, 2202, None),
                                         (8, 2203, None), (8, 4020, 1.1)])
def test_small_batch_decode_matches_oracle(T, seed, zipf):
    """Decode of T = 2..8 tokens in one call: every token's picks bit-exact, its weights and
    output within the layer tolerance.  With the Zipf router bias the tokens share experts."""
    print(f"[decode-batch] T={T} seed={seed} zipf={zipf}", flush=True)
    inp = make_layer(seed, T=T, H=2048, I=512, zipf_s=zipf)
    ids, tw, y = run_decode(inp)
    y_ref, ids_ref, w_ref = oracle.Layer(inp).tokens(range(T))
    np.testing.assert_array_equal(ids, ids_ref)
    check_topk_weights(tw, w_ref)
    ratio = check_y(y, y_ref)
    print(f"  max err / rms = {ratio:.4g}, distinct experts = {len(set(ids.ravel().tolist()))}",
          flush=True)


@pytest.mark.parametrize("T,seed", [(1, 2300), (4, 2301)])
def test_decode_asymmetric_bias(T, seed):
    """Decode with biases b != -8 s in half of the groups (the affine format's general
    case): picks bit-exact, output within the layer tolerance."""
    print(f"[decode-bias] T={T} seed={seed}", flush=True)
    inp = make_layer(seed, T=T, H=2048, I=512)
    asymmetric_bias(inp, seed)
    ids, tw, y = run_decode(inp)
    y_ref, ids_ref, w_ref = oracle.Layer(inp).tokens(range(T))
    if T == 1:
        ids, tw, y = ids[None], tw[None], y[None]
    np.testing.assert_array_equal(ids, ids_ref)
    check_topk_weights(tw, w_ref)
    ratio = check_y(y, y_ref)
    print(f"  max err / rms = {ratio:.4g}", flush=True)


def test_small_batch_equals_single_tokens():
    """Each token of a batched decode gets exactly what a batch-1 call on it alone returns."""
    inp = make_layer(2210, T=8, H=768, I=384)
    w = upload(inp)
    ids, tw, y = run_decode(inp, w)
    for t in range(inp.T):
        one = make_layer(2210, T=1, H=768, I=384, with_x=False)
        one.x = inp.x[t:t + 1].copy()
        i1, w1, y1 = run_decode(one, w)
        np.testing.assert_array_equal(i1, ids[t])
        np.testing.assert_array_equal(w1, tw[t])
        np.testing.assert_array_equal(y1, y[t])


@pytest.mark.parametrize("T,H,I", [(1, 2048, 512), (3, 2048, 512), (2, 768, 384)])
def test_decode_stack_fused_residual(T, H, I):
    """Layers after the first through moe_decode_residual, which folds the residual add and
    RMSNorm into the router pass: r must be the exact fp32 sum, u within one bf16 ulp of the
    oracle's RMSNorm of it, and each layer is checked against the oracle on the u it wrote
    (teacher forcing).  The y of the previous layer is overwritten in place.  The whole chain
    captured in a HIP graph replays bit for bit."""
    L = 4
    print(f"[decode-stack-fused] T={T} H={H} I={I} layers={L}", flush=True)
    dev = device()
    layers = [make_layer(2300 + 10 * T + l, T=T, H=H, I=I, with_x=(l == 0)) for l in range(L)]
    ws_ = [upload(inp, dev) for inp in layers]
    sh = shape_of(layers[0])
    ws = moe.workspace(sh, dev)
    x0 = torch.from_numpy(layers[0].x.copy()).view(torch.int16).to(dev)
    ids = torch.empty((T, 8), dtype=torch.int32, device=dev)
    tw = torch.empty((T, 8), dtype=torch.float32, device=dev)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    r = torch.empty((T, H), dtype=torch.float32, device=dev)
    u = torch.empty((T, H), dtype=torch.int16, device=dev)

    def chain(check):
        r.copy_(x0.view(torch.bfloat16).float())
        moe.moe_decode(sh, x0, ws_[0], ids, tw, y, ws)
        for l in range(1, L):
            if check:
                torch.cuda.synchronize()
                r_prev, y_prev = r.cpu().numpy().copy(), y.cpu().numpy().copy()
            moe.moe_decode_residual(sh, r, y, 1e-6, u, ws_[l], ids, tw, y, ws)
            if check:
                torch.cuda.synchronize()
                np.testing.assert_array_equal(r.cpu().numpy(), r_prev + y_prev)
                _, u_ref = oracle.rmsnorm_residual(r_prev.astype(np.float64),
                                                   y_prev.astype(np.float64), 1e-6)
                ug = bf16_bits_to_f32(u.cpu().numpy().view(np.uint16)).astype(np.float64)
                ur = bf16_bits_to_f32(u_ref).astype(np.float64)
                assert np.all(np.abs(ug - ur) <= 2.0 ** -7 * np.abs(ur) + 1e-30), l
                inp = layers[l]
                inp.x = u.cpu().numpy().view(np.uint16).copy()
                y_ref, ids_ref, _ = oracle.Layer(inp).tokens(range(T))
                np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
                ratio = check_y(y.cpu().numpy(), y_ref)
                print(f"  layer {l}: max err / rms = {ratio:.4g}", flush=True)

    chain(check=True)
    torch.cuda.synchronize()
    r_eager, y_eager = r.clone(), y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain(check=False)
    for rep in range(3):
        r.zero_()
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(r, r_eager) and torch.equal(y, y_eager), rep
