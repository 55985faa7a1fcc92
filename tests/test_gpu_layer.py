"""The whole layer (route -> gate/up GEMM -> down + combine) against the oracle."""
import numpy as np
import pytest
import torch

import bit_quantized_expert_top_amd as moe
import oracle
from synth import make_layer
from moe_case import (LayerRun, asymmetric_bias, check_topk_weights, check_y, device, f16_np,
                      oracle_tokens, upload)

pytestmark = pytest.mark.gpu


def sample_tokens(T, n, seed):
    if T <= n:
        return list(range(T))
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(T, size=n - 3, replace=False).tolist()) | {0, T - 1, T // 2}
    return sorted(pick)


CASES = [
    ("tiny", dict(T=32, H=512, I=128), 1000),
    ("tiny_zipf", dict(T=32, H=512, I=128, zipf_s=1.1), 1001),
    ("ragged129", dict(T=129, H=512, I=128, zipf_s=1.1), 1003),
    ("T1_prefill_path", dict(T=1, H=2048, I=512), 2001),
    ("prefill512", dict(T=512, H=2048, I=512), 3000),
    ("prefill2048_zipf", dict(T=2048, H=2048, I=512, zipf_s=1.1), 4000),
    # one layer of the 40-layer stack workload (T=4096, random router)
    ("stack_layer_T4096", dict(T=4096, H=2048, I=512), 5000),
    # narrow H (one router chunk per K quarter, one down tile), wide I, ragged T
    ("narrowH_wideI", dict(T=77, H=256, I=1024), 4200),
    # H not a power of two, I = 3 x 128
    ("H768_I384", dict(T=200, H=768, I=384, zipf_s=1.1), 4201),
    # one GPU's share under expert parallelism over 8 GPUs: every pick among experts 0-31
    # (512 rows per expert, no small blocks)
    ("ep8_share_T2048", dict(T=2048, H=2048, I=512, ep_share=8), 6000),
]


@pytest.mark.parametrize("name,kw,seed", CASES, ids=[c[0] for c in CASES])
def test_layer_matches_oracle(name, kw, seed):
    """Every output of the layer (all T x H values) against the oracle."""
    print(f"[layer] {name} seed={seed} {kw}", flush=True)
    inp = make_layer(seed, **kw)
    run = LayerRun(inp).layer().sync()
    y = run.y.cpu().numpy()
    y_ref, ids_ref, w_ref = oracle_tokens(inp, range(inp.T), key=(seed, name))
    got = run.routing_np()
    np.testing.assert_array_equal(got["ids"], ids_ref)
    if "ep_share" in kw:
        assert got["ids"].max() < inp.E // kw["ep_share"]
    check_topk_weights(got["w"], w_ref)
    ratio = check_y(y, y_ref)
    print(f"  max err / rms = {ratio:.4g}", flush=True)


def test_max_tokens_sampled():
    """The largest T one call accepts (65536 tokens, 131 MB of x): routing takes the multi-pass
    path (more than 32 superblocks of token blocks).  Given the GPU's picks, the expert counts,
    offsets, scatter and block map of all 524288 picks equal the oracle's bit for bit; on
    sampled tokens the picks, weights and outputs match the oracle; every output is finite."""
    T = 65536
    print(f"[layer] max tokens T={T}", flush=True)
    inp = make_layer(7000, T=T, H=2048, I=512, zipf_s=1.1)
    run = LayerRun(inp).layer().sync()
    got = run.routing_np()
    ref = oracle.routing(got["ids"], inp.E, 128)
    for key in ("counts", "offsets", "row_token", "tok_row"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    assert got["num_blocks"] == ref["num_blocks"]
    np.testing.assert_array_equal(got["blocks"], ref["blocks"])
    y = run.y.cpu().numpy()
    assert np.isfinite(y).all()
    toks = sample_tokens(T, 16, 7000)
    y_ref, ids_ref, w_ref = oracle_tokens(inp, toks)
    np.testing.assert_array_equal(got["ids"][toks], ids_ref)
    check_topk_weights(got["w"][toks], w_ref)
    ratio = check_y(y[toks], y_ref)
    print(f"  max err / rms = {ratio:.4g}", flush=True)


def test_prefill_graph_replays_two_weight_sets():
    """The timed form of the prefill step: two layers with independently seeded weights share
    the routing buffers, the workspace and h, captured together in one HIP graph.  Each of three
    replays reproduces the eager outputs bit for bit (the GEMM work-queue counters re-arm
    between launches), and the outputs match the oracle on every token."""
    kw = dict(T=2048, H=2048, I=512, zipf_s=1.1)
    print(f"[graph] prefill2048_zipf, weight sets 4000 and 4100", flush=True)
    inp_a = make_layer(4000, **kw)
    inp_b = make_layer(4100, **kw)
    inp_b.x = inp_a.x
    dev = device()
    wa, wb = upload(inp_a, dev), upload(inp_b, dev)
    run = LayerRun(inp_a, w=wa)
    ya = torch.zeros_like(run.y)
    yb = torch.zeros_like(run.y)

    def step(w, y):
        moe.moe_layer(run.shape, run.x, w, run.r, run.h, y, run.ws)

    step(wa, ya)
    step(wb, yb)
    torch.cuda.synchronize()
    ya_e, yb_e = ya.clone(), yb.clone()
    routing_b = run.routing_np()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(wa, ya)
        step(wb, yb)
    for rep in range(3):
        ya.zero_()
        yb.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ya, ya_e) and torch.equal(yb, yb_e), f"replay {rep} differs from eager"
        got = run.routing_np()
        for key in ("ids", "w", "row_token", "tok_row", "blocks"):
            np.testing.assert_array_equal(got[key], routing_b[key], err_msg=key)
    del g
    for inp, y, name in ((inp_a, ya_e, "a"), (inp_b, yb_e, "b")):
        y_ref, _, _ = oracle_tokens(inp, range(inp.T),
                                    key=(4000, "prefill2048_zipf") if name == "a" else None)
        ratio = check_y(y.cpu().numpy(), y_ref)
        print(f"  set {name}: max err / rms = {ratio:.4g}", flush=True)


def test_largest_shape_prefill_and_decode():
    """The largest supported shape, H = I = 2048 (gate/up over 16 n-tiles, down with K = 2048),
    through the prefill layer (sampled tokens) and the T=1 decode path on the same weights."""
    T, H, I, seed = 96, 2048, 2048, 4202
    print(f"[layer-max] T={T} H={H} I={I}", flush=True)
    inp = make_layer(seed, T=T, H=H, I=I)
    dev = device()
    w = upload(inp, dev)
    run = LayerRun(inp, w=w).layer().sync()
    toks = list(range(T))
    L = oracle.Layer(inp)
    y_ref, ids_ref, w_ref = L.tokens(toks)
    got = run.routing_np()
    np.testing.assert_array_equal(got["ids"][toks], ids_ref)
    ratio = check_y(run.y.cpu().numpy()[toks], y_ref)
    print(f"  prefill max err / rms = {ratio:.4g}", flush=True)
    # token 0 alone through moe_decode
    sh1 = moe.Shape(T=1, H=H, I=I, E=inp.E, top_k=inp.top_k)
    ids = torch.empty((1, inp.top_k), dtype=torch.int32, device=dev)
    tw = torch.empty((1, inp.top_k), dtype=torch.float32, device=dev)
    y1 = torch.empty((1, H), dtype=torch.float32, device=dev)
    moe.moe_decode(sh1, run.x[:1].contiguous(), w, ids, tw, y1, moe.workspace(sh1, dev))
    torch.cuda.synchronize()
    i0 = toks.index(0)
    np.testing.assert_array_equal(ids.cpu().numpy()[0], ids_ref[i0])
    check_topk_weights(tw.cpu().numpy()[0], w_ref[i0])
    ratio = check_y(y1.cpu().numpy(), y_ref[i0:i0 + 1])
    print(f"  decode max err / rms = {ratio:.4g}", flush=True)


def test_hidden_rows_match_oracle():
    """h rows (SwiGLU activations) of routed and shared rows against the oracle's.

    h is stored in fp16, so each element may differ from the float64 value by
    half an fp16 ulp (2^-11 relative; the bound allows 2^-10); the fp32
    arithmetic before the rounding adds at most a small fraction of the row's
    RMS."""
    inp = make_layer(4000, T=2048, H=2048, I=512, zipf_s=1.1)
    run = LayerRun(inp).route().gemm().sync()
    got = run.routing_np()
    h = f16_np(run.h)
    L = oracle.Layer(inp)
    T, k = inp.T, inp.top_k
    rng = np.random.default_rng(5)
    checks = [(int(t), int(j)) for t, j in zip(rng.integers(0, T, 12), rng.integers(0, k, 12))]
    for t, j in checks:
        e = int(got["ids"][t, j])
        a = L.expert_act(e, t)
        r = int(got["tok_row"][t, j])
        bound = 2.0 ** -10 * np.abs(a) + 1e-4 * np.sqrt(np.mean(a ** 2))
        assert np.all(np.abs(h[r] - a) <= bound), (t, j, e, np.max(np.abs(h[r] - a) - bound))
    for t in (0, 1000, T - 1):
        a = L.expert_act(inp.E, t)
        bound = 2.0 ** -10 * np.abs(a) + 1e-4 * np.sqrt(np.mean(a ** 2))
        assert np.all(np.abs(h[T * k + t] - a) <= bound), t


def test_layer_zero_experts_and_single_live_expert():
    inp = make_layer(1020, T=64, H=512, I=128)
    for p in (inp.gate, inp.up, inp.down):
        p.q[...] = np.uint32(0x88888888)           # code 8 with bias -8*scale: zero weight
    live = 5
    rng = np.random.default_rng(3)
    for p in (inp.gate, inp.up, inp.down):
        p.q[live] = rng.integers(0, 2 ** 32, size=p.q[live].shape, dtype=np.uint32)
    run = LayerRun(inp).layer().sync()
    y_ref, _, _ = oracle.Layer(inp).tokens(range(inp.T))
    check_y(run.y.cpu().numpy(), y_ref)


def test_layer_all_tokens_one_expert_set():
    """Every token on the same 8 experts: 8 groups of T rows, blocks of exactly 128 and a ragged tail."""
    inp = make_layer(1021, T=300, H=512, I=128)
    inp.router_bias = np.zeros(inp.E, np.float32)
    inp.router_bias[[3, 50, 99, 120, 180, 201, 230, 255]] = 50.0
    run = LayerRun(inp).layer().sync()
    got = run.routing_np()
    assert got["num_blocks"] == 8 * 3
    toks = list(range(inp.T))
    y_ref, _, _ = oracle.Layer(inp).tokens(toks)
    check_y(run.y.cpu().numpy()[toks], y_ref)


def test_layer_repeat_bit_identical():
    """Two runs give identical bits: the combine adds each token's rows in a fixed order."""
    inp = make_layer(3001, T=512, H=2048, I=512)
    run = LayerRun(inp)
    run.layer().sync()
    y1 = run.y.clone()
    h1 = run.h.clone()
    run.layer().sync()
    assert torch.equal(run.h, h1)
    assert torch.equal(run.y, y1)


@pytest.mark.parametrize("name,kw,seed", [
    ("tiny", dict(T=32, H=512, I=128), 1100),
    ("medium_zipf", dict(T=256, H=2048, I=512, zipf_s=1.1), 1101),
    # 12 groups along H and 6 along I: group counts that are not multiples of 8
    ("H768_I384", dict(T=150, H=768, I=384, zipf_s=1.1), 1102),
])
def test_layer_asymmetric_bias(name, kw, seed):
    print(f"[layer-bias] {name} seed={seed} {kw}", flush=True)
    inp = make_layer(seed, **kw)
    asymmetric_bias(inp, seed)
    run = LayerRun(inp).route().gemm().down().sync()
    toks = list(range(inp.T))
    y_ref, ids_ref, _ = oracle.Layer(inp).tokens(toks)
    got = run.routing_np()
    np.testing.assert_array_equal(got["ids"][toks], ids_ref)
    ratio = check_y(run.y.cpu().numpy()[toks], y_ref)
    print(f"  max err / rms = {ratio:.4g}", flush=True)
    h = f16_np(run.h)
    L = oracle.Layer(inp)
    for t in toks[:6]:
        for j in (0, 7):
            e = int(got["ids"][t, j])
            a = L.expert_act(e, t)
            r = int(got["tok_row"][t, j])
            bound = 2.0 ** -10 * np.abs(a) + 1e-4 * np.sqrt(np.mean(a ** 2))
            assert np.all(np.abs(h[r] - a) <= bound), (t, j, e, np.max(np.abs(h[r] - a) - bound))


@pytest.mark.parametrize("lo,hi", [(-13, -9), (8, 12), (-40, -36)], ids=["small", "large", "tiny"])
def test_hidden_rows_scale_extremes(lo, hi):
    """Scales far from the usual ones (each weight row is rebuilt at its own power of two,
    so the fp16 weights are exact at any magnitude): h matches the oracle to the fp16
    storage bound.  x is chosen so that the bound (row norm x ||x||)^2 on |h| stays in
    the range where h is stored unscaled (larger h: test_gpu_range)."""
    from synth.inputs import f32_to_bf16_bits
    print(f"[scale-extremes] 2^{lo} .. 2^{hi}", flush=True)
    inp = make_layer(4100 + lo, T=64, H=512, I=128)
    rng = np.random.default_rng(lo + 50)
    for p in (inp.gate, inp.up, inp.sh_gate, inp.sh_up):
        e = rng.integers(lo, hi + 1, size=p.scale.shape)
        m = 1.0 + rng.integers(0, 128, size=p.scale.shape) / 128.0
        s = (m * 2.0 ** e).astype(np.float32)
        p.scale[...] = f32_to_bf16_bits(s)
        p.bias[...] = f32_to_bf16_bits(-8.0 * s)
    # |x| in [2^-19, 2^-18) for the large scales (the activations then enter the GEMM
    # at a token power of two), [1, 2) for the small ones, [2^30, 2^31) for the tiny ones
    xmag = {"large": 2.0 ** -19, "small": 1.0, "tiny": 2.0 ** 30}[
        "large" if hi > 0 else ("tiny" if lo < -20 else "small")]
    mag = rng.uniform(1.0, 2.0, size=inp.x.shape) * xmag
    sign = np.where(rng.random(size=inp.x.shape) < 0.5, -1.0, 1.0)
    inp.x[...] = f32_to_bf16_bits((sign * mag).astype(np.float32))
    run = LayerRun(inp).route().gemm().sync()
    got = run.routing_np()
    h = f16_np(run.h)
    L = oracle.Layer(inp)
    T, k = inp.T, inp.top_k
    for t in range(0, T, 7):
        for j in (0, 3, 7):
            e = int(got["ids"][t, j])
            a = L.expert_act(e, t)
            r = int(got["tok_row"][t, j])
            bound = 2.0 ** -10 * np.abs(a) + 1e-4 * np.sqrt(np.mean(a ** 2))
            assert np.all(np.abs(h[r] - a) <= bound), (t, j, e, np.max(np.abs(h[r] - a) - bound))
        a = L.expert_act(inp.E, t)
        bound = 2.0 ** -10 * np.abs(a) + 1e-4 * np.sqrt(np.mean(a ** 2))
        assert np.all(np.abs(h[T * k + t] - a) <= bound), t
