"""moe_expert_ffn_q4 (both expert GEMMs in one persistent launch) against the two calls it
replaces, moe_expert_gemm_q4 + moe_down_combine: h and y bit for bit, over the layer shapes
(tiny to T=4096, ragged, narrow and wide, one expert-parallel share), with asymmetric biases
(the rank-G term reads h's group sums across XCDs), repeated calls and graph replays (the
launch's queue and per-block counters are zeroed again by its last workgroup), one workspace
reused across token counts, and malformed block maps (skipped items still report)."""
import numpy as np
import pytest
import torch

import bit_quantized_expert_top_amd as moe
from moe_case import LayerRun, asymmetric_bias, check_y, oracle_tokens
from synth import make_layer

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny", dict(T=32, H=512, I=128), 1000),
    ("ragged129_zipf", dict(T=129, H=512, I=128, zipf_s=1.1), 1003),
    ("T1", dict(T=1, H=2048, I=512), 2001),
    ("T3", dict(T=3, H=2048, I=512), 2002),
    ("prefill512", dict(T=512, H=2048, I=512), 3000),
    ("prefill2048_zipf", dict(T=2048, H=2048, I=512, zipf_s=1.1), 4000),
    ("stack_layer_T4096", dict(T=4096, H=2048, I=512), 5000),
    ("narrowH_wideI", dict(T=77, H=256, I=1024), 4200),
    ("H768_I384", dict(T=200, H=768, I=384, zipf_s=1.1), 4201),
    ("ep8_share_T2048", dict(T=2048, H=2048, I=512, ep_share=8), 6000),
]


def two_calls(run):
    run.h.zero_()
    run.y.zero_()
    run.gemm().down().sync()
    return run.h.clone(), run.y.clone()


def fused(run, fill=0):
    run.h.fill_(fill)
    run.y.fill_(float("nan"))
    moe.moe_expert_ffn_q4(run.shape, run.x, run.w, run.r, run.h, run.y, run.ws)
    torch.cuda.synchronize()
    return run.h.clone(), run.y.clone()


def assert_same(a, b, what):
    if not torch.equal(a, b):
        diff = (a != b).nonzero()
        raise AssertionError(f"{what}: {diff.shape[0]} elements differ, first at {diff[0].tolist()}")


@pytest.mark.parametrize("name,kw,seed", CASES, ids=[c[0] for c in CASES])
def test_ffn_bit_identical_to_two_calls(name, kw, seed):
    print(f"[ffn] {name} seed={seed} {kw}", flush=True)
    inp = make_layer(seed, **kw)
    run = LayerRun(inp).route().sync()
    h2, y2 = two_calls(run)
    for rep in range(3):                     # the counters start from zero on every call
        h1, y1 = fused(run, fill=rep)
        nrows = inp.T * inp.top_k + inp.T
        assert_same(h1[:nrows], h2[:nrows], f"h (call {rep})")
        assert_same(y1, y2, f"y (call {rep})")


def test_ffn_asymmetric_bias_bit_identical_and_oracle():
    """Biases away from -8 s in half of the groups: down items start from the rank-G term over
    h's group sums, which the gate/up items of the same launch wrote on other XCDs."""
    seed = 4300
    inp = make_layer(seed, T=1024, H=2048, I=512, zipf_s=1.1)
    asymmetric_bias(inp, seed)
    run = LayerRun(inp).route().sync()
    h2, y2 = two_calls(run)
    h1, y1 = fused(run)
    assert_same(h1, h2, "h")
    assert_same(y1, y2, "y")
    toks = [0, 1, 511, 1022, 1023]
    y_ref, _, _ = oracle_tokens(inp, toks)
    ratio = check_y(y1.cpu().numpy()[toks], y_ref)
    print(f"  max err / rms = {ratio:.4g}", flush=True)


def test_ffn_graph_replays_match_eager():
    """route + ffn for two weight sets captured in one graph; three replays, with eager work and
    synchronisations between them, each equal bit for bit to the eager results."""
    dev = torch.device("cuda:0")
    inps = [make_layer(8100 + i, T=1024, H=2048, I=512, zipf_s=1.1) for i in range(2)]
    runs = [LayerRun(inp) for inp in inps]
    eager = []
    for run in runs:
        run.route().sync()
        eager.append(fused(run))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for run in runs:
                moe.moe_route(run.shape, run.x, run.w, run.r, run.ws)
                moe.moe_expert_ffn_q4(run.shape, run.x, run.w, run.r, run.h, run.y, run.ws)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for run in runs:
            run.h.fill_(7)
            run.y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, run in enumerate(runs):
            assert_same(run.h, eager[i][0], f"h replay {rep} set {i}")
            assert_same(run.y, eager[i][1], f"y replay {rep} set {i}")
        # eager work between replays
        z = torch.randn(1024, 1024, device=dev)
        (z @ z).sum().item()


def test_ffn_workspace_reused_across_token_counts():
    """One workspace (sized for the largest call) for T = 2048, 100, 2048, 1: each call's
    routing zeroes the counters of its own layout."""
    big = moe.Shape(T=2048, H=2048, I=512)
    ws = moe.workspace(big, torch.device("cuda:0"))
    for i, T in enumerate((2048, 100, 2048, 1)):
        inp = make_layer(8200 + i, T=T, H=2048, I=512, zipf_s=1.1)
        run = LayerRun(inp)
        run.ws = ws
        run.route().sync()
        h2, y2 = two_calls(run)
        h1, y1 = fused(run)
        assert_same(h1, h2, f"h T={T}")
        assert_same(y1, y2, f"y T={T}")


def test_ffn_without_combine_then_combine():
    """combine=False leaves y = the shared expert's part (the down launch's y before its combine)
    and the staged rows; moe_combine then gives the combined y, and moe_combine_residual the
    res and u of moe_down_combine_residual, bit for bit."""
    inp = make_layer(8400, T=1024, H=2048, I=512, zipf_s=1.1)
    run = LayerRun(inp).route().sync()
    h2, y2 = two_calls(run)
    # reference residual step: the two-call path's down + residual + norm
    g = torch.Generator().manual_seed(8400)
    res0 = torch.randn((inp.T, inp.H), generator=g).to(run.y.device)
    res_ref = res0.clone()
    u_ref = torch.empty((inp.T, inp.H), dtype=torch.int16, device=run.y.device)
    y_scr = torch.empty_like(run.y)
    moe.moe_down_combine_residual(run.shape, run.h, run.w, run.r, y_scr, res_ref, 1e-6, u_ref, run.ws)
    torch.cuda.synchronize()
    y_shared = y_scr.clone()                 # the shared expert's part only
    run.h.zero_()
    run.y.fill_(float("nan"))
    moe.moe_expert_ffn_q4(run.shape, run.x, run.w, run.r, run.h, run.y, run.ws, combine=False)
    torch.cuda.synchronize()
    assert_same(run.h, h2, "h")
    assert_same(run.y, y_shared, "y before the combine")
    res = res0.clone()
    u = torch.empty_like(u_ref)
    moe.moe_combine_residual(run.shape, run.r, run.y, res, 1e-6, u, run.ws)
    torch.cuda.synchronize()
    assert_same(res, res_ref, "res")
    assert_same(u, u_ref, "u")
    assert_same(run.y, y_shared, "y is only read")
    moe.moe_combine(run.shape, run.r, run.y, run.ws)
    torch.cuda.synchronize()
    assert_same(run.y, y2, "y after moe_combine")


def test_layer_uses_one_launch_path_bit_identical():
    """moe_layer (route + the one-launch FFN) equals route + the two calls."""
    inp = make_layer(8300, T=700, H=2048, I=512, zipf_s=1.1)
    run = LayerRun(inp).route().sync()
    h2, y2 = two_calls(run)
    run.h.zero_()
    run.y.zero_()
    run.layer().sync()
    assert_same(run.h, h2, "h")
    assert_same(run.y, y2, "y")


@pytest.mark.debug_flags
def test_ffn_malformed_block_map_is_skipped():
    """Three broken block map entries: their gate/up items are skipped but still counted, their
    down items skipped without waiting; every other block's h and every shared row equal the
    intact map's, the broken blocks' rows keep the sentinel, the launch ends."""
    inp = make_layer(1400, T=64, H=512, I=128)
    run = LayerRun(inp).route().sync()
    moe.moe_debug_status(clear=True)
    got = run.routing_np()
    nb = got["num_blocks"]
    assert nb >= 4
    h_ok, _ = fused(run)
    blocks = run.r.blocks.clone()
    bad = blocks.clone()
    bad[0, 0] = 300
    bad[1, 1] = -5
    bad[2, 2] = 200
    run.r.blocks.copy_(bad)
    sentinel = 0x7BFF
    h, y = fused(run, fill=sentinel)
    flags = moe.moe_debug_status(clear=True)
    h = h.cpu().numpy()
    ok_rows = np.zeros(h.shape[0], bool)
    for b in range(3, nb):
        e, r0, n = (int(v) for v in blocks[b].cpu())
        ok_rows[r0:r0 + n] = True
    ok_rows[inp.T * inp.top_k:] = True
    np.testing.assert_array_equal(h[ok_rows], h_ok.cpu().numpy()[ok_rows])
    for b in range(3):
        e, r0, n = (int(v) for v in blocks[b].cpu())
        assert np.all(h[r0:r0 + n] == sentinel), b
    if flags is not None:
        assert flags & 2, flags                          # block map entries
        assert not flags & 32, flags                     # no down item gave up waiting
    run.r.blocks.copy_(blocks)
    h2, _ = fused(run)
    np.testing.assert_array_equal(h2.cpu().numpy(), h_ok.cpu().numpy())
