"""GPU routing vs the oracle: logits, ids, counts, offsets, scatter and block map bit-exact."""
import numpy as np
import pytest

import oracle
from synth import make_layer
from moe_case import LayerRun, check_topk_weights

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny", dict(T=32, H=512, I=128), 1000),
    ("tiny_zipf", dict(T=32, H=512, I=128, zipf_s=1.1), 1001),
    ("ragged33", dict(T=33, H=512, I=128), 1002),
    ("ragged129", dict(T=129, H=512, I=128, zipf_s=1.1), 1003),
    ("decode_shape", dict(T=1, H=2048, I=512), 2000),
    ("prefill512", dict(T=512, H=2048, I=512), 3000),
    ("prefill2048_zipf", dict(T=2048, H=2048, I=512, zipf_s=1.1), 4000),
    ("prefill2048_zipf_s1", dict(T=2048, H=2048, I=512, zipf_s=1.1), 4001),
    # one layer of the 40-layer stack workload (T=4096, random router)
    ("stack_layer_T4096", dict(T=4096, H=2048, I=512), 5000),
]


def compare_routing(inp, got):
    l_ref = oracle.router_logits(inp.x, inp.router_wt, inp.router_bias)
    if got["logits"] is not None:
        np.testing.assert_array_equal(got["logits"].view(np.uint32), l_ref.view(np.uint32))
    ids_ref, w_ref = oracle.topk(l_ref, inp.top_k)
    np.testing.assert_array_equal(got["ids"], ids_ref)
    # weights: both routing modes take them from the picks' fixed-order logits
    check_topk_weights(got["w"], w_ref)
    _, _, BM = 0, 0, 128
    ref = oracle.routing(ids_ref, inp.E, BM)
    for key in ("counts", "offsets", "row_token", "tok_row"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    assert got["num_blocks"] == ref["num_blocks"]
    np.testing.assert_array_equal(got["blocks"], ref["blocks"])
    # row weights are the pick weights moved to their rows, bit for bit
    np.testing.assert_array_equal(got["row_w"][got["tok_row"].ravel()], got["w"].ravel())


@pytest.mark.parametrize("logits", [False, True], ids=["fast", "all_logits"])
@pytest.mark.parametrize("name,kw,seed", CASES, ids=[c[0] for c in CASES])
def test_route_matches_oracle(name, kw, seed, logits):
    print(f"[route] {name} seed={seed} {kw} logits={logits}", flush=True)
    inp = make_layer(seed, **kw)
    run = LayerRun(inp, logits=logits).route().sync()
    compare_routing(inp, run.routing_np())


@pytest.mark.parametrize("logits", [False, True], ids=["fast", "all_logits"])
def test_route_forced_ties_and_hot_experts(logits):
    """Duplicate router rows (exact ties) and a bias that sends every token to experts 0..7."""
    inp = make_layer(1010, T=100, H=512, I=128)
    inp.router_wt[7] = inp.router_wt[200]        # experts 7 and 200 always tie
    inp.router_wt[3] = inp.router_wt[4]
    inp.router_bias = np.zeros(inp.E, np.float32)
    inp.router_bias[:8] = 40.0
    run = LayerRun(inp, logits=logits).route().sync()
    got = run.routing_np()
    compare_routing(inp, got)
    assert set(np.unique(got["ids"]).tolist()) == set(range(8))
    assert got["num_blocks"] == 8


@pytest.mark.parametrize("logits", [False, True], ids=["fast", "all_logits"])
def test_route_exact_ties_everywhere(logits):
    """Zero router: every logit ties, so the certified path must fall back and pick 0..7."""
    inp = make_layer(1011, T=40, H=512, I=128)
    inp.router_wt[:] = 0
    run = LayerRun(inp, logits=logits).route().sync()
    got = run.routing_np()
    compare_routing(inp, got)
    assert np.all(got["ids"] == np.arange(8))


@pytest.mark.parametrize("logits", [False, True], ids=["fast", "all_logits"])
def test_route_near_ties_take_the_exact_path(logits):
    """Router rows that differ in one low bit: approximate intervals overlap, exact order decides."""
    inp = make_layer(1012, T=64, H=2048, I=512)
    rng = np.random.default_rng(0)
    for e in range(0, 64, 2):
        inp.router_wt[e + 1] = inp.router_wt[e]
        k = int(rng.integers(0, inp.H))
        inp.router_wt[e + 1, k] ^= 1               # one ulp of one bf16 weight
    run = LayerRun(inp, logits=logits).route().sync()
    compare_routing(inp, run.routing_np())


def test_route_deterministic_repeats():
    inp = make_layer(4002, T=2048, H=2048, I=512, zipf_s=1.1)
    run = LayerRun(inp)
    first = None
    for _ in range(5):
        run.route().sync()
        got = run.routing_np()
        if first is None:
            first = got
            continue
        for k in ("logits", "ids", "w", "row_token", "tok_row", "blocks", "counts"):
            np.testing.assert_array_equal(got[k], first[k])
