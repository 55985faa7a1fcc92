"""Pins for the CPU oracle (no GPU).

The Lily pages print no worked example for the mixture-of-experts layer, so the
oracle is pinned by closed forms, hand-derived fixtures (tests/golden), library
routines (math.fsum, numpy argsort/softmax) and dense brute force, chosen so
that a dropped term, a wrong sign or index, or a transposed operand anywhere in
the oracle fails at least one test.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from synth import bf16_bits_to_f32, f32_to_bf16_bits, make_layer, make_projection

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U = 2.0 ** -24   # unit roundoff of float32


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture(scope="module")
def tiny():
    return make_layer(1000, T=32, H=512, I=128)


@pytest.fixture(scope="module")
def tiny_layer(tiny):
    return oracle.Layer(tiny)


# ---------------------------------------------------------------- format ---

def test_unpack_golden():
    g = _golden("unpack.json")
    for case in g["cases"]:
        words = np.array([int(w, 16) for w in case["words"]], np.uint32)
        K = 8 * len(words)
        got = [oracle.code(words, K, 0, k) for k in range(K)]
        assert got == case["codes"], case


def test_pack_roundtrip():
    rng = np.random.default_rng(1)
    N, K = 5, 128
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint32)
    # independent packer: word = sum_i code_i << 4i
    words = np.zeros((N, K // 8), np.uint32)
    for i in range(8):
        words |= codes[:, i::8] << np.uint32(4 * i)
    for n in range(N):
        for k in range(K):
            assert oracle.code(words, K, n, k) == codes[n, k]


def test_dequant_closed_form_all_codes():
    # every code against a sweep of bf16 scales across the exponent range,
    # with bias = -8*scale (the workload) and with an unrelated bias
    scales = f32_to_bf16_bits(np.array([2.0 ** -20, 0.002, 0.0123, 0.02, 1.0, 3.75, 2.0 ** 10,
                                        -0.5], np.float32))
    K = 64
    for s16 in scales:
        s = float(bf16_bits_to_f32(np.array([s16]))[0])
        for bias in (-8.0 * s, 0.3125):
            b16 = f32_to_bf16_bits(np.array([bias], np.float32))
            b = float(bf16_bits_to_f32(b16)[0])
            for code in range(16):
                word = np.uint32(sum(code << (4 * i) for i in range(8)))
                q = np.full((1, K // 8), word, np.uint32)
                w = oracle.dequant(q, np.array([[s16]]), b16.reshape(1, 1), 1, K)
                exact = Fraction(code) * Fraction(s) + Fraction(b)
                assert all(Fraction(v) == exact for v in w[0]), (code, s, b)
                if bias == -8.0 * s:
                    assert w[0, 0] == (code - 8) * s


def test_dequant_matches_numpy_unpack():
    rng = np.random.default_rng(2)
    N, K = 48, 256
    p = make_projection(rng, (), N, K)
    w = oracle.dequant(p.q, p.scale, p.bias, N, K)
    shifts = np.arange(8, dtype=np.uint32) * 4
    codes = ((p.q[:, :, None] >> shifts) & 0xF).reshape(N, K).astype(np.float64)
    s = np.repeat(bf16_bits_to_f32(p.scale).astype(np.float64), 64, axis=1)
    b = np.repeat(bf16_bits_to_f32(p.bias).astype(np.float64), 64, axis=1)
    np.testing.assert_array_equal(w, codes * s + b)
    # groups run along K: changing one scale changes exactly 64 consecutive weights of one row
    s2 = p.scale.copy()
    s2[3, 2] = f32_to_bf16_bits(np.array([1.0], np.float32))[0]
    w2 = oracle.dequant(p.q, s2, p.bias, N, K)
    diff = np.argwhere(w2 != w)
    assert set(diff[:, 0]) == {3} and diff[:, 1].min() >= 128 and diff[:, 1].max() < 192


# ---------------------------------------------------------------- router ---

def _expand(spec, H):
    out = np.zeros(H, np.uint16)
    for key, val in spec.items():
        v = int(val, 16)
        if key in ("all",):
            out[:] = v
        elif key == "rest":
            pass
        elif ".." in key:
            a, b = key.split("..")
            out[int(a):int(b) + 1] = v
        else:
            out[int(key)] = v
    if "rest" in spec:
        mask = np.ones(H, bool)
        for key in spec:
            if key == "rest":
                continue
            if ".." in key:
                a, b = key.split("..")
                mask[int(a):int(b) + 1] = False
            elif key != "all":
                mask[int(key)] = False
        out[mask] = int(spec["rest"], 16)
    return out


def test_router_order_golden():
    for case in _golden("router_order.json")["cases"]:
        H = case["H"]
        x = _expand(case["x"], H).reshape(1, H)
        w = _expand(case["w"], H).reshape(1, H)
        bias = None
        if case["bias"] is not None:
            bias = np.array([int(case["bias"], 16)], np.uint32).view(np.float32)
        l = oracle.router_logits(x, w, bias)
        assert hex(int(l.view(np.uint32)[0, 0])) == hex(int(case["expected_f32"], 16)), case["name"]


def _exact_logits(inp):
    """Logits from math.fsum over exact float64 products: the exactly rounded dot product."""
    x = bf16_bits_to_f32(inp.x).astype(np.float64)
    w = bf16_bits_to_f32(inp.router_wt).astype(np.float64)
    T, E = x.shape[0], w.shape[0]
    out = np.empty((T, E))
    mag = np.empty((T, E))
    for t in range(T):
        p = x[t][None, :] * w          # exact: bf16 x bf16 fits in float64
        for e in range(E):
            out[t, e] = math.fsum(p[e])
        mag[t] = np.abs(p).sum(axis=1)
    if inp.router_bias is not None:
        out += inp.router_bias.astype(np.float64)
        mag += np.abs(inp.router_bias.astype(np.float64))
    return out, mag


@pytest.mark.parametrize("zipf", [None, 1.1])
def test_router_within_error_bound_of_exact(zipf):
    inp = make_layer(1001, T=32, H=512, I=128, zipf_s=zipf)
    l = oracle.router_logits(inp.x, inp.router_wt, inp.router_bias).astype(np.float64)
    exact, mag = _exact_logits(inp)
    # every product takes part in at most 63 in-chunk additions, H/64 - 1
    # chunk additions and one bias addition (Higham, recursive summation)
    n = 63 + inp.H // 64 - 1 + 1
    gamma = n * U / (1 - n * U)
    bound = gamma * mag
    assert np.all(np.abs(l - exact) <= bound + 1e-15 * np.abs(exact))
    # canonical order vs exact: same top-8 set wherever the exact 8th/9th gap exceeds 2*bound
    srt = np.sort(exact, axis=1)[:, ::-1]
    gap = srt[:, 7] - srt[:, 8]
    ids, _ = oracle.topk(l.astype(np.float32), 8)
    certified = 0
    for t in range(inp.T):
        if gap[t] > 2 * bound[t].max():
            ex = set(np.argsort(-exact[t], kind="stable")[:8].tolist())
            assert set(ids[t].tolist()) == ex
            certified += 1
    assert certified >= inp.T - 2


def test_router_canonical_order_numpy():
    # the same order written with numpy's sequential accumulate in float32
    inp = make_layer(1002, T=8, H=512, I=128, zipf_s=1.1)
    x = bf16_bits_to_f32(inp.x)
    w = bf16_bits_to_f32(inp.router_wt)
    p = x[:, None, :] * w[None, :, :]                       # exact products, float32
    chunks = p.reshape(inp.T, inp.E, inp.H // 64, 64)
    part = np.add.accumulate(chunks, axis=3, dtype=np.float32)[..., -1]
    tot = np.add.accumulate(part, axis=2, dtype=np.float32)[..., -1]
    tot = (tot + inp.router_bias[None, :]).astype(np.float32)
    l = oracle.router_logits(inp.x, inp.router_wt, inp.router_bias)
    np.testing.assert_array_equal(l.view(np.uint32), tot.view(np.uint32))


# ----------------------------------------------------------------- top-k ---

def test_topk_textbook_sort(tiny):
    l = oracle.router_logits(tiny.x, tiny.router_wt)
    ids, _ = oracle.topk(l, 8)
    for t in range(tiny.T):
        ref = sorted(range(tiny.E), key=lambda e: (-float(l[t, e]), e))[:8]
        assert ids[t].tolist() == ref


def test_ep_share_bias_keeps_picks_on_the_share():
    """The expert-parallel share workload: with experts 32-255 biased by -32, every token's
    top-8 lies in experts 0-31, and the routing covers only those experts."""
    inp = make_layer(6000, T=64, H=512, I=128, ep_share=8)
    l = oracle.router_logits(inp.x, inp.router_wt, inp.router_bias)
    ids, _ = oracle.topk(l, 8)
    assert ids.max() < 32 and ids.min() >= 0
    r = oracle.routing(ids, inp.E, 128)
    assert (np.asarray(r["counts"])[32:] == 0).all() and int(np.asarray(r["counts"]).sum()) == 64 * 8


def test_topk_ties_lower_index():
    rng = np.random.default_rng(5)
    E = 256
    l = rng.standard_normal((6, E)).astype(np.float32)
    l[0, :] = 0.0                               # all tied -> 0..7
    l[1, [200, 3, 77]] = 9.0                    # three-way tie at the top
    l[2, 10:20] = 5.0                           # ten-way tie straddling the cut
    l[3, [250, 251]] = np.float32(-0.0), 0.0    # signed zeros compare equal
    l[3, :250] = -1.0
    l[3, 252:] = -2.0
    ids, w = oracle.topk(l, 8)
    assert ids[0].tolist() == list(range(8))
    assert ids[1, :3].tolist() == [3, 77, 200]
    assert ids[2].tolist() == list(range(10, 18))
    assert ids[3, :2].tolist() == [250, 251]
    np.testing.assert_allclose(w[0], 1 / 8, rtol=0, atol=1e-15)


def test_router_duplicate_rows_tie():
    inp = make_layer(1003, T=16, H=512, I=128)
    wr = inp.router_wt.copy()
    l0 = oracle.router_logits(inp.x, wr)
    top = np.argsort(-l0, axis=1, kind="stable")[:, 0]
    # copy each token's winner row onto a lower expert index -> exact tie, lower index must win
    for t in range(2):
        e = int(top[t])
        if e == 0:
            continue
        wr2 = wr.copy()
        wr2[e - 1] = wr2[e]
        l = oracle.router_logits(inp.x, wr2)
        assert l[t, e - 1] == l[t, e]
        ids, _ = oracle.topk(l, 8)
        pos = ids[t].tolist()
        assert pos.index(e - 1) + 1 == pos.index(e)


def test_weights_full_softmax_renormalised(tiny):
    l = oracle.router_logits(tiny.x, tiny.router_wt)
    ids, w = oracle.topk(l, 8)
    ld = l.astype(np.float64)
    full = np.exp(ld - ld.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)                  # softmax over all 256
    sel = np.take_along_axis(full, ids.astype(np.int64), axis=1)
    ref = sel / sel.sum(axis=1, keepdims=True)               # renormalise over the picks
    np.testing.assert_allclose(w, ref, rtol=1e-12, atol=0)
    assert np.all(np.abs(w.sum(axis=1) - 1) <= 1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)


# --------------------------------------------------------------- routing ---

def _check_routing(ids, E, BM, r):
    T, k = ids.shape
    counts, offsets = r["counts"], r["offsets"]
    assert counts.sum() == T * k
    np.testing.assert_array_equal(counts, np.bincount(ids.ravel(), minlength=E))
    assert offsets[0] == 0 and offsets[E] == T * k
    np.testing.assert_array_equal(np.diff(offsets), counts)
    order = np.argsort(ids.ravel(), kind="stable")           # (expert, token) order
    np.testing.assert_array_equal(r["row_token"], order // k)
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    np.testing.assert_array_equal(r["tok_row"].ravel(), inv)
    for t in range(T):
        assert len(set(ids[t].tolist())) == k
    blocks, nb = r["blocks"], r["num_blocks"]
    assert nb == int(np.sum(-(-counts // BM)))
    cover = np.zeros(T * k, np.int32)
    prev = (-1, -1)
    for e, r0, n in blocks:
        assert 1 <= n <= BM and offsets[e] <= r0 and r0 + n <= offsets[e + 1]
        assert (e, r0) > prev
        prev = (e, r0)
        cover[r0:r0 + n] += 1
    assert np.all(cover == 1)


@pytest.mark.parametrize("BM", [16, 64, 128])
def test_routing_invariants(tiny, BM):
    l = oracle.router_logits(tiny.x, tiny.router_wt)
    ids, _ = oracle.topk(l, 8)
    _check_routing(ids, tiny.E, BM, oracle.routing(ids, tiny.E, BM))


def test_routing_invariants_adversarial():
    E, k, T = 256, 8, 100
    # all tokens on experts 0..7; only 8 experts used
    ids = np.tile(np.arange(8, dtype=np.int32), (T, 1))
    for BM in (16, 100, 128):
        _check_routing(ids, E, BM, oracle.routing(ids, E, BM))
    # random permutations per token
    rng = np.random.default_rng(9)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _check_routing(ids, E, 32, oracle.routing(ids, E, 32))


# ------------------------------------------------------------------ layer ---

def _np_dequant(p, N, K):
    shifts = np.arange(8, dtype=np.uint32) * 4
    lead = p.q.shape[:-2]
    codes = ((p.q[..., None] >> shifts) & 0xF).reshape(lead + (N, K)).astype(np.float64)
    s = np.repeat(bf16_bits_to_f32(p.scale).astype(np.float64), 64, axis=-1)
    b = np.repeat(bf16_bits_to_f32(p.bias).astype(np.float64), 64, axis=-1)
    return codes * s + b


def _np_swiglu(X, Wg, Wu, Wd):
    g = X @ Wg.T
    u = X @ Wu.T
    return ((g / (1 + np.exp(-g))) * u) @ Wd.T


def _np_routing(inp):
    """Routing re-derived with numpy: canonical-order logits, sort, full softmax renormalised."""
    x = bf16_bits_to_f32(inp.x)
    w = bf16_bits_to_f32(inp.router_wt)
    p = x[:, None, :] * w[None, :, :]
    part = np.add.accumulate(p.reshape(inp.T, inp.E, -1, 64), axis=3, dtype=np.float32)[..., -1]
    l = np.add.accumulate(part, axis=2, dtype=np.float32)[..., -1]
    if inp.router_bias is not None:
        l = (l + inp.router_bias[None, :]).astype(np.float32)
    G = np.zeros((inp.T, inp.E))
    for t in range(inp.T):
        ids = sorted(range(inp.E), key=lambda e: (-float(l[t, e]), e))[:inp.top_k]
        z = np.exp(l[t].astype(np.float64) - l[t].max())
        G[t, ids] = z[ids] / z[ids].sum()
    return G


def test_layer_dense_bruteforce(tiny, tiny_layer):
    """Per-token loop == dense evaluation of all 256 experts times a 0-off-top-8 gate matrix."""
    inp = tiny
    X = bf16_bits_to_f32(inp.x).astype(np.float64)
    G = _np_routing(inp)
    Wg = _np_dequant(inp.gate, inp.I, inp.H)
    Wu = _np_dequant(inp.up, inp.I, inp.H)
    Wd = _np_dequant(inp.down, inp.H, inp.I)
    y = np.zeros((inp.T, inp.H))
    for e in range(inp.E):
        y += G[:, e:e + 1] * _np_swiglu(X, Wg[e], Wu[e], Wd[e])
    y += _np_swiglu(X, _np_dequant(inp.sh_gate, inp.I, inp.H), _np_dequant(inp.sh_up, inp.I, inp.H),
                    _np_dequant(inp.sh_down, inp.H, inp.I))
    yo, ids, w = tiny_layer.tokens(range(inp.T))
    assert np.max(np.abs(yo - y)) <= 1e-12 * np.max(np.abs(y))
    for t in range(inp.T):
        assert set(np.nonzero(G[t])[0].tolist()) == set(ids[t].tolist())
        np.testing.assert_allclose(G[t, ids[t]], w[t], rtol=1e-12)


def test_layer_expert_parts(tiny, tiny_layer):
    """expert_act / expert_down against numpy for a routed and the shared expert."""
    X = bf16_bits_to_f32(tiny.x).astype(np.float64)
    for e in (0, 131, tiny.E):
        if e == tiny.E:
            Wg, Wu = _np_dequant(tiny.sh_gate, tiny.I, tiny.H), _np_dequant(tiny.sh_up, tiny.I, tiny.H)
            Wd = _np_dequant(tiny.sh_down, tiny.H, tiny.I)
        else:
            Wg = _np_dequant(tiny.gate, tiny.I, tiny.H)[e]
            Wu = _np_dequant(tiny.up, tiny.I, tiny.H)[e]
            Wd = _np_dequant(tiny.down, tiny.H, tiny.I)[e]
        g, u = Wg @ X[5], Wu @ X[5]
        a_ref = g / (1 + np.exp(-g)) * u
        a = tiny_layer.expert_act(e, 5)
        np.testing.assert_allclose(a, a_ref, rtol=1e-12, atol=1e-13 * np.abs(a_ref).max())
        o = tiny_layer.expert_down(e, a)
        np.testing.assert_allclose(o, Wd @ a, rtol=1e-12, atol=1e-13 * np.abs(o).max())


def _zero_codes(p):
    # code 8 with bias = -8*scale gives a zero weight
    p.q[...] = np.uint32(0x88888888)


def test_layer_zero_experts_shared_only():
    inp = make_layer(1004, T=4, H=512, I=128)
    for p in (inp.gate, inp.up, inp.down):
        _zero_codes(p)
    L = oracle.Layer(inp)
    y, _, _ = L.tokens(range(4))
    X = bf16_bits_to_f32(inp.x).astype(np.float64)
    ref = _np_swiglu(X, _np_dequant(inp.sh_gate, inp.I, inp.H), _np_dequant(inp.sh_up, inp.I, inp.H),
                     _np_dequant(inp.sh_down, inp.H, inp.I))
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    for p in (inp.sh_gate, inp.sh_up, inp.sh_down):
        _zero_codes(p)
    y0, _, _ = oracle.Layer(inp).tokens(range(4))
    assert np.all(y0 == 0.0)


def test_layer_single_live_expert():
    inp = make_layer(1005, T=3, H=512, I=128)
    live = 77
    keep = [p.q[live].copy() for p in (inp.gate, inp.up, inp.down)]
    for p, kq in zip((inp.gate, inp.up, inp.down), keep):
        _zero_codes(p)
        p.q[live] = kq
    for p in (inp.sh_gate, inp.sh_up, inp.sh_down):
        _zero_codes(p)
    inp.router_bias = np.zeros(inp.E, np.float32)
    inp.router_bias[live] = 50.0        # force the live expert into every token's top-8
    y, ids, w = oracle.Layer(inp).tokens(range(3))
    X = bf16_bits_to_f32(inp.x).astype(np.float64)
    o = _np_swiglu(X, _np_dequant(inp.gate, inp.I, inp.H)[live], _np_dequant(inp.up, inp.I, inp.H)[live],
                   _np_dequant(inp.down, inp.H, inp.I)[live])
    for t in range(3):
        assert ids[t, 0] == live
        np.testing.assert_allclose(y[t], w[t, 0] * o[t], rtol=1e-12, atol=1e-12 * np.abs(o).max())
        assert w[t, 0] > 0.999


def test_layer_closed_form_golden():
    g = _golden("swiglu_uniform.json")
    sh = g["shape"]
    inp = make_layer(0, T=sh["T"], H=sh["H"], I=sh["I"], E=sh["E"])
    inp.x[:] = 0x3C80
    inp.router_wt[:] = 0
    for p in (inp.gate, inp.up, inp.down, inp.sh_gate, inp.sh_up, inp.sh_down):
        p.q[...] = np.uint32(0x99999999)
        p.scale[...] = 0x3F80
        p.bias[...] = 0xC100
    y, ids, w = oracle.Layer(inp).tokens([0])
    assert ids[0].tolist() == g["expected"]["ids"]
    np.testing.assert_allclose(w[0], g["expected"]["w"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(y[0], g["expected"]["y_all"], rtol=1e-14)


def test_layer_zipf_routing_is_skewed():
    inp = make_layer(4000, T=256, H=512, I=128, zipf_s=1.1)
    l = oracle.router_logits(inp.x, inp.router_wt, inp.router_bias)
    ids, _ = oracle.topk(l, 8)
    counts = np.bincount(ids.ravel(), minlength=256)
    assert counts[0] > 0.8 * inp.T and (counts == 0).sum() > 64


# --------------------------------------------------------------- rmsnorm ---

def test_rmsnorm_closed_form():
    rng = np.random.default_rng(11)
    r = rng.standard_normal((6, 2048)) * 3.0
    y = rng.standard_normal((6, 2048))
    eps = 1e-6
    r_out, u = oracle.rmsnorm_residual(r, y, eps)
    np.testing.assert_array_equal(r_out, r + y)
    uf = bf16_bits_to_f32(u).astype(np.float64)
    ms = (r_out ** 2).mean(axis=1)
    # before rounding, mean(u^2) = ms / (ms + eps); bf16 rounding moves each u by <= 2^-8 relative
    np.testing.assert_allclose((uf ** 2).mean(axis=1), ms / (ms + eps), rtol=2 ** -7)
    ref = r_out / np.sqrt(ms + eps)[:, None]
    assert np.all(np.abs(uf - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)


def _bf16_rne_direct(v):
    """float64 -> nearest bfloat16 value (8 significant bits), ties to even, written from the
    format's definition: v = m 2^e with m in [0.5, 1), kept as round_half_even(m 2^8) 2^(e-8).
    Also returns the distance of m 2^8 from the nearest tie, to flag near-ties."""
    m, e = np.frexp(v)
    scaled = m * 256.0
    k = np.rint(scaled)                                   # numpy rounds halves to even
    frac = np.abs(scaled - np.floor(scaled) - 0.5)
    return np.ldexp(k, e - 8), frac


@pytest.mark.parametrize("H,eps", [(2048, 1e-6), (64, 1e-6), (512, 0.25), (96, 3.0)])
def test_rmsnorm_bit_exact_direct_rounding(H, eps):
    """u bit for bit against the definition r/sqrt(mean(r^2) + eps) evaluated in float64 and
    rounded once to bfloat16 (the oracle rounds through float32 first, which can only differ at
    near-ties, skipped here).  A large eps and a short row make eps and the 1/H of the mean
    visible in most roundings (a missing eps or a mean over H - 1 fails)."""
    rng = np.random.default_rng(H + 7)
    T = 16
    r = rng.standard_normal((T, H)) * 1.5
    y = rng.standard_normal((T, H)) * 0.5
    r_out, u = oracle.rmsnorm_residual(r, y, eps)
    s = r + y
    ms = np.array([sum(float(v) * float(v) for v in row) for row in s]) / H
    ref, frac = _bf16_rne_direct(s / np.sqrt(ms + eps)[:, None])
    got = bf16_bits_to_f32(u).astype(np.float64)
    near_tie = frac < 1e-9
    assert near_tie.mean() < 1e-3
    np.testing.assert_array_equal(got[~near_tie], ref[~near_tie])
    # the rounding really depends on eps and on the 1/H of the mean
    alt, _ = _bf16_rne_direct(s / np.sqrt(ms * H / (H - 1) + eps)[:, None])
    assert np.mean(alt != ref) > 0.005
    if eps > 1e-3:
        alt, _ = _bf16_rne_direct(s / np.sqrt(ms)[:, None])
        assert np.mean(alt != ref) > 0.05
