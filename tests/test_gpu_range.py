"""Inputs outside the usual magnitudes, each against the oracle: activations of 1e6 and 1e-6
(the expert GEMM takes each token at its own power of two), quantisation scales of 1e-5 and
4 (each weight row at its own power of two; hidden activations h far outside the fp16 range
are kept at a per-row power of two), tokens of wildly different magnitudes in one batch with
asymmetric biases (the rank-G bias term at large group sums), and the weights that the load
validation refuses."""
import numpy as np
import pytest
import torch

import bit_quantized_expert_top_amd as moe
import oracle
from moe_case import (LayerRun, asymmetric_bias, check_topk_weights, check_y, device, shape_of,
                      upload, x_dev)
from synth import bf16_bits_to_f32, f32_to_bf16_bits, make_layer

pytestmark = pytest.mark.gpu


def scale_x(inp, factors):
    """x times a per-token factor (bf16 rounding of the product)."""
    f = np.asarray(factors, np.float64).reshape(-1, 1)
    inp.x[...] = f32_to_bf16_bits((bf16_bits_to_f32(inp.x).astype(np.float64) * f).astype(np.float32))


def set_scales(inp, lo, hi, seed, names=("gate", "up", "down", "sh_gate", "sh_up", "sh_down")):
    rng = np.random.default_rng(seed)
    for nm in names:
        p = getattr(inp, nm)
        s = f32_to_bf16_bits(rng.uniform(lo, hi, size=p.scale.shape).astype(np.float32))
        p.scale[...] = s
        p.bias[...] = f32_to_bf16_bits(-8.0 * bf16_bits_to_f32(s))


def check_y_per_token(y, y_ref, tol=2e-2):
    """Each token's outputs within tol x that token's RMS (tokens of very different
    magnitudes in one batch: one RMS over all outputs would be the largest token's)."""
    assert np.all(np.isfinite(y)), "non-finite output"
    err = np.abs(y.astype(np.float64) - y_ref).max(axis=1)
    rms = np.sqrt((y_ref ** 2).mean(axis=1))
    ratio = err / rms
    assert np.all(ratio <= tol), (int(np.argmax(ratio)), float(ratio.max()))
    return float(ratio.max())


def layer_vs_oracle(inp, label, per_token=False):
    run = LayerRun(inp).layer().sync()
    y = run.y.cpu().numpy()
    y_ref, ids_ref, w_ref = oracle.Layer(inp).tokens(range(inp.T))
    got = run.routing_np()
    np.testing.assert_array_equal(got["ids"], ids_ref)
    check_topk_weights(got["w"], w_ref)
    ratio = check_y_per_token(y, y_ref) if per_token else check_y(y, y_ref)
    print(f"  {label}: layer max err / rms = {ratio:.4g}", flush=True)
    return run


def decode_vs_oracle(inp, label, tokens, per_token=False):
    dev = device()
    w = upload(inp, dev)
    n = len(tokens)
    sh = moe.Shape(T=n, H=inp.H, I=inp.I, E=inp.E, top_k=inp.top_k)
    x = torch.from_numpy(inp.x[tokens].copy()).view(torch.int16).to(dev)
    ids = torch.empty((n, inp.top_k), dtype=torch.int32, device=dev)
    tw = torch.empty((n, inp.top_k), dtype=torch.float32, device=dev)
    y = torch.empty((n, inp.H), dtype=torch.float32, device=dev)
    moe.moe_decode(sh, x, w, ids, tw, y, moe.workspace(sh, dev))
    torch.cuda.synchronize()
    y_ref, ids_ref, w_ref = oracle.Layer(inp).tokens(tokens)
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
    check_topk_weights(tw.cpu().numpy(), w_ref)
    ratio = check_y_per_token(y.cpu().numpy(), y_ref) if per_token else check_y(y.cpu().numpy(), y_ref)
    print(f"  {label}: decode max err / rms = {ratio:.4g}", flush=True)


@pytest.mark.parametrize("factor", [1e6, 1e-6, 3e4, 2.0 ** -10], ids=["x1e6", "x1e-6", "x3e4", "x2^-10"])
def test_activation_magnitude(factor):
    print(f"[range] x times {factor}", flush=True)
    inp = make_layer(4300, T=96, H=512, I=128)
    scale_x(inp, [factor] * inp.T)
    layer_vs_oracle(inp, f"x*{factor}")
    decode_vs_oracle(inp, f"x*{factor}", [0])


@pytest.mark.parametrize("lo,hi", [(0.5e-5, 1e-5), (2.0, 4.0), (1e-12, 3e-12)],
                         ids=["scale1e-5", "scale4", "scale1e-12"])
def test_scale_magnitude(lo, hi):
    print(f"[range] scales in [{lo}, {hi}]", flush=True)
    inp = make_layer(4301, T=64, H=1024, I=256)
    set_scales(inp, lo, hi, 7)
    layer_vs_oracle(inp, f"scale {lo}..{hi}")
    decode_vs_oracle(inp, f"scale {lo}..{hi}", [0, 5, 9])


def test_mixed_tokens_and_asymmetric_bias():
    """Per-token magnitudes from 1e-5 to 1e5 in one batch, scales up to 4 and biases b != -8 s:
    the token powers of two, the h row powers of two and the scaled rank-G term together."""
    print("[range] mixed token magnitudes, asymmetric biases", flush=True)
    inp = make_layer(4302, T=150, H=512, I=256, zipf_s=1.1)
    rng = np.random.default_rng(11)
    scale_x(inp, 10.0 ** rng.uniform(-5, 5, size=inp.T))
    set_scales(inp, 0.02, 4.0, 12)
    asymmetric_bias(inp, 13)
    layer_vs_oracle(inp, "mixed", per_token=True)
    decode_vs_oracle(inp, "mixed", [0, 1, 2, 3], per_token=True)


def test_large_hidden_rows_with_asymmetric_bias():
    """|h| around 1e8 and its 64-wide group sums far beyond 65504, with biases b != -8 s in
    the down projection (the rank-G term reads the group sums of h)."""
    print("[range] large h, asymmetric bias", flush=True)
    inp = make_layer(4303, T=80, H=512, I=128)
    scale_x(inp, [100.0] * inp.T)
    set_scales(inp, 1.0, 2.0, 14, names=("gate", "up", "sh_gate", "sh_up"))
    asymmetric_bias(inp, 15)
    run = layer_vs_oracle(inp, "large h")
    assert np.all(np.isfinite(run.y.cpu().numpy()))
    decode_vs_oracle(inp, "large h", [0, 1])


def test_row_norm_bound_keeps_h_exact_in_usual_range():
    """In the usual range (the workloads' distributions) every h row is stored unscaled."""
    inp = make_layer(4304, T=64, H=2048, I=512)
    run = LayerRun(inp).route().gemm().sync()
    from moe_case import f16_np
    h = f16_np(run.h)
    L = oracle.Layer(inp)
    got = run.routing_np()
    for t in (0, 31, 63):
        e = int(got["ids"][t, 0])
        a = L.expert_act(e, t)
        r = int(got["tok_row"][t, 0])
        bound = 2.0 ** -10 * np.abs(a) + 1e-4 * np.sqrt(np.mean(a ** 2))
        assert np.all(np.abs(h[r] - a) <= bound)


@pytest.mark.parametrize("case", ["nan_scale", "inf_bias", "scale_span"])
def test_load_refuses_unsupported_weights(case):
    inp = make_layer(4305, T=4, H=256, I=128)
    if case == "nan_scale":
        inp.up.scale[3, 5, 1] = 0x7FC0                      # NaN
    elif case == "inf_bias":
        inp.sh_down.bias[7, 0] = 0x7F80                      # +inf
    else:
        # one group's scale 2^-30 next to 2^0 in the same row: span 2^30 > 2^23
        inp.down.scale[9, 17, 0] = f32_to_bf16_bits(np.float32(2.0 ** -30))[0]
        inp.down.scale[9, 17, 1] = f32_to_bf16_bits(np.float32(1.0))[0]
    with pytest.raises(moe.UnsupportedWeights) as ex:
        upload(inp)
    want = {"nan_scale": 1, "inf_bias": 1, "scale_span": 2}[case]
    assert ex.value.flags & want, ex.value.flags
