"""Stacked layers with a residual add and RMSNorm between them (the 40-layer stack
workload's structure, on fewer layers), teacher-forced against the oracle: every
layer's oracle reference takes the GPU's own bf16 input u_l, so errors do not
compound and each layer is held to the single-layer bar."""
import numpy as np
import pytest
import torch

import bit_quantized_expert_top_amd as moe
import oracle
from moe_case import LayerRun, check_y, device
from synth import make_layer
from synth.inputs import bf16_bits_to_f32

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,H,I,layers,nsamp", [
    (64, 512, 128, 4, 64),
    (256, 2048, 512, 3, 256),
    # the stack workload's own shape (T=4096), three layers, a quarter of the tokens each
    (4096, 2048, 512, 3, 1024),
])
def test_stack_teacher_forced(T, H, I, layers, nsamp):
    print(f"[stack] T={T} H={H} I={I} layers={layers}", flush=True)
    dev = device()
    x0 = make_layer(5000, T=T, H=H, I=I).x                      # stack input, bf16 bits
    r = torch.from_numpy(bf16_bits_to_f32(x0).copy()).to(dev)     # residual r_0 = x
    u = torch.from_numpy(x0.copy()).view(torch.int16).to(dev)     # layer input u_0 = x
    rng = np.random.default_rng(T + layers)
    toks = sorted(set(rng.choice(T, size=min(nsamp, T), replace=False).tolist()) | {0, T - 1})
    for layer in range(layers):
        inp = make_layer(5000 + layer, T=T, H=H, I=I, with_x=False)
        inp.x = u.cpu().numpy().view(np.uint16).copy()             # teacher forcing
        run = LayerRun(inp).layer().sync()
        y = run.y.cpu().numpy()
        y_ref, ids_ref, _ = oracle.Layer(inp).tokens(toks)
        np.testing.assert_array_equal(run.routing_np()["ids"][toks], ids_ref)
        ratio = check_y(y[toks], y_ref)
        print(f"  layer {layer}: max err / rms = {ratio:.4g}", flush=True)
        # residual add + RMSNorm into the next layer's input
        r_prev = r.cpu().numpy()
        moe.moe_rmsnorm_residual(T, H, 1e-6, r, run.y, u)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(r.cpu().numpy(), r_prev + y)   # fp32 add
        _, u_ref = oracle.rmsnorm_residual(r_prev.astype(np.float64), y.astype(np.float64), 1e-6)
        ug = bf16_bits_to_f32(u.cpu().numpy().view(np.uint16)).astype(np.float64)
        ur = bf16_bits_to_f32(u_ref).astype(np.float64)
        # the oracle adds in fp64, the GPU in fp32: at most one bf16 ulp apart
        assert np.all(np.abs(ug - ur) <= 2.0 ** -7 * np.abs(ur) + 1e-30), layer


@pytest.mark.parametrize("T,H,I", [(64, 512, 128), (333, 768, 384), (4096, 2048, 512)])
def test_fused_down_residual_norm_is_bit_identical(T, H, I):
    """moe_down_combine_residual gives exactly the residual and the next layer's input that
    moe_down_combine followed by moe_rmsnorm_residual give (ragged T, another H, the stack
    workload's T), on every element."""
    print(f"[stack] fused down + residual + norm, T={T} H={H} I={I}", flush=True)
    dev = device()
    inp = make_layer(5100 + T, T=T, H=H, I=I)
    run = LayerRun(inp).route().gemm().sync()
    g = torch.Generator(device="cpu").manual_seed(T)
    r0 = (torch.randn((T, H), generator=g) * 3.0).to(dev)
    # unfused: y, then r += y and u = norm(r)
    run.down().sync()
    r_a = r0.clone()
    u_a = torch.empty((T, H), dtype=torch.int16, device=dev)
    moe.moe_rmsnorm_residual(T, H, 1e-6, r_a, run.y, u_a)
    # fused (y is scratch there)
    r_b = r0.clone()
    u_b = torch.empty((T, H), dtype=torch.int16, device=dev)
    y_b = torch.empty((T, H), dtype=torch.float32, device=dev)
    moe.moe_down_combine_residual(run.shape, run.h, run.w, run.r, y_b, r_b, 1e-6, u_b, run.ws)
    torch.cuda.synchronize()
    assert torch.equal(r_a, r_b)
    assert torch.equal(u_a, u_b)
    assert torch.all(torch.isfinite(r_b))
