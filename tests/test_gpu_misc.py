"""Dequantisation hook and the between-layer residual RMSNorm on the GPU."""
import numpy as np
import pytest
import torch

import bit_quantized_expert_top_amd as moe
import oracle
from synth import bf16_bits_to_f32, f32_to_bf16_bits, make_projection
from moe_case import device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K", [(64, 64), (512, 2048), (2048, 512), (3, 4096)])
def test_dequant_bit_exact(N, K):
    rng = np.random.default_rng(N + K)
    p = make_projection(rng, (), N, K)
    # exact weights from the oracle; q*s+b has at most ~16 significant bits, so float32 holds it exactly
    w = oracle.dequant(p.q, p.scale, p.bias, N, K)
    ref = f32_to_bf16_bits(w.astype(np.float32))
    dev = device()
    out = torch.empty((N, K), dtype=torch.int16, device=dev)
    moe.moe_dequant_q4(torch.from_numpy(p.q).view(torch.int32).to(dev),
                       torch.from_numpy(p.scale).view(torch.int16).to(dev),
                       torch.from_numpy(p.bias).view(torch.int16).to(dev), N, K, out)
    got = out.cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("T,H", [(1, 2048), (7, 512), (64, 2048)])
def test_rmsnorm_residual(T, H):
    rng = np.random.default_rng(T * H)
    r = (rng.standard_normal((T, H)) * 2).astype(np.float32)
    y = rng.standard_normal((T, H)).astype(np.float32)
    r_ref, u_ref = oracle.rmsnorm_residual(r.astype(np.float64), y.astype(np.float64), 1e-6)
    dev = device()
    rt = torch.from_numpy(r).to(dev)
    ut = torch.empty((T, H), dtype=torch.int16, device=dev)
    moe.moe_rmsnorm_residual(T, H, 1e-6, rt, torch.from_numpy(y).to(dev), ut)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(rt.cpu().numpy(), (r + y))      # fp32 add, same rounding
    u = bf16_bits_to_f32(ut.cpu().numpy().view(np.uint16)).astype(np.float64)
    uref = bf16_bits_to_f32(u_ref).astype(np.float64)
    # one bf16 ulp apart at most
    assert np.all(np.abs(u - uref) <= 2.0 ** -7 * np.abs(uref) + 1e-30)
