"""Malformed routing structures fed to the expert GEMMs and the combine on purpose: entries
of the block map out of range (an expert id past 255, a negative first row, more rows than a
block holds) and a pick's row out of range.  The kernels' own index checks skip them: the
valid blocks' rows of h come out exactly as with the intact map, the broken blocks' rows are
left untouched, and no access leaves its buffer.  A MOE_DEBUG build also records each kind."""
import numpy as np
import pytest
import torch

import bit_quantized_expert_top_amd as moe
from moe_case import LayerRun
from synth import make_layer

pytestmark = [pytest.mark.gpu, pytest.mark.debug_flags]


def test_malformed_block_map_and_rows_are_skipped():
    inp = make_layer(1400, T=64, H=512, I=128)
    run = LayerRun(inp).route().sync()
    moe.moe_debug_status(clear=True)
    got = run.routing_np()
    nb = got["num_blocks"]
    assert nb >= 4
    run.gemm().down().sync()
    h_ok, y_ok = run.h.clone(), run.y.clone()
    assert moe.moe_debug_status(clear=True) in (None, 0)

    # break three blocks of the map: expert 300, first row -5, 200 rows
    blocks = run.r.blocks.clone()
    bad = blocks.clone()
    bad[0, 0] = 300
    bad[1, 1] = -5
    bad[2, 2] = 200
    run.r.blocks.copy_(bad)
    sentinel = 0x7BFF                                   # fp16 65504: never a computed h value
    run.h.fill_(sentinel)
    run.gemm().sync()
    flags = moe.moe_debug_status(clear=True)
    h = run.h.cpu().numpy()
    ok_rows = np.zeros(run.h.shape[0], bool)
    for b in range(3, nb):
        e, r0, n = (int(v) for v in blocks[b].cpu())
        ok_rows[r0:r0 + n] = True
    ok_rows[inp.T * inp.top_k:] = True                  # the shared expert's rows
    np.testing.assert_array_equal(h[ok_rows], h_ok.cpu().numpy()[ok_rows])
    for b in range(3):
        e, r0, n = (int(v) for v in blocks[b].cpu())
        assert np.all(h[r0:r0 + n] == sentinel), b
    if flags is not None:
        assert flags & 2, flags                          # block map entries

    # an intact map again, and one pick's row out of range in the combine
    run.r.blocks.copy_(blocks)
    run.gemm().sync()
    tok_row = run.r.tok_row.clone()
    run.r.tok_row[0, 3] = 10 ** 6
    run.down().sync()
    flags = moe.moe_debug_status(clear=True)
    y = run.y.cpu().numpy()
    np.testing.assert_array_equal(y[1:], y_ok.cpu().numpy()[1:])     # other tokens unchanged
    assert np.all(np.isfinite(y[0]))
    if flags is not None:
        assert flags & 8, flags                          # combine row
    run.r.tok_row.copy_(tok_row)
