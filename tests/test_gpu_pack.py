"""moe_pack_weights against a numpy rendering of the tile layout that
include/moe_q4.h documents: every byte of the packed buffer is checked."""
import numpy as np
import pytest

import bit_quantized_expert_top_amd as moe
from moe_case import device, upload
from synth import make_layer

pytestmark = pytest.mark.gpu

BLOCK, CODES = 9216, 8192


def _blocks(q, s, b, rows_of_col):
    """Tile-layout blocks of one stack of projections.

    q: list of uint32 [n_exp][N][K/8] code arrays (one per projection that the
    columns draw from), s/b likewise for bf16 bits [n_exp][N][G];
    rows_of_col(j) -> list of (projection index, row) for the 256 columns of tile j.
    Returns uint8 [n_exp][JT][G][BLOCK]."""
    n_exp, _, W = q[0].shape
    G = W // 8
    JT = len(rows_of_col.tiles)
    out = np.zeros((n_exp, JT, G, BLOCK), dtype=np.uint8)
    for j in range(JT):
        cols = rows_of_col(j)
        for c, (p, n) in enumerate(cols):
            words = q[p][:, n, :].reshape(n_exp, G, 8)           # [e][g][8 words]
            sw = (c >> 3) & 1
            for hh in range(2):
                src = words[:, :, 4 * (hh ^ sw):4 * (hh ^ sw) + 4]
                out[:, j, :, 32 * c + 16 * hh:32 * c + 16 * hh + 16] = \
                    src.astype("<u4").view(np.uint8).reshape(n_exp, G, 16)
            out[:, j, :, CODES + 2 * c:CODES + 2 * c + 2] = \
                s[p][:, n, :].astype("<u2").view(np.uint8).reshape(n_exp, G, 2)
            out[:, j, :, CODES + 512 + 2 * c:CODES + 512 + 2 * c + 2] = \
                b[p][:, n, :].astype("<u2").view(np.uint8).reshape(n_exp, G, 2)
    return out


class _Cols:
    def __init__(self, tiles, fn):
        self.tiles = tiles
        self.fn = fn

    def __call__(self, j):
        return self.fn(j)


@pytest.mark.parametrize("H,I", [(256, 128), (512, 256)])
def test_pack_matches_documented_layout(H, I):
    print(f"[pack] H={H} I={I}", flush=True)
    inp = make_layer(77, T=4, H=H, I=I)
    w = upload(inp, device())
    got = w.packed.cpu().numpy()
    E = inp.E

    def proj(name, shared):
        p = getattr(inp, name)
        q, s, b = p.q, p.scale, p.bias
        if shared:
            q, s, b = q[None], s[None], b[None]
        return q, s, b

    def gu_cols(j):   # column c: row 128 j + 32 (c // 64) + c % 32 of gate (c % 64 < 32) or up
        return [((c >> 5) & 1, 128 * j + 32 * (c >> 6) + (c & 31)) for c in range(256)]

    def dn_cols(j):
        return [(0, 256 * j + c) for c in range(256)]

    sections = []
    for shared in (False, True):
        g, u = proj("sh_gate" if shared else "gate", shared), proj("sh_up" if shared else "up", shared)
        sections.append(_blocks([g[0], u[0]], [g[1], u[1]], [g[2], u[2]],
                                _Cols(range(I // 128), gu_cols)))
    for shared in (False, True):
        d = proj("sh_down" if shared else "down", shared)
        sections.append(_blocks([d[0]], [d[1]], [d[2]], _Cols(range(H // 256), dn_cols)))
    off = 0
    for sec in sections:
        flat = sec.reshape(-1)
        np.testing.assert_array_equal(got[off:off + flat.size], flat)
        off = (off + flat.size + 255) // 256 * 256
    assert off == got.size == moe.moe_packed_bytes(moe.Shape(T=1, H=H, I=I, E=E))
