"""moe_pack_weights against a numpy rendering of the tile layout that
include/moe_q4.h documents: every byte of the blocks is checked (each code word's even
codes in its low nibbles and odd codes in its high nibbles, each row's scales and biases
times its power of two 2^k), and the meta section's status, column factors and
per-expert row-norm bounds."""
import numpy as np
import pytest

import bit_quantized_expert_top_amd as moe
from moe_case import device, upload
from synth import bf16_bits_to_f32, f32_to_bf16_bits, make_layer

pytestmark = pytest.mark.gpu

BLOCK, CODES = 9216, 8192


def _row_shift(s_bits):
    """k per row: the power of two that puts the row's largest |scale| in [2^10, 2^11)."""
    sf = np.abs(bf16_bits_to_f32(s_bits)).astype(np.float64)
    smax = sf.max(axis=-1)
    _, e = np.frexp(smax)                    # smax = m 2^e, m in [0.5, 1)
    return np.where(smax > 0, 10 - (e - 1), 0)


def _shifted(bits, k):
    """bf16 values times 2^k (exact), as bf16 bits."""
    return f32_to_bf16_bits(np.ldexp(bf16_bits_to_f32(bits).astype(np.float64), k[..., None])
                            .astype(np.float32))


def _unzip(words):
    """Checkpoint code words -> tile-layout words: code 2m to nibble m, code 2m+1 to
    nibble m + 4 (m = 0..3)."""
    w = words.astype(np.uint64)
    r = np.zeros_like(w)
    for m in range(4):
        r |= ((w >> (8 * m)) & 0xF) << (4 * m)
        r |= ((w >> (8 * m + 4)) & 0xF) << (4 * m + 16)
    return r.astype(np.uint32)


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
            words = _unzip(q[p][:, n, :]).reshape(n_exp, G, 8)   # [e][g][8 words]
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

    def shifted(p):
        q, s_, b_ = p
        k = _row_shift(s_)
        return q, _shifted(s_, k), _shifted(b_, k), k

    sections, colk = [], []
    for shared in (False, True):
        g = shifted(proj("sh_gate" if shared else "gate", shared))
        u = shifted(proj("sh_up" if shared else "up", shared))
        sections.append(_blocks([g[0], u[0]], [g[1], u[1]], [g[2], u[2]],
                                _Cols(range(I // 128), gu_cols)))
        # column factors 2^-k in the blocks' column order: [n_exp][tile][256]
        colk.append(np.stack([np.ldexp(1.0, -np.array([(g[3], u[3])[p][:, n] for p, n in gu_cols(j)]).T)
                              for j in range(I // 128)], axis=1))
    for shared in (False, True):
        d = shifted(proj("sh_down" if shared else "down", shared))
        sections.append(_blocks([d[0]], [d[1]], [d[2]], _Cols(range(H // 256), dn_cols)))
        colk.append(np.stack([np.ldexp(1.0, -d[3][:, 256 * j:256 * j + 256])
                              for j in range(H // 256)], axis=1))
    off = 0
    for sec in sections:
        flat = sec.reshape(-1)
        np.testing.assert_array_equal(got[off:off + flat.size], flat)
        off = (off + flat.size + 255) // 256 * 256
    # meta: status line, per-expert bounds, then the column factors of the four sections
    assert got[off:off + 4].view(np.int32)[0] == 0 and w.status == 0
    off += 256
    emeta = got[off:off + 257 * 16].view(np.float32).reshape(257, 4)
    off = (off + 257 * 16 + 255) // 256 * 256
    for ck in colk:
        # per tile: 2^-k of the 256 columns, a flags word, padding
        n = ck.shape[0] * ck.shape[1] * 260 * 4
        cf = got[off:off + n].view(np.float32).reshape(ck.shape[0], ck.shape[1], 260)
        np.testing.assert_array_equal(cf[:, :, :256], ck.astype(np.float32))
        assert np.all(cf[:, :, 256:].view(np.int32) == 0)       # b = -8 s: no rank-G term
        off = (off + n + 255) // 256 * 256
    assert off == got.size == moe.moe_packed_bytes(moe.Shape(T=1, H=H, I=I, E=E))
    # the bound on the L2 norm of every gate and up row of each expert slot
    import oracle
    for e in list(range(0, E, 37)) + [E]:
        names = ("sh_gate", "sh_up") if e == E else ("gate", "up")
        norms = []
        for nm in names:
            p = getattr(inp, nm)
            q, s_, b_ = (p.q, p.scale, p.bias) if e == E else (p.q[e], p.scale[e], p.bias[e])
            wd = oracle.dequant(q, s_, b_, I, H)
            norms.append(np.sqrt((wd ** 2).sum(axis=1)).max())
        nb = max(norms)
        assert nb <= emeta[e, 0] <= nb * 1.002, (e, nb, emeta[e, 0])
