"""GPU test of eagle_pack_weights: the packed buffer must equal, byte for
byte, the tile layout documented in include/eagle_mi355x.h, built here with
numpy indexing from the row-major matrices (ragged rows and ragged K, both
dtypes, the q/k/v rotation-pair row grouping, zero padding)."""
from __future__ import annotations

import numpy as np
import pytest

try:
    import torch
    HAVE_GPU = torch.cuda.is_available()
except Exception:  # pragma: no cover
    HAVE_GPU = False

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not HAVE_GPU, reason="needs a GPU")]


def _expected(w: np.ndarray, ks: int, pair_hd: int) -> np.ndarray:
    """Packed bytes of row-major w [N][K] (uint16 or uint32 element bits)."""
    N, K = w.shape
    per = 16 // w.itemsize
    ntile, nks = -(-N // 16), -(-K // ks)
    wp = np.zeros((ntile * 16 + 1, nks * ks), dtype=w.dtype)  # the last row stays zero
    wp[:N, :K] = w
    t = np.arange(ntile)[:, None]
    c = np.arange(16)[None, :]
    if pair_hd:
        tph = pair_hd // 16
        head, j = t // tph, t % tph
        rows = head * pair_hd + np.where(c < 8, 8 * j + c, pair_hd // 2 + 8 * j + (c - 8))
    else:
        rows = 16 * t + c
    rows = np.where(rows < N, rows, ntile * 16)               # rows past N: the zero row
    blk = wp[rows]                                            # [ntile][16][Kp]
    blk = blk.reshape(ntile, 16, nks, ks // per, per)         # [t][c][s][g][e]
    return np.ascontiguousarray(blk.transpose(0, 2, 3, 1, 4)).view(np.uint8).ravel()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pack_layout_is_the_documented_tiles(dtype):
    from eagle_draft_trees_amd import _lib as L
    d, H, Hkv, hd, F, V = 192, 3, 1, 64, 408, 1003
    es = 2 if dtype == "bf16" else 4
    ks = 32 if es == 2 else 16
    dims = L.EagleDims(d, H, Hkv, hd, F, V, L.EAGLE_BF16 if es == 2 else L.EAGLE_F32, 1e-6, 1e4)
    rng = np.random.default_rng(7)
    et = np.uint16 if es == 2 else np.uint32
    shapes = {"fc_w": (d, 2 * d), "wq": (H * hd, d), "wk": (Hkv * hd, d), "wv": (Hkv * hd, d),
              "wo": (d, H * hd), "w_gate": (F, d), "w_up": (F, d), "w_down": (d, F), "lm_head": (V, d),
              "fc_b": (d,), "post_norm": (d,), "embed": (V, d)}
    host = {n: rng.integers(0, np.iinfo(et).max, size=s, dtype=et) for n, s in shapes.items()}
    tdt = torch.int16 if es == 2 else torch.int32
    dev = {n: torch.from_numpy(a.view(np.int16 if es == 2 else np.int32)).to("cuda") for n, a in host.items()}
    assert all(t.dtype == tdt for t in dev.values())
    src = L.make_weights(dev)
    nbytes = L.eagle_packed_weights_bytes(dims)
    dst = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device="cuda")
    out = L.eagle_pack_weights(dims, src, dst)
    torch.cuda.synchronize()
    assert out.packed == L.EAGLE_PACKED_WEIGHTS
    got = dst.cpu().numpy()
    base = dst.data_ptr()
    off = 0
    for n in ("fc_w", "wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "lm_head"):
        w = host[n][:, :d] if n == "fc_w" else host[n]   # only the FC's feature half is packed
        exp = _expected(np.ascontiguousarray(w), ks, hd if n in ("wq", "wk", "wv") else 0)
        assert getattr(out, n) == base + off, n
        np.testing.assert_array_equal(got[off:off + exp.size], exp, err_msg=n)
        off += -(-exp.size // 256) * 256
    assert out.tok_proj == base + off      # then the fp32 token-projection table [V][d]
    off += -(-(V * d * 4) // 256) * 256
    assert off == nbytes
    for n in ("fc_b", "post_norm", "embed"):
        assert getattr(out, n) == dev[n].data_ptr()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_token_projection_table(dtype):
    # tok_proj[v] = fc_w[:, d:2d] @ embed[v]: the token half of the FC per vocabulary
    # entry, fp32 sums of the exact products; checked against the fp64 product
    # within the fp32 summation bound (K terms: K * 2^-24 of the sum of |products|)
    import synth
    from eagle_draft_trees_amd import _lib as L
    d, H, Hkv, hd, F, V = 256, 4, 2, 64, 64, 1003
    es = 2 if dtype == "bf16" else 4
    dims = L.EagleDims(d, H, Hkv, hd, F, V, L.EAGLE_BF16 if es == 2 else L.EAGLE_F32, 1e-6, 1e4)
    rng = np.random.default_rng(8)
    shapes = {"fc_w": (d, 2 * d), "wq": (H * hd, d), "wk": (Hkv * hd, d), "wv": (Hkv * hd, d),
              "wo": (d, H * hd), "w_gate": (F, d), "w_up": (F, d), "w_down": (d, F), "lm_head": (V, d),
              "fc_b": (d,), "post_norm": (d,), "embed": (V, d)}
    f32 = {n: rng.normal(0, 1, s).astype(np.float32) for n, s in shapes.items()}
    if es == 2:
        bits = {n: synth.bf16_bits(a) for n, a in f32.items()}
        val = {n: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64) for n, b in bits.items()}
        dev = {n: torch.from_numpy(b.view(np.int16)).to("cuda") for n, b in bits.items()}
    else:
        val = {n: a.astype(np.float64) for n, a in f32.items()}
        dev = {n: torch.from_numpy(a).to("cuda") for n, a in f32.items()}
    dst = torch.empty(L.eagle_packed_weights_bytes(dims), dtype=torch.uint8, device="cuda")
    out = L.eagle_pack_weights(dims, L.make_weights(dev), dst)
    torch.cuda.synchronize()
    off = out.tok_proj - dst.data_ptr()
    got = dst[off:off + V * d * 4].view(torch.float32).view(V, d).double().cpu().numpy()
    w2 = val["fc_w"][:, d:]
    exp = val["embed"] @ w2.T
    bound = d * 2.0 ** -24 * (np.abs(val["embed"]) @ np.abs(w2).T) + 1e-30
    assert np.all(np.abs(got - exp) <= bound), float(np.max(np.abs(got - exp) / bound))
