"""CPU pins of the oracle's target-side tree-verify attention (reading R14).

The oracle lists each query's visible keys explicitly.  These tests hold it to
a library routine over the full key range with a boolean mask (torch's CPU
scaled-dot-product attention in float64), to textbook causal attention on a
chain, and to relabelling invariance.
"""
import numpy as np
import pytest
import torch

from oracle import eagle_oracle as O


def _random_tree_mask(rng, m):
    """Ancestor-or-self mask of a random tree in flat order (parent before child)."""
    parent = [-1] + [int(rng.integers(0, i)) for i in range(1, m)]
    mask = np.zeros((m, m), dtype=np.uint8)
    for i in range(m):
        j = i
        while j >= 0:
            mask[i, j] = 1
            j = parent[j]
    return mask


def _sdpa_full(q, kc, vc, P, mask):
    """Library attention over rows 0..P+m-1 with a [m, P+m] boolean mask."""
    m, H, hd = q.shape
    Hkv = kc.shape[1]
    g = H // Hkv
    n = P + m
    vis = np.concatenate([np.ones((m, P), dtype=bool), mask.astype(bool)], axis=1)
    kt = torch.from_numpy(np.repeat(kc[:n], g, axis=1)).permute(1, 0, 2)  # [H, n, hd]
    vt = torch.from_numpy(np.repeat(vc[:n], g, axis=1)).permute(1, 0, 2)
    qt = torch.from_numpy(q).permute(1, 0, 2)  # [H, m, hd]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(vis))
    return o.permute(1, 0, 2).reshape(m, H * hd).numpy()


@pytest.mark.parametrize("H,Hkv,hd,P,m", [(2, 2, 8, 5, 6), (4, 2, 16, 17, 9), (6, 1, 8, 1, 12)])
def test_tree_verify_matches_library_masked_attention(H, Hkv, hd, P, m):
    rng = np.random.default_rng(H * 1000 + P * 10 + m)
    q = rng.normal(size=(m, H, hd))
    kc = rng.normal(size=(P + m + 3, Hkv, hd))  # rows past P+m are never visible
    vc = rng.normal(size=(P + m + 3, Hkv, hd))
    mask = _random_tree_mask(rng, m)
    out = O.tree_verify_attention(q, kc, vc, P, mask)
    assert np.allclose(out, _sdpa_full(q, kc, vc, P, mask), atol=1e-12)


def test_tree_verify_chain_is_causal_attention():
    """topk = 1: the tree is a chain, its mask lower-triangular, and tree
    verification is ordinary causal attention over the prefix plus the chain."""
    rng = np.random.default_rng(7)
    m, H, hd, P = 7, 2, 8, 4
    q = rng.normal(size=(m, H, hd))
    kc, vc = rng.normal(size=(P + m, H, hd)), rng.normal(size=(P + m, H, hd))
    chain = np.tril(np.ones((m, m), dtype=np.uint8))
    out = O.tree_verify_attention(q, kc, vc, P, chain)
    # causal over the full sequence: query i is row P+i and sees rows 0..P+i
    for i in range(m):
        for h in range(H):
            s = kc[: P + i + 1, h] @ q[i, h] / np.sqrt(hd)
            p = np.exp(s - s.max())
            p /= p.sum()
            assert np.allclose(out[i, h * hd:(h + 1) * hd], p @ vc[: P + i + 1, h], atol=1e-12)


def test_tree_verify_mask_selects_exactly_the_ancestors():
    """A node that sees only itself in the tree ignores every other tree row;
    changing a non-ancestor's key or value leaves a node's output unchanged."""
    rng = np.random.default_rng(11)
    m, H, hd, P = 6, 2, 4, 3
    q = rng.normal(size=(m, H, hd))
    kc, vc = rng.normal(size=(P + m, H, hd)), rng.normal(size=(P + m, H, hd))
    eye = np.eye(m, dtype=np.uint8)
    out = O.tree_verify_attention(q, kc, vc, P, eye)
    for i in range(m):
        rows = list(range(P)) + [P + i]
        assert np.allclose(out[i], O.attend_row(q[i], kc[rows], vc[rows]), atol=1e-12)
    mask = _random_tree_mask(rng, m)
    base = O.tree_verify_attention(q, kc, vc, P, mask)
    for j in range(m):
        kc2, vc2 = kc.copy(), vc.copy()
        kc2[P + j] += 5.0
        vc2[P + j] -= 3.0
        pert = O.tree_verify_attention(q, kc2, vc2, P, mask)
        for i in range(m):
            same = np.allclose(pert[i], base[i])
            assert same == (not mask[i, j]), (i, j)


def test_tree_verify_relabelling_invariance():
    """Renumbering the tree nodes (query rows, tree cache rows and both mask
    axes by one permutation) permutes the outputs and nothing else."""
    rng = np.random.default_rng(13)
    m, H, hd, P = 8, 4, 8, 5
    q = rng.normal(size=(m, H, hd))
    kc, vc = rng.normal(size=(P + m, 2, hd)), rng.normal(size=(P + m, 2, hd))
    mask = _random_tree_mask(rng, m)
    out = O.tree_verify_attention(q, kc, vc, P, mask)
    perm = rng.permutation(m)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[P:] = kc[P + perm]
    vc2[P:] = vc[P + perm]
    out2 = O.tree_verify_attention(q[perm], kc2, vc2, P, mask[np.ix_(perm, perm)])
    assert np.allclose(out2, out[perm], atol=1e-12)
