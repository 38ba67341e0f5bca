"""GPU parity of eagle_verify_relaxed against the oracle's relaxed walk (R15).

Inputs are seeded here: random flat trees of bounded depth with distinct
sibling tokens, target logits N(0, 3^2) with planted children whose target
probability sits well above or below the threshold (so most walks go several
levels deep), and one uniform per sequence.  The kernel decides in fp32 and
the oracle in fp64; a sequence whose decisions all have margins above 1e-5
(|p(c) - threshold| for every child tried, and the draw's distance from its
CDF interval ends) must match exactly: path, accept_len and bonus.  Closer
sequences are reported as near-ties and checked for validity only.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import eagle_oracle as O

try:
    import torch
    HAVE_GPU = torch.cuda.is_available()
except Exception:  # pragma: no cover
    HAVE_GPU = False

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not HAVE_GPU, reason="needs a GPU")]

MARGIN = 1e-5


def say(msg):
    print(msg, flush=True)


def _tree(rng, m, D, V, root_kids=None):
    """Flat tree, parent before child, depth <= D, distinct sibling tokens."""
    parents, depth = [-1], [0]
    for i in range(1, m):
        if root_kids is not None and i <= root_kids:
            par = 0
        else:
            cand = [j for j in range(i) if depth[j] < D]
            par = int(cand[int(rng.integers(0, len(cand)))])
        parents.append(par)
        depth.append(depth[par] + 1)
    tokens = np.zeros(m, dtype=np.int64)
    tokens[0] = int(rng.integers(0, V))
    for x in range(m):
        kids = [c for c in range(m) if parents[c] == x]
        for c, t in zip(kids, rng.choice(V, size=len(kids), replace=False)):
            tokens[c] = int(t)
    return tokens, np.array(parents, dtype=np.int64)


def _plant(rng, logits, tokens, parents, T, thr):
    """Along a random walk, give one child of each node a target probability
    drawn from [thr/3, thr*0.7] or [thr*1.4, 0.97] (fp64, then fp32 logits)."""
    m, V = logits.shape
    node = 0
    for _ in range(m):
        kids = [c for c in range(m) if parents[c] == node]
        if not kids:
            return
        c = kids[int(rng.integers(0, len(kids)))]
        hi = rng.random() < 0.75
        rho = rng.uniform(thr * 1.4, 0.97) if hi and thr * 1.4 < 0.97 else rng.uniform(thr / 3, thr * 0.7)
        row = logits[node].astype(np.float64) / T
        t = int(tokens[c])
        others = np.delete(row, t)
        mx = others.max()
        s_rest = np.exp(others - mx).sum()
        logits[node, t] = np.float32(T * (mx + np.log(rho * s_rest / (1.0 - rho))))
        if not hi:
            return
        node = c


CASES = [  # name, B, m, D, V, T, threshold
    ("small_f", 3, 9, 4, 1003, 1.0, 0.2),
    ("wide", 2, 64, 6, 2048, 0.7, 0.1),
    ("hot", 4, 12, 5, 515, 2.0, 0.05),
    ("7b_shape", 1, 60, 6, 32000, 1.0, 0.15),
    ("large_vocab", 2, 8, 7, 128256, 1.0, 0.3),
]


def _run(B, m, D, V, T, thr, tokens, parents, logits, u):
    from eagle_draft_trees_amd import _lib as L
    dev = "cuda:0"
    cfg = L.EagleTreeCfg(B, D, 16, m, 4 * m + 8)
    tl = torch.from_numpy(logits).to(dev)
    tk = torch.from_numpy(tokens.astype(np.int32)).to(dev)
    pa = torch.from_numpy(parents.astype(np.int32)).to(dev)
    un = torch.from_numpy(u.astype(np.float32)).to(dev)
    alen = torch.full((B,), -7, dtype=torch.int32, device=dev)
    apath = torch.full((B, D + 1), -7, dtype=torch.int32, device=dev)
    bonus = torch.full((B,), -7, dtype=torch.int32, device=dev)
    scr = torch.empty(L.eagle_verify_relaxed_scratch_bytes(cfg), dtype=torch.uint8, device=dev)
    L.eagle_verify_relaxed(cfg, V, tl, tk, pa, T, thr, un, alen, apath, bonus, scr)
    torch.cuda.synchronize()
    return alen.cpu().numpy(), apath.cpu().numpy(), bonus.cpu().numpy()


def _check(name, B, m, D, V, T, thr, tokens, parents, logits, u, g):
    galen, gpath, gbonus = g
    exact = near = 0
    lens = []
    for b in range(B):
        path, alen, bonus, margins = O.verify_relaxed(logits[b].astype(np.float64), tokens[b],
                                                      parents[b], T, thr, float(u[b]))
        lens.append(alen)
        gp = [int(x) for x in gpath[b][:galen[b]]]
        if thr <= 0.0:  # every child passes whatever its probability: only the draw can flip
            margins = margins[-1:]
        if min(margins) > MARGIN:
            exact += 1
            assert galen[b] == alen and gp == path and gbonus[b] == bonus, (name, b, gp, path, gbonus[b], bonus)
            assert all(int(x) == -1 for x in gpath[b][alen:])
        else:
            near += 1
            assert 1 <= galen[b] <= D + 1 and gp[0] == 0 and 0 <= gbonus[b] < V
            assert all(parents[b][gp[i + 1]] == gp[i] for i in range(len(gp) - 1))
    say(f"  relaxed {name}: accept lengths {lens}, exact {exact}, near-tie {near}")
    assert exact >= 1


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_relaxed_matches_oracle(case):
    name, B, m, D, V, T, thr = case
    say(f"[relaxed] {name}")
    rng = np.random.default_rng([m, D, V, B])
    tokens = np.zeros((B, m), dtype=np.int64)
    parents = np.zeros((B, m), dtype=np.int64)
    logits = (rng.standard_normal((B, m, V)) * 3.0).astype(np.float32)
    for b in range(B):
        tokens[b], parents[b] = _tree(rng, m, D, V)
        _plant(rng, logits[b], tokens[b], parents[b], T, thr)
    u = rng.random(B).astype(np.float32)
    g = _run(B, m, D, V, T, thr, tokens, parents, logits, u)
    _check(name, B, m, D, V, T, thr, tokens, parents, logits, u, g)


def test_relaxed_edge_cases():
    """Threshold 0 (every first child), threshold above 1 (the root residual),
    a root whose children hold all the mass (the draw falls back to p),
    uniforms at and past the ends of [0, 1), -inf logits, and a two-node tree."""
    say("[relaxed] edge cases")
    rng = np.random.default_rng(77)
    B, m, D, V = 6, 10, 4, 300
    tokens = np.zeros((B, m), dtype=np.int64)
    parents = np.zeros((B, m), dtype=np.int64)
    for b in range(B):
        tokens[b], parents[b] = _tree(rng, m, D, V)
    logits = (rng.standard_normal((B, m, V)) * 2.0).astype(np.float32)
    logits[3, :, 100:] = -np.inf  # only ids < 100 carry mass at any node of sequence 3
    u = np.array([0.0, 0.999999, 1.5, 0.3, -0.2, 0.61], dtype=np.float32)
    for thr in (0.0, -1.0, 1.5, 0.02):
        g = _run(B, m, D, V, 1.0, thr, tokens, parents, logits, u)
        uc = np.clip(np.nan_to_num(u), 0.0, np.float32(0.99999994))
        _check(f"thr={thr}", B, m, D, V, 1.0, thr, tokens, parents, logits, uc, g)
        if thr >= 1.5:
            assert np.all(g[0] == 1)
        if thr <= 0:
            assert np.all(g[0] >= 2)
    # V = 4 and a root with 4 children: the residual is empty, the draw is from p
    m2, V2 = 6, 4
    t2 = np.array([[0, 0, 1, 2, 3, 1]], dtype=np.int64)
    p2 = np.array([[-1, 0, 0, 0, 0, 1]], dtype=np.int64)
    l2 = np.log(np.array([[[0.1, 0.2, 0.3, 0.4]] * m2], dtype=np.float64)).astype(np.float32)
    for uu in (0.05, 0.25, 0.55, 0.95):
        g = _run(1, m2, 3, V2, 1.0, 0.9, t2, p2, l2, np.array([uu], np.float32))
        _check(f"all-children u={uu}", 1, m2, 3, V2, 1.0, 0.9, t2, p2, l2, np.array([uu], np.float32), g)
    # siblings carrying the same token (not a rerank output, but accepted by
    # the ABI): the token is removed from the residual once
    t4 = np.array([[3, 7, 7, 9, 7]], dtype=np.int64)
    p4 = np.array([[-1, 0, 0, 0, 1]], dtype=np.int64)
    l4 = (rng.standard_normal((1, 5, 40)) * 0.3).astype(np.float32)
    for uu in (0.1, 0.45, 0.8):
        g = _run(1, 5, 3, 40, 1.0, 0.9, t4, p4, l4, np.array([uu], np.float32))
        _check(f"duplicate siblings u={uu}", 1, 5, 3, 40, 1.0, 0.9, t4, p4, l4, np.array([uu], np.float32), g)
        assert g[2][0] not in (7, 9)
    # two nodes: root and one child
    t3 = np.array([[5, 9]], dtype=np.int64)
    p3 = np.array([[-1, 0]], dtype=np.int64)
    l3 = (rng.standard_normal((1, 2, 50))).astype(np.float32)
    for thr in (0.0, 0.9):
        g = _run(1, 2, 2, 50, 0.5, thr, t3, p3, l3, np.array([0.4], np.float32))
        _check(f"two-node thr={thr}", 1, 2, 2, 50, 0.5, thr, t3, p3, l3, np.array([0.4], np.float32), g)
