"""GPU parity of eagle_verify_rejection_topk against the oracle's rejection
sampling of deterministic candidates (R18).

Inputs are seeded here: random flat trees of bounded depth, target logits
N(0, 3^2), each node's children carrying the top tokens (distinct, in rank
order) of a draft row = target row + N(0, s^2) noise, as EAGLE-2's top-k
children do, and random uniforms.  The kernel decides in fp32 and the oracle
in fp64; a sequence whose decisions all have relative margins above 1e-5
(|u * left - p(t)| over the larger side for every child tried, the draw's
distance from its CDF interval ends) must match exactly, closer ones are
checked for validity only.
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


def _inputs(rng, B, m, D, V, noise):
    tokens = np.zeros((B, m), dtype=np.int64)
    parents = np.zeros((B, m), dtype=np.int64)
    tl = (rng.standard_normal((B, m, V)) * 3.0).astype(np.float32)
    for b in range(B):
        par, dep = [-1], [0]
        for i in range(1, m):
            cand = [j for j in range(i) if dep[j] < D]
            pj = int(cand[int(rng.integers(0, len(cand)))])
            par.append(pj)
            dep.append(dep[pj] + 1)
        parents[b] = par
        tokens[b, 0] = int(rng.integers(0, V))
        for node in range(m):
            kids = [c for c in range(1, m) if par[c] == node]
            if kids:
                draft = tl[b, node] + rng.standard_normal(V).astype(np.float32) * noise
                top = np.argsort(-draft, kind="stable")[:len(kids)]
                for c, t in zip(kids, top):
                    tokens[b, c] = int(t)
    u = rng.random((B, m + 1)).astype(np.float32)
    return tokens, parents, tl, u


def _run(B, m, D, V, T, tokens, parents, tl, u):
    from eagle_draft_trees_amd import _lib as L
    dev = "cuda:0"
    cfg = L.EagleTreeCfg(B, D, 16, m, 4 * m + 8)
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).astype(dt)).to(dev)
    alen = torch.full((B,), -7, dtype=torch.int32, device=dev)
    apath = torch.full((B, D + 1), -7, dtype=torch.int32, device=dev)
    bonus = torch.full((B,), -7, dtype=torch.int32, device=dev)
    scr = torch.empty(L.eagle_verify_relaxed_scratch_bytes(cfg), dtype=torch.uint8, device=dev)
    L.eagle_verify_rejection_topk(cfg, V, t(tl, np.float32), t(tokens, np.int32), t(parents, np.int32), T,
                                  t(u, np.float32), alen, apath, bonus, scr)
    torch.cuda.synchronize()
    return alen.cpu().numpy(), apath.cpu().numpy(), bonus.cpu().numpy()


def _check(name, B, m, D, V, T, tokens, parents, tl, u, g):
    galen, gpath, gbonus = g
    exact = near = 0
    lens = []
    for b in range(B):
        path, alen, bonus, margins = O.verify_rejection_topk(tl[b].astype(np.float64), tokens[b], parents[b], T,
                                                             u[b].astype(np.float64))
        lens.append(alen)
        gp = [int(x) for x in gpath[b][:galen[b]]]
        if min(margins) > MARGIN:
            exact += 1
            assert galen[b] == alen and gp == path and gbonus[b] == bonus, (name, b, gp, path, gbonus[b], bonus)
            assert all(int(x) == -1 for x in gpath[b][alen:])
        else:
            near += 1
            assert 1 <= galen[b] <= D + 1 and gp[0] == 0 and 0 <= gbonus[b] < V
            assert all(parents[b][gp[i + 1]] == gp[i] for i in range(len(gp) - 1))
    print(f"  rejection topk {name}: accept lengths {lens}, exact {exact}, near-tie {near}", flush=True)
    assert exact >= 1


CASES = [  # name, B, m, D, V, T, draft noise
    ("small", 4, 9, 4, 1003, 1.0, 0.3),
    ("wide", 2, 64, 6, 2048, 0.7, 0.5),
    ("hot", 4, 12, 5, 515, 2.0, 1.0),
    ("7b_shape", 2, 60, 6, 32000, 1.0, 0.3),
    ("cold", 4, 12, 5, 2048, 0.05, 0.3),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_rejection_topk_matches_oracle(case):
    name, B, m, D, V, T, noise = case
    print(f"[rejection topk] {name}", flush=True)
    rng = np.random.default_rng([m, D, V, B, 9])
    tokens, parents, tl, u = _inputs(rng, B, m, D, V, noise)
    g = _run(B, m, D, V, T, tokens, parents, tl, u)
    _check(name, B, m, D, V, T, tokens, parents, tl, u, g)


def test_rejection_topk_edge_cases():
    """Siblings carrying the same token (the copy is never accepted), -inf
    logits on the children's tokens, uniforms at and past the ends of [0, 1),
    and a two-node tree."""
    print("[rejection topk] edge cases", flush=True)
    rng = np.random.default_rng(43)
    B, m, D, V = 3, 8, 4, 300
    tokens, parents, tl, u = _inputs(rng, B, m, D, V, 0.3)
    for b in range(B):  # duplicate the first child's token into its next sibling
        kids = [c for c in range(m) if parents[b][c] == 0]
        if len(kids) >= 2:
            tokens[b, kids[1]] = tokens[b, kids[0]]
    u2 = u.copy()
    u2[:, :] = 0.999
    g = _run(B, m, D, V, 1.0, tokens, parents, tl, u2)
    _check("duplicates", B, m, D, V, 1.0, tokens, parents, tl, u2, g)
    tl3 = tl.copy()
    for b in range(B):
        for c in range(1, m):
            tl3[b, parents[b][c], tokens[b, c]] = -np.inf
    for uu in (0.0, 0.5, 1.5):
        u3 = np.full((B, m + 1), uu, dtype=np.float32)
        g = _run(B, m, D, V, 1.0, tokens, parents, tl3, u3)
        uc = np.clip(u3, 0.0, np.float32(0.99999994))
        _check(f"no mass u={uu}", B, m, D, V, 1.0, tokens, parents, tl3, uc, g)
        assert np.all(g[0] == 1)
    t4, p4 = np.array([[5, 9]]), np.array([[-1, 0]])
    l4 = rng.standard_normal((1, 2, 50)).astype(np.float32)
    for uu in (0.0, 0.97):
        u4 = np.array([[0.2, uu, 0.4]], dtype=np.float32)
        g = _run(1, 2, 2, 50, 0.5, t4, p4, l4, u4)
        _check(f"two-node u={uu}", 1, 2, 2, 50, 0.5, t4, p4, l4, u4, g)
