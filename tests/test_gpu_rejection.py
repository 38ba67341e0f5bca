"""GPU parity of eagle_verify_rejection against the oracle's recursive
rejection sampling (R17).

Inputs are seeded here: random flat trees of bounded depth, target logits
N(0, 3^2), draft logits = target logits plus N(0, s^2) noise (so that q is
close to p and children are often accepted), children's tokens drawn from the
draft distribution at their parent, and random uniforms.  The kernel decides
in fp32 and the oracle in fp64; a sequence whose decisions all have margins
above 1e-5 (|u q(t) - p(t)| for every child tried, the draw's distance from
its CDF interval ends; p - q cancels but keeps fp32's relative error of about
1e-6, which renormalising by its mass preserves) must match exactly, closer
ones are checked for validity only.  Margins are relative (|u q - p| over the
larger side), so decisions between tiny probabilities at low temperatures
are compared like any other.
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


def _inputs(rng, B, m, D, V, T, noise):
    tokens = np.zeros((B, m), dtype=np.int64)
    parents = np.zeros((B, m), dtype=np.int64)
    tl = (rng.standard_normal((B, m, V)) * 3.0).astype(np.float32)
    dl = (tl + rng.standard_normal((B, m, V)) * noise).astype(np.float32)
    for b in range(B):
        par, dep = [-1], [0]
        for i in range(1, m):
            cand = [j for j in range(i) if dep[j] < D]
            pj = int(cand[int(rng.integers(0, len(cand)))])
            par.append(pj)
            dep.append(dep[pj] + 1)
        parents[b] = par
        tokens[b, 0] = int(rng.integers(0, V))
        for c in range(1, m):  # the child's token drawn from the draft at its parent
            q = O.target_probs(dl[b, par[c]].astype(np.float64), T)
            tokens[b, c] = int(rng.choice(V, p=q))
    u = rng.random((B, m + 1)).astype(np.float32)
    return tokens, parents, tl, dl, u


def _run(B, m, D, V, T, tokens, parents, tl, dl, u):
    from eagle_draft_trees_amd import _lib as L
    dev = "cuda:0"
    cfg = L.EagleTreeCfg(B, D, 16, m, 4 * m + 8)
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).astype(dt)).to(dev)
    alen = torch.full((B,), -7, dtype=torch.int32, device=dev)
    apath = torch.full((B, D + 1), -7, dtype=torch.int32, device=dev)
    bonus = torch.full((B,), -7, dtype=torch.int32, device=dev)
    scr = torch.empty(L.eagle_verify_rejection_scratch_bytes(cfg, V), dtype=torch.uint8, device=dev)
    L.eagle_verify_rejection(cfg, V, t(tl, np.float32), t(dl, np.float32), t(tokens, np.int32),
                             t(parents, np.int32), T, t(u, np.float32), alen, apath, bonus, scr)
    torch.cuda.synchronize()
    return alen.cpu().numpy(), apath.cpu().numpy(), bonus.cpu().numpy()


def _check(name, B, m, D, V, T, tokens, parents, tl, dl, u, g):
    galen, gpath, gbonus = g
    exact = near = 0
    lens = []
    for b in range(B):
        path, alen, bonus, margins = O.verify_rejection(tl[b].astype(np.float64), dl[b].astype(np.float64),
                                                        tokens[b], parents[b], T, u[b].astype(np.float64))
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
    print(f"  rejection {name}: accept lengths {lens}, exact {exact}, near-tie {near}", flush=True)
    assert exact >= 1


CASES = [  # name, B, m, D, V, T, draft noise
    ("small", 4, 9, 4, 1003, 1.0, 0.3),
    ("wide", 2, 64, 6, 2048, 0.7, 0.5),
    ("hot", 4, 12, 5, 515, 2.0, 1.0),
    ("7b_shape", 2, 60, 6, 32000, 1.0, 0.3),
    ("far_draft", 3, 10, 4, 777, 1.0, 3.0),
    # a low temperature: q and p underflow to 0 for most tokens in fp32, and a
    # child without target mass must still be rejected
    ("cold", 4, 12, 5, 2048, 0.02, 0.3),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_rejection_matches_oracle(case):
    name, B, m, D, V, T, noise = case
    print(f"[rejection] {name}", flush=True)
    rng = np.random.default_rng([m, D, V, B, 5])
    tokens, parents, tl, dl, u = _inputs(rng, B, m, D, V, T, noise)
    g = _run(B, m, D, V, T, tokens, parents, tl, dl, u)
    _check(name, B, m, D, V, T, tokens, parents, tl, dl, u, g)


def test_rejection_edge_cases():
    """Draft equal to the target (every first child accepted), a draft with no
    mass where the target has any (everything rejected, the bonus from p),
    uniforms at and past the ends of [0, 1), and a two-node tree."""
    print("[rejection] edge cases", flush=True)
    rng = np.random.default_rng(41)
    B, m, D, V = 3, 8, 4, 200
    tokens, parents, tl, dl, u = _inputs(rng, B, m, D, V, 1.0, 0.0)
    g = _run(B, m, D, V, 1.0, tokens, parents, tl, tl.copy(), u)
    _check("q = p", B, m, D, V, 1.0, tokens, parents, tl, tl.copy(), u, g)
    first = [0]
    while True:
        kids = [c for c in range(m) if parents[0][c] == first[-1]]
        if not kids:
            break
        first.append(kids[0])
    assert g[0][0] == len(first)
    # disjoint supports: q on ids < 100 only, p on ids >= 100 only
    tl2, dl2 = tl.copy(), tl.copy()
    tl2[:, :, :100] = -np.inf
    dl2[:, :, 100:] = -np.inf
    tok2 = tokens.copy() % 100
    for uu in ([0.3] * (m + 1), [0.999999] * (m + 1), [1.5] * (m + 1)):
        u2 = np.tile(np.array(uu, dtype=np.float32), (B, 1))
        g = _run(B, m, D, V, 1.0, tok2, parents, tl2, dl2, u2)
        uc = np.clip(u2, 0.0, np.float32(0.99999994))
        _check("disjoint", B, m, D, V, 1.0, tok2, parents, tl2, dl2, uc, g)
        assert np.all(g[0] == 1) and np.all(g[2] >= 100)
    t3, p3 = np.array([[5, 9]]), np.array([[-1, 0]])
    l3 = rng.standard_normal((1, 2, 50)).astype(np.float32)
    for uu in (0.0, 0.97):
        u3 = np.array([[0.2, uu, 0.4]], dtype=np.float32)
        g = _run(1, 2, 2, 50, 0.5, t3, p3, l3, l3 * 0.5, u3)
        _check(f"two-node u={uu}", 1, 2, 2, 50, 0.5, t3, p3, l3, l3 * 0.5, u3, g)
