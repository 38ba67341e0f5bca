"""GPU test of eagle_verify_rejection_topk_noalloc (the variant for callers
that cannot allocate): through the C ABI, two calls in a row, the second on
a smaller input, each against eagle_verify_rejection_topk with a caller
scratch buffer on the same inputs (bit-identical: the same kernels)."""
from __future__ import annotations

import numpy as np
import pytest

try:
    import torch
    HAVE_GPU = torch.cuda.is_available()
except Exception:  # pragma: no cover
    HAVE_GPU = False

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not HAVE_GPU, reason="needs a GPU")]


def _tree(rng, B, m, D, V):
    tokens = np.zeros((B, m), dtype=np.int32)
    parents = np.zeros((B, m), dtype=np.int32)
    for b in range(B):
        par, dep = [-1], [0]
        for i in range(1, m):
            cand = [j for j in range(i) if dep[j] < D]
            pj = int(cand[int(rng.integers(0, len(cand)))])
            par.append(pj)
            dep.append(dep[pj] + 1)
        parents[b] = par
        tokens[b] = rng.integers(0, V, size=m)
    return tokens, parents


def _call(noalloc, B, m, D, V, T, tl, tokens, parents, u):
    from eagle_draft_trees_amd import _lib as L
    dev = "cuda:0"
    cfg = L.EagleTreeCfg(B, D, 16, m, 4 * m + 8)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    alen = torch.full((B,), -7, dtype=torch.int32, device=dev)
    apath = torch.full((B, D + 1), -7, dtype=torch.int32, device=dev)
    bonus = torch.full((B,), -7, dtype=torch.int32, device=dev)
    if noalloc:
        L.eagle_verify_rejection_topk_noalloc(cfg, V, t(tl), t(tokens), t(parents), T, t(u), alen, apath, bonus)
    else:
        scr = torch.empty(L.eagle_verify_relaxed_scratch_bytes(cfg), dtype=torch.uint8, device=dev)
        L.eagle_verify_rejection_topk(cfg, V, t(tl), t(tokens), t(parents), T, t(u), alen, apath, bonus, scr)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in (alen, apath, bonus)]


def test_noalloc_matches_scratch_variant_twice():
    from eagle_draft_trees_amd import _lib as L
    print("[no-alloc] rejection topk, two calls", flush=True)
    rng = np.random.default_rng(77)
    for B, m, D, V in ((6, 40, 6, 4000), (2, 9, 4, 700)):   # the second call is smaller
        tokens, parents = _tree(rng, B, m, D, V)
        tl = (rng.standard_normal((B, m, V)) * 3.0).astype(np.float32)
        for node in range(m):  # plant some acceptances
            for b in range(B):
                kids = [c for c in range(m) if parents[b][c] == node]
                if kids and rng.random() < 0.7:
                    tl[b, node, tokens[b, kids[0]]] += 20.0
        u = rng.random((B, m + 1)).astype(np.float32)
        want = _call(False, B, m, D, V, 1.0, tl, tokens, parents, u)
        got = _call(True, B, m, D, V, 1.0, tl, tokens, parents, u)
        for a, b in zip(want, got):
            assert np.array_equal(a, b), (B, m, a, b)
        print(f"  B={B} m={m}: accept lengths {[int(x) for x in got[0]]}", flush=True)
    # beyond the limit: a clear error, nothing launched
    cfg = L.EagleTreeCfg(L.EAGLE_NOALLOC_MAX_ROWS // 2 + 1, 2, 1, 2, 8)
    with pytest.raises(L.EagleError) as ei:
        L.eagle_verify_rejection_topk_noalloc(cfg, 10, 1 << 40, 1 << 40, 1 << 40, 1.0, 1 << 40, 1 << 40,
                                              1 << 40, 1 << 40)
    assert "no-allocation limit" in str(ei.value)
