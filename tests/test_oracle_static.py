"""CPU pins of the oracle's static-tree variant (reading R16).

The static tail is held to the dynamic tail when the template is the dynamic
selection, the static tree to the dynamic tree on a chain (topk 1), and the
built tree to brute-force structure: every node is the template's child of
its parent, scores are path sums of draft log-probabilities, the mask is the
ancestor-or-self relation, parents precede children and a truncated tree is
ancestor-closed.
"""
import numpy as np
import pytest

from oracle import eagle_oracle as O
from tests._tiny import seq_state, tensors, tiny_cfg


def _model(cfg, seed):
    rng = np.random.default_rng(seed)
    return O.Model(cfg, tensors(cfg, rng, scale=0.4)), seq_state(cfg, rng)


def _template(rng, k):
    """k distinct (parent slot, child rank) pairs."""
    pairs = rng.choice(k * k, size=k, replace=False)
    return [int(p) // k for p in pairs], [int(p) % k for p in pairs]


def _static_levels(model, st, D, k, templates):
    pool, F, _ = O.level_one(model, st, k)
    frontiers, feats, intree = [F], {}, {}
    for level in range(2, D + 1):
        h = O.level_step_forward(model, st, level, F, feats, intree)
        par, rk = templates[level]
        F, _ = O.level_step_tail_static(model, level, F, h, pool, k, par, rk)
        frontiers.append(F)
    return pool, frontiers


@pytest.mark.parametrize("D,k", [(3, 2), (4, 3), (2, 5)])
def test_static_tail_with_the_dynamic_selection_is_the_dynamic_tail(D, k):
    """Take the template from what the dynamic tail selected at each level:
    the static tail then yields the same frontiers and the same pool."""
    cfg = tiny_cfg(D=D, k=k, m=1 + D * k)
    model, st = _model(cfg, 10 * D + k)
    pool_d, F, _ = O.level_one(model, st, k)
    pool_s = list(pool_d)
    Fd, Fs = F, F
    feats_d, intree_d, feats_s, intree_s = {}, {}, {}, {}
    for level in range(2, D + 1):
        hd = O.level_step_forward(model, st, level, Fd, feats_d, intree_d)
        base = len(pool_d)
        Fd2, _, _ = O.level_step_tail(model, level, Fd, hd, pool_d, k)
        par = [x.pslot for x in Fd2]
        rk = [(x.pool_idx - base) % k for x in Fd2]
        hs = O.level_step_forward(model, st, level, Fs, feats_s, intree_s)
        Fs2, _ = O.level_step_tail_static(model, level, Fs, hs, pool_s, k, par, rk)
        assert [(x.token, x.pool_idx, x.pslot, x.anc) for x in Fs2] == \
               [(x.token, x.pool_idx, x.pslot, x.anc) for x in Fd2]
        assert np.allclose([x.score for x in Fs2], [x.score for x in Fd2], atol=0, rtol=0)
        Fd, Fs = Fd2, Fs2
    assert [(e.token, e.parent, e.depth, e.pslot) for e in pool_s] == \
           [(e.token, e.parent, e.depth, e.pslot) for e in pool_d]


@pytest.mark.parametrize("D", [2, 4])
def test_static_chain_equals_dynamic_chain(D):
    """topk 1: the only template is (slot 0, rank 0) and both trees are the
    chain of the draft's top token at each depth."""
    cfg = tiny_cfg(D=D, k=1, m=D + 1)
    model, st = _model(cfg, 3 + D)
    pool_d, Fd = O.level_one(model, st, 1)[:2]
    feats, intree, frontiers_d = {}, {}, [Fd]
    for level in range(2, D + 1):
        h = O.level_step_forward(model, st, level, Fd, feats, intree)
        Fd, _, _ = O.level_step_tail(model, level, Fd, h, pool_d, 1)
        frontiers_d.append(Fd)
    dyn = O.build_tree(pool_d, O.rerank(pool_d, D + 1)[0], st.root_token, st.P)
    _, frontiers_s = _static_levels(model, st, D, 1, {L: ([0], [0]) for L in range(2, D + 1)})
    stat = O.build_static_tree(frontiers_s, st.root_token, st.P, D + 1)
    for f in ("tokens", "parents", "depth", "positions", "mask"):
        assert np.array_equal(getattr(stat, f), getattr(dyn, f)), f
    assert np.allclose(stat.logscore, dyn.logscore, atol=1e-12)


@pytest.mark.parametrize("D,k,m", [(3, 2, 7), (4, 3, 13), (4, 3, 8), (3, 4, 2)])
def test_static_tree_structure(D, k, m):
    cfg = tiny_cfg(D=D, k=k, m=m)
    model, st = _model(cfg, 100 + D * 10 + k)
    rng = np.random.default_rng(7 * D + k)
    templates = {L: _template(rng, k) for L in range(2, D + 1)}
    pool, frontiers = _static_levels(model, st, D, k, templates)
    tr = O.build_static_tree(frontiers, st.root_token, st.P, m)
    n = min(m, 1 + D * k)
    assert len(tr.tokens) == n and tr.parents[0] == -1 and tr.tokens[0] == st.root_token
    for f in range(1, n):
        L, j = 1 + (f - 1) // k, (f - 1) % k
        p = int(tr.parents[f])
        assert 0 <= p < f and tr.depth[f] == tr.depth[p] + 1 == L
        # the node is the template's child of its parent: its pool entry is the
        # child of rank r of slot s, with (s, r) the template pair (depth 1: rank j)
        e = pool[int(tr.pool_idx[f])]
        if L == 1:
            assert int(tr.pool_idx[f]) == j and e.parent == -1
        else:
            s, r = templates[L][0][j], templates[L][1][j]
            base = k + (L - 2) * k * k
            assert int(tr.pool_idx[f]) == base + s * k + r and e.pslot == s
            assert p == 1 + (L - 2) * k + s
        assert tr.tokens[f] == e.token
        # score = sum of the draft log-probabilities along the path
        lp, a = 0.0, f
        while a > 0:
            lp += pool[int(tr.pool_idx[a])].logp
            a = int(tr.parents[a])
        assert abs(tr.logscore[f] - lp) < 1e-12
    # mask: ancestor-or-self, by brute force over parent chains
    for f in range(n):
        anc = set()
        a = f
        while a != -1:
            anc.add(a)
            a = int(tr.parents[a])
        assert [c for c in range(n) if tr.mask[f, c]] == sorted(anc)
    assert np.array_equal(tr.positions, st.P - 1 + tr.depth)


def test_static_template_out_of_range_is_rejected():
    cfg = tiny_cfg(D=2, k=2, m=5)
    model, st = _model(cfg, 1)
    with pytest.raises(ValueError):
        _static_levels(model, st, 2, 2, {2: ([0, 2], [0, 0])})
