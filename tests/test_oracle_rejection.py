"""CPU pins of the oracle's recursive rejection sampling (readings R17, R18).

[P1] §6.2 states that the scheme leaves the target distribution exactly
unchanged.  Here that is checked on the oracle itself: with one or two
children drawn i.i.d. from the draft distribution q (every token pair
enumerated with its probability), the first emitted token, measured by
calling the oracle over grids of uniforms, is distributed as p.  Also: q = p
accepts every child (the first draft token is always accepted, [P1] §7.1), a
draft with no mass where the target has any rejects everything, and the
temperature scales both logits.  R18 (the same rule with each fixed
candidate a point-mass proposal): the first emitted token is distributed as
p for fixed candidate lists over nested grids of uniforms, duplicates are
never accepted, the all-rejected draw is the residual draw, and at T -> 0
the walk is the greedy walk.
"""
import itertools

import numpy as np
import pytest

from oracle import eagle_oracle as O

N = 2000
GRID = (np.arange(N) + 0.5) / N
HI = 1.0 - 0.25 / N  # above every grid point: a rejection wherever one is possible


def _first_token(tl, dl, tokens, parents, T, u):
    path, alen, bonus, _ = O.verify_rejection(tl, dl, tokens, parents, T, u)
    return int(tokens[path[1]]) if alen > 1 else bonus


def _frac(values):
    return float(np.mean(values))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_one_child_drawn_from_q_is_lossless(seed):
    rng = np.random.default_rng(seed)
    V, T = 6, 1.0
    tl = rng.normal(size=(2, V)) * 1.5
    dl = rng.normal(size=(2, V)) * 1.5
    p, q = O.target_probs(tl[0], T), O.target_probs(dl[0], T)
    parents = np.array([-1, 0])
    out = np.zeros(V)
    for t1 in range(V):
        tokens = np.array([0, t1])
        u = np.array([0.0, 0.0, 0.0])
        acc = []
        for x in GRID:
            u[1] = x
            acc.append(_first_token(tl, dl, tokens, parents, T, u) == t1 and
                       O.verify_rejection(tl, dl, tokens, parents, T, u)[1] == 2)
        f1 = _frac(acc)
        draws = np.zeros(V)
        u[1] = HI
        for x in GRID:
            u[2] = x
            draws[_first_token(tl, dl, tokens, parents, T, u)] += 1.0 / N
        out[t1] += q[t1] * f1
        out += q[t1] * (1.0 - f1) * draws
    assert np.allclose(out, p, atol=4.0 / N)


def test_two_children_drawn_iid_from_q_are_lossless():
    rng = np.random.default_rng(9)
    V, T = 4, 0.8
    tl = rng.normal(size=(3, V)) * 1.5
    dl = rng.normal(size=(3, V)) * 1.5
    p, q = O.target_probs(tl[0], T), O.target_probs(dl[0], T)
    parents = np.array([-1, 0, 0])
    out = np.zeros(V)
    for t1, t2 in itertools.product(range(V), repeat=2):
        tokens = np.array([0, t1, t2])
        u = np.zeros(4)
        f1 = _frac([O.verify_rejection(tl, dl, tokens, parents, T, np.array([0, x, 0, 0]))[0][1:2] == [1]
                    for x in GRID])
        f2 = _frac([O.verify_rejection(tl, dl, tokens, parents, T, np.array([0, HI, x, 0]))[0][1:2] == [2]
                    for x in GRID])
        draws = np.zeros(V)
        for x in GRID:
            u[:] = [0, HI, HI, x]
            path, alen, bonus, _ = O.verify_rejection(tl, dl, tokens, parents, T, u)
            if alen == 1:
                draws[bonus] += 1.0 / N
        w = q[t1] * q[t2]
        out[t1] += w * f1
        out[t2] += w * (1 - f1) * f2
        if f2 < 1.0:
            out += w * (1 - f1) * draws
    assert np.allclose(out, p, atol=6.0 / N)


def test_draft_equal_to_target_accepts_every_first_child():
    rng = np.random.default_rng(4)
    m, V = 9, 10
    parents = np.array([-1, 0, 0, 1, 1, 2, 3, 3, 6])
    tokens = rng.integers(0, V, size=m)
    tl = rng.normal(size=(m, V))
    for u_val in (0.0, 0.5, HI):
        path, alen, _, _ = O.verify_rejection(tl, tl.copy(), tokens, parents, 1.3, np.full(m + 1, u_val))
        assert path == [0, 1, 3, 6, 8] and alen == 5


def test_draft_without_target_mass_rejects_everything():
    """q lives on tokens 0..2 where p is zero: every child is rejected, the
    residual max(0, p - q) is p itself and the bonus is drawn from p."""
    V = 6
    tl = np.log(np.array([[1e-300, 1e-300, 1e-300, 0.2, 0.3, 0.5]] * 3))
    dl = np.log(np.array([[0.5, 0.3, 0.2, 1e-300, 1e-300, 1e-300]] * 3))
    tokens = np.array([4, 0, 2])
    parents = np.array([-1, 0, 0])
    for x, want in ((0.1, 3), (0.3, 4), (0.9, 5)):
        path, alen, bonus, _ = O.verify_rejection(tl, dl, tokens, parents, 1.0, np.array([0.0, 0.5, 0.5, x]))
        assert path == [0] and bonus == want


def test_temperature_divides_both_logits():
    rng = np.random.default_rng(6)
    m, V, T = 6, 8, 2.5
    parents = np.array([-1, 0, 0, 1, 2, 2])
    tokens = rng.integers(0, V, size=m)
    tl, dl = rng.normal(size=(m, V)) * 2, rng.normal(size=(m, V)) * 2
    for s in range(5):
        u = np.random.default_rng(s).random(m + 1)
        a = O.verify_rejection(tl, dl, tokens, parents, T, u)
        b = O.verify_rejection(tl / T, dl / T, tokens, parents, 1.0, u)
        assert a[:3] == b[:3]


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_residual_closed_form(seed):
    """The GPU walk keeps the residual after j rejections at a node as
    max(0, p - c q) / N, with c <- c + N and N <- sum max(0, p - c q) on each
    rejection (kept when that sum is 0).  Held here to the residual as [P1]
    §6.2 defines it, norm(max(0, r - q)) applied j times, in fp64."""
    rng = np.random.default_rng(seed)
    V = 50
    p = O.target_probs(rng.normal(size=V) * 2, 1.0)
    q = O.target_probs(rng.normal(size=V) * 2, 1.0)
    if seed == 3:
        q[:10] = 0.0  # the draft misses part of the target's support
        q /= q.sum()
    r, c, N = p.copy(), 0.0, 1.0
    for _ in range(12):
        d = np.maximum(0.0, r - q)
        if d.sum() > 0:
            r = d / d.sum()
        cn = c + N
        Nn = np.maximum(0.0, p - cn * q).sum()
        if Nn > 0:
            c, N = cn, Nn
        assert np.allclose(np.maximum(0.0, p - c * q) / N, r, rtol=1e-9, atol=1e-12)


def test_token_without_target_mass_is_never_accepted():
    """min(1, p/q) is 0 where p(t) is 0: such a child is rejected even with
    u = 0 and a draft probability that is 0 too (at a low temperature both
    can vanish; 0 <= 0 must not accept)."""
    V = 5
    tl = np.array([[0.0, 0.0, -np.inf, 10.0, 0.0]] * 2)
    dl = np.array([[10.0, -np.inf, -np.inf, 0.0, 0.0]] * 2)
    tokens, parents = np.array([0, 2]), np.array([-1, 0])
    for T in (1.0, 0.05):
        path, alen, bonus, margins = O.verify_rejection(tl, dl, tokens, parents, T, np.zeros(3))
        assert path == [0] and alen == 1 and margins[0] == np.inf


# ------------------------------------------------------------------ R18: deterministic candidates

def _first_token_topk(tl, tokens, parents, T, u):
    path, alen, bonus, _ = O.verify_rejection_topk(tl, tokens, parents, T, u)
    return int(tokens[path[1]]) if alen > 1 else bonus


@pytest.mark.parametrize("kids", [(3,), (1, 4), (5, 0, 2), (2, 2)])
def test_fixed_candidates_are_lossless(kids):
    """[P1] §6.2's guarantee for a fixed candidate list (EAGLE-2's top-k
    children are not draws from q): over a grid of every child's uniform and
    the bonus uniform, the first emitted token is distributed as p.  The
    children's uniforms are walked in nested grids (a later child's only
    matters where the earlier ones rejected), the bonus's over a grid."""
    rng = np.random.default_rng(sum(kids) + 10 * len(kids))
    V, T, n = 6, 0.9, 400
    grid = (np.arange(n) + 0.5) / n
    m = 1 + len(kids)
    tl = rng.normal(size=(m, V)) * 1.5
    p = O.target_probs(tl[0], T)
    tokens = np.array([0] + list(kids))
    parents = np.array([-1] + [0] * len(kids))
    out = np.zeros(V)

    def walk(c, u, weight):
        # child c decides: the grid fraction that accepts it, then deeper
        if c == m:
            draws = np.zeros(V)
            for x in grid:
                u[m] = x
                draws[_first_token_topk(tl, tokens, parents, T, u)] += 1.0 / n
            out[:] += weight * draws
            return
        acc = 0.0
        for x in grid:
            u[c] = x
            path, alen, _, _ = O.verify_rejection_topk(tl, tokens, parents, T, u)
            acc += (alen > 1 and path[1] == c) / n
        out[int(tokens[c])] += weight * acc
        u[c] = 1.0 - 0.25 / n  # above every grid point: child c rejected
        if acc < 1.0:
            walk(c + 1, u, weight * (1.0 - acc))

    walk(1, np.zeros(m + 1), 1.0)
    assert np.allclose(out, p, atol=2.0 * len(kids) / n)


def test_fixed_candidates_duplicate_and_draw():
    """A token an earlier sibling already carries is never accepted; when
    every child is rejected the bonus is the residual draw with the children
    removed (sample_residual)."""
    rng = np.random.default_rng(3)
    V, T = 7, 1.0
    tl = rng.normal(size=(4, V))
    tokens, parents = np.array([0, 3, 3, 5]), np.array([-1, 0, 0, 0])
    p = O.target_probs(tl[0], T)
    for ub in (0.1, 0.5, 0.93):
        u = np.array([0.0, 0.999, 0.0, 0.999, ub])  # child 1 and 3 rejected; 2 duplicates 1
        path, alen, bonus, margins = O.verify_rejection_topk(tl, tokens, parents, T, u)
        assert path == [0] and margins[1] == np.inf
        assert bonus == O.sample_residual(p, [3, 3, 5], ub)[0]
    # a child is accepted with the residual probability: p(t)/(1 - mass removed)
    r = p[5] / (1.0 - p[3])
    for x, want in ((r * 0.999, [0, 3]), (r * 1.001, [0])):
        path = O.verify_rejection_topk(tl, tokens, parents, T, np.array([0.0, 0.999, 0.0, x, 0.5]))[0]
        assert path == want


def test_fixed_candidates_equal_target_greedy_at_low_temperature():
    """As T -> 0 the residual puts all mass on the argmax: the walk descends
    exactly where the greedy walk does (its first child carrying the argmax)."""
    rng = np.random.default_rng(8)
    m, V = 9, 12
    parents = np.array([-1, 0, 0, 1, 1, 2, 3, 3, 6])
    tl = rng.normal(size=(m, V)) * 3
    tokens = rng.integers(0, V, size=m)
    for node in range(m):  # plant: some node's child carries the argmax
        kids = [c for c in range(m) if parents[c] == node]
        if kids and rng.random() < 0.8:
            tokens[kids[-1]] = int(np.argmax(tl[node]))
    u = np.random.default_rng(1).random(m + 1) * 0.98
    a = O.verify_rejection_topk(tl, tokens, parents, 1e-3, u)
    g = O.verify_greedy(tl, tokens, parents)
    assert a[0] == g[0] and a[2] == g[2]
