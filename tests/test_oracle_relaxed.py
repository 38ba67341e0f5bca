"""CPU pins of the oracle's relaxed-acceptance walk (reading R15).

The walk is held to the greedy walk in the zero-temperature limit, to the
first-child chain at a zero threshold, to a brute-force sweep of the residual
draw over a fine grid of uniforms, to hand-built cases of the flat-order rule,
and to the invariance of softmax(l / T) under scaling l and T together.
"""
import numpy as np
import pytest

from oracle import eagle_oracle as O


def _random_tree(rng, m, V):
    """Flat tree (parent before child) whose siblings carry distinct tokens."""
    parents = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, m)], dtype=np.int64)
    tokens = np.zeros(m, dtype=np.int64)
    tokens[0] = int(rng.integers(0, V))
    for x in range(m):
        kids = [c for c in range(m) if parents[c] == x]
        ids = rng.choice(V, size=len(kids), replace=False)
        for c, t in zip(kids, ids):
            tokens[c] = int(t)
    return tokens, parents


def _plant_path(rng, logits, tokens, parents, gap):
    """Make the target's argmax at each node along a random root path a child
    of that node (by `gap` over the row's other logits); the path's last node
    gets an argmax that is none of its children."""
    m, V = logits.shape
    node = 0
    while True:
        kids = [c for c in range(m) if parents[c] == node]
        row = logits[node]
        if kids and rng.random() < 0.8:
            c = kids[int(rng.integers(0, len(kids)))]
            row[tokens[c]] = row.max() + gap
            node = c
            continue
        banned = {int(tokens[c]) for c in kids}
        t = next(int(x) for x in rng.permutation(V) if int(x) not in banned)
        row[t] = row.max() + gap
        return


@pytest.mark.parametrize("seed", range(12))
def test_relaxed_at_low_temperature_is_the_greedy_walk(seed):
    """T -> 0 makes p one-hot at the argmax: with threshold 1/2 a child passes
    iff it is the argmax, and the residual at the stop is the argmax itself,
    so the walk, its length and the bonus are those of the greedy walk."""
    rng = np.random.default_rng(100 + seed)
    m, V = 14, 40
    tokens, parents = _random_tree(rng, m, V)
    logits = rng.normal(size=(m, V))
    _plant_path(rng, logits, tokens, parents, gap=1.0)
    g_path, g_len, g_bonus, _ = O.verify_greedy(logits, tokens, parents)
    for u in (0.0, 0.37, 0.999):
        path, alen, bonus, _ = O.verify_relaxed(logits, tokens, parents, 1e-3, 0.5, u)
        assert (path, alen, bonus) == (g_path, g_len, g_bonus)


def test_relaxed_zero_threshold_follows_first_children():
    """threshold 0: every child passes, so the walk takes the first child in
    flat order until a leaf, where nothing is removed and the bonus is the
    inverse-CDF draw from p itself."""
    rng = np.random.default_rng(5)
    m, V, T = 12, 30, 0.8
    tokens, parents = _random_tree(rng, m, V)
    logits = rng.normal(size=(m, V))
    node, want = 0, [0]
    while True:
        kids = [c for c in range(m) if parents[c] == node]
        if not kids:
            break
        node = kids[0]
        want.append(node)
    p = np.exp(logits[node] / T - (logits[node] / T).max())
    p /= p.sum()
    for u in (0.01, 0.5, 0.93):
        path, alen, bonus, _ = O.verify_relaxed(logits, tokens, parents, T, 0.0, u)
        assert path == want and alen == len(want)
        assert bonus == int(np.argmax(np.cumsum(p) > u))


def test_residual_draw_matches_its_distribution_on_a_grid():
    """Sweeping u over N evenly spaced points, each token is drawn a number of
    times within one of N times its residual probability; removed tokens never."""
    rng = np.random.default_rng(9)
    V, N = 7, 20000
    p = rng.random(V) + 0.05
    p /= p.sum()
    removed = [1, 4]
    r = p.copy()
    r[removed] = 0.0
    r /= r.sum()
    counts = np.zeros(V)
    for i in range(N):
        x, mg = O.sample_residual(p, removed, (i + 0.5) / N)
        assert mg >= 0.0
        counts[x] += 1
    assert counts[removed].sum() == 0
    assert np.all(np.abs(counts / N - r) <= 1.0 / N + 1e-12)
    # the ends of [0, 1): first and last token with mass
    assert O.sample_residual(p, removed, 0.0)[0] == 0
    assert O.sample_residual(p, removed, np.nextafter(1.0, 0.0))[0] == 6


def test_residual_with_all_mass_removed_draws_from_p():
    p = np.array([0.5, 0.3, 0.2])
    assert O.sample_residual(p, [0, 1, 2], 0.6)[0] == 1
    assert O.sample_residual(p, [0, 1, 2], 0.1)[0] == 0


def test_relaxed_bonus_at_the_root_is_the_root_residual():
    """A threshold above 1 accepts nothing: over a grid of uniforms the bonus
    follows p with the root's children removed."""
    rng = np.random.default_rng(21)
    m, V, T, N = 9, 12, 1.3, 6000
    tokens, parents = _random_tree(rng, m, V)
    logits = rng.normal(size=(m, V)) * 2.0
    kids = [int(tokens[c]) for c in range(m) if parents[c] == 0]
    p = np.exp(logits[0] / T - (logits[0] / T).max())
    p /= p.sum()
    r = p.copy()
    r[kids] = 0.0
    r /= r.sum()
    counts = np.zeros(V)
    for i in range(N):
        path, alen, bonus, _ = O.verify_relaxed(logits, tokens, parents, T, 1.5, (i + 0.5) / N)
        assert path == [0] and alen == 1
        counts[bonus] += 1
    assert np.all(np.abs(counts / N - r) <= 1.0 / N + 1e-12)


def test_relaxed_takes_the_first_passing_child_in_flat_order():
    """Children c1 (flat index 1) and c2 (flat index 2) of the root with target
    probabilities 0.35 and 0.45: threshold 0.3 takes c1 although c2 is more
    likely, 0.4 takes c2, 0.5 takes neither."""
    V = 6
    tokens = np.array([0, 2, 5], dtype=np.int64)
    parents = np.array([-1, 0, 0], dtype=np.int64)
    p_root = np.array([0.05, 0.05, 0.35, 0.05, 0.05, 0.45])
    logits = np.zeros((3, V))
    logits[0] = np.log(p_root)
    assert O.verify_relaxed(logits, tokens, parents, 1.0, 0.3, 0.5)[0] == [0, 1]
    assert O.verify_relaxed(logits, tokens, parents, 1.0, 0.4, 0.5)[0] == [0, 2]
    path, alen, bonus, margins = O.verify_relaxed(logits, tokens, parents, 1.0, 0.5, 0.6)
    assert path == [0] and alen == 1
    # residual over tokens {0, 1, 3, 4}, each 1/4: u = 0.6 falls in token 3's quarter
    assert bonus == 3
    assert margins[:2] == pytest.approx([0.15, 0.05])
    assert margins[2] == pytest.approx(0.1)


def test_residual_draw_interval_convention():
    """Token x owns [C(x-1), C(x)): a uniform exactly on a boundary belongs to
    the token above it (exactly representable cumulative sums)."""
    p = np.array([0.25, 0.25, 0.5])
    assert O.sample_residual(p, [], 0.25)[0] == 1
    assert O.sample_residual(p, [], 0.5)[0] == 2
    assert O.sample_residual(p, [], 0.0)[0] == 0
    assert O.sample_residual(p, [1], 0.25)[0] == 0  # residual [1/3, 0, 2/3]
    assert O.sample_residual(p, [1], 0.4)[0] == 2


@pytest.mark.parametrize("T", [0.5, 2.0])
def test_relaxed_depends_on_logits_over_temperature(T):
    """softmax(l / T): scaling l and T by the same factor changes nothing, while
    the same logits at another temperature do change the probabilities."""
    rng = np.random.default_rng(int(T * 10))
    m, V = 10, 25
    tokens, parents = _random_tree(rng, m, V)
    logits = rng.normal(size=(m, V)) * 2.0
    for u in (0.2, 0.7):
        a = O.verify_relaxed(logits, tokens, parents, T, 0.08, u)
        b = O.verify_relaxed(logits / T, tokens, parents, 1.0, 0.08, u)
        assert a[:3] == b[:3]
    p1 = O.target_probs(logits[0], 1.0)
    pT = O.target_probs(logits[0], T)
    assert np.allclose(pT, p1 ** (1.0 / T) / (p1 ** (1.0 / T)).sum())
    assert not np.allclose(pT, p1)
