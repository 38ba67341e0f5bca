"""CPU pins of the oracle's expansion, rerank, flattening, verify walk and
extend, against brute force, invariants the pages state, special cases and
the pages' worked numbers (tests/golden/)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import eagle_oracle as O
from tests._tiny import seq_state, tensors, tiny_cfg

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _levels(model, st, D, k, perturb=None):
    pool, F, _ = O.level_one(model, st, k)
    frontiers, feats, intree = [F], {}, {}
    for level in range(2, D + 1):
        if perturb is not None and level == perturb[0]:
            depth, slot, delta = perturb[1:]
            kk, vv = intree[(depth, slot)]
            intree[(depth, slot)] = (kk + delta, vv + delta)
        h = O.level_step_forward(model, st, level, F, feats, intree)
        F, _, _ = O.level_step_tail(model, level, F, h, pool, k)
        frontiers.append(F)
    return pool, frontiers, feats, intree


def _random_model(cfg, seed, scale=0.4):
    rng = np.random.default_rng(seed)
    return O.Model(cfg, tensors(cfg, rng, scale=scale)), seq_state(cfg, rng)


@pytest.mark.parametrize("D,k", [(2, 1), (3, 2), (4, 3), (3, 5)])
def test_pool_scores_are_path_sums_and_frontier_is_best_k(D, k):
    cfg = tiny_cfg(D=D, k=k, V=23, m=4)
    model, st = _random_model(cfg, 100 + 10 * D + k)
    pool, frontiers, _, _ = _levels(model, st, D, k)
    assert len(pool) == k + (D - 1) * k * k
    for i, e in enumerate(pool):
        # value(t_i) = prod of confidences on the root path ([P1] §10.3): re-walk parents
        s, j = 0.0, i
        while j != -1:
            s += pool[j].logp
            j = pool[j].parent
        assert abs(e.score - s) < 1e-12
        assert e.logp <= 0
        if e.parent != -1:
            assert e.score <= pool[e.parent].score       # property 1 of [P1] §10.3
            assert e.depth == pool[e.parent].depth + 1
    for level, F in enumerate(frontiers, start=1):
        lo = k if level == 1 else k + (level - 2) * k * k
        hi = k if level == 1 else lo + k * k
        cand = set(range(0 if level == 1 else lo, hi))
        chosen = [x.pool_idx for x in F]
        assert len(F) == min(k, len(cand)) and set(chosen) <= cand
        for x in chosen:  # everything kept beats everything dropped
            for y in cand - set(chosen):
                assert (-pool[x].score, x) < (-pool[y].score, y)
        for j, x in enumerate(F):
            assert x.anc[-1] == j and len(x.anc) == level
            if level > 1:
                assert x.anc[:-1] == frontiers[level - 2][x.pslot].anc
                assert pool[x.pool_idx].parent == frontiers[level - 2][x.pslot].pool_idx


def test_feature_plumbing_through_levels():
    # FC = [I | I], no attention or MLP output: h(x) = h(parent) + e(tok(x)), so a
    # node's feature is the root feature plus the embeddings along its path.
    cfg = tiny_cfg(D=4, k=2, V=15)
    d = cfg.d
    rng = np.random.default_rng(12)
    t = tensors(cfg, rng, fc_w=np.hstack([np.eye(d), np.eye(d)]), fc_b=np.zeros(d),
                wo=np.zeros((d, d)), w_down=np.zeros((d, cfg.F)))
    model = O.Model(cfg, t)
    st = seq_state(cfg, rng)
    pool, frontiers, feats, _ = _levels(model, st, cfg.D, cfg.k)
    for depth in range(1, cfg.D):
        for j, x in enumerate(frontiers[depth - 1]):
            want, i = st.root_feat.copy(), x.pool_idx
            while i != -1:
                want += model.embed_rows([pool[i].token])[0]
                i = pool[i].parent
            assert np.allclose(feats[(depth, j)], want, atol=1e-12)


def test_ancestor_only_visibility():
    # perturbing the in-tree K/V of a slot changes exactly the rows that have it as
    # an ancestor ([P1] §12 item 5: the mask looks only at ancestors)
    cfg = tiny_cfg(D=4, k=3, V=19)
    model, st = _random_model(cfg, 13)
    _, fr0, feats0, _ = _levels(model, st, cfg.D, cfg.k)
    for slot in range(cfg.k):
        _, fr1, feats1, _ = _levels(model, st, cfg.D, cfg.k, perturb=(3, 1, slot, 5.0))
        for j, x in enumerate(fr0[1]):  # rows forwarded at level 3 (depth 2)
            same = np.allclose(feats0[(2, j)], feats1[(2, j)], atol=1e-12)
            assert same == (x.anc[0] != slot)


def test_rerank_is_best_m_minus_1_and_ancestor_closed():
    cfg = tiny_cfg(D=4, k=3, V=19)
    model, st = _random_model(cfg, 14)
    pool, _, _, _ = _levels(model, st, cfg.D, cfg.k)
    for m in (2, 5, 11, len(pool) + 1):
        sel, margin = O.rerank(pool, m)
        assert len(sel) == m - 1
        rest = set(range(len(pool))) - set(sel)
        key = lambda i: (-pool[i].score, pool[i].depth, i)
        assert all(key(a) < key(b) for a in sel for b in rest)
        assert all(pool[i].parent == -1 or pool[i].parent in sel for i in sel)
        if rest:
            assert margin >= 0
        # the root's best child always makes it in ([P1] §10.3: it has the top value)
        assert 0 in sel


def test_rerank_tie_prefers_shallow():
    # a child with probability 1 ties its parent; the parent (shallower) ranks first
    pool = [O.PoolEntry(-0.5, -0.5, 3, -1, 1, -1), O.PoolEntry(-0.9, -0.9, 4, -1, 1, -1),
            O.PoolEntry(-0.5, 0.0, 7, 0, 2, 0), O.PoolEntry(-2.0, -1.5, 8, 0, 2, 0)]
    sel, _ = O.rerank(pool, 2)
    assert sel == [0]
    sel, _ = O.rerank(pool, 3)
    assert sel == [0, 2]


def test_flatten_order_matches_p4_diagram():
    g = json.load(open(os.path.join(GOLDEN, "flatten_order_p4.json")))
    names, pool = [], []
    # level-1 nodes in rank order; x2's children outscore x1's later children, so a
    # score-sorted flatten would put x2a before x1b
    probs1 = [0.45, 0.35, 0.2]
    child_probs = {"x1": [0.5, 0.3, 0.2], "x2": [0.9, 0.05, 0.05], "x3": [0.6, 0.2, 0.2]}
    for r, n in enumerate(g["level1"]):
        pool.append(O.PoolEntry(math.log(probs1[r]), math.log(probs1[r]), 100 + r, -1, 1, -1))
        names.append(n)
    for j, n in enumerate(g["level1"]):
        for c, cn in enumerate(g["children"][n]):
            lp = math.log(child_probs[n][c])
            pool.append(O.PoolEntry(pool[j].score + lp, lp, 200 + 3 * j + c, j, 2, j))
            names.append(cn)
    sel, _ = O.rerank(pool, len(pool) + 1)
    tree = O.build_tree(pool, sel, 7, P=10)
    flat = ["root"] + [names[i] for i in tree.pool_idx[1:]]
    assert flat[:len(g["flat_prefix"])] == g["flat_prefix"]
    assert list(tree.positions[:5]) == [9, 10, 10, 10, 11]


@pytest.mark.parametrize("D,k,m", [(3, 2, 6), (4, 3, 11), (5, 4, 20)])
def test_tree_structure_invariants(D, k, m):
    cfg = tiny_cfg(D=D, k=k, m=m, V=29)
    model, st = _random_model(cfg, 15 + m)
    pool, _, _, _ = _levels(model, st, D, k)
    sel, _ = O.rerank(pool, m)
    tr = O.build_tree(pool, sel, st.root_token, st.P)
    assert len(tr.tokens) == m and tr.parents[0] == -1 and tr.tokens[0] == st.root_token
    assert np.all(np.diff(tr.depth) >= 0)                      # depth-major
    for i in range(1, m):
        assert 0 <= tr.parents[i] < i
        assert tr.depth[i] == tr.depth[tr.parents[i]] + 1
    assert np.all(tr.positions == st.P - 1 + tr.depth)
    assert np.all(np.triu(tr.mask, 1) == 0)                    # only earlier columns
    assert np.all(tr.mask.sum(axis=1) == tr.depth + 1)         # ancestors + self
    for i in range(m):
        for j in range(m):
            a, anc = i, False
            while a != -1:
                anc |= a == j
                a = tr.parents[a]
            assert tr.mask[i, j] == int(anc)


def test_topk_one_is_a_chain():
    # [P2] Core Idea / [P3]: top-k = 1 degenerates the tree to a chain
    cfg = tiny_cfg(D=5, k=1, m=6, V=17)
    model, st = _random_model(cfg, 16)
    pool, _, _, _ = _levels(model, st, cfg.D, 1)
    assert len(pool) == cfg.D
    sel, _ = O.rerank(pool, cfg.m)
    tr = O.build_tree(pool, sel, st.root_token, st.P)
    assert list(tr.parents) == [-1, 0, 1, 2, 3, 4]
    assert np.array_equal(tr.mask, np.tril(np.ones((6, 6), dtype=np.uint8)))
    assert list(tr.positions) == [st.P - 1 + i for i in range(6)]


# ------------------------------------------------------------------ verify walk

def _brute_walk(TL, tokens, parents):
    """Longest root path whose every edge is the parent's target argmax."""
    m = len(tokens)
    best = [0]
    for node in range(m):
        path, a = [], node
        while a != -1:
            path.append(a)
            a = parents[a]
        path = path[::-1]
        ok = all(int(np.argmax(TL[path[i]])) == tokens[path[i + 1]] for i in range(len(path) - 1))
        if ok and len(path) > len(best):
            best = path
    return best, int(np.argmax(TL[best[-1]]))


def test_walk_matches_brute_force_on_planted_paths():
    rng = np.random.default_rng(17)
    cfg = tiny_cfg(D=4, k=3, V=21, m=12)
    model, st = _random_model(cfg, 18)
    pool, _, _, _ = _levels(model, st, cfg.D, cfg.k)
    sel, _ = O.rerank(pool, cfg.m)
    tr = O.build_tree(pool, sel, st.root_token, st.P)
    for trial in range(200):
        TL = rng.normal(0, 3, (cfg.m, cfg.V))
        # plant: follow random children with probability 0.7 per step
        node = 0
        while True:
            kids = [c for c in range(cfg.m) if tr.parents[c] == node]
            if not kids or rng.random() > 0.7:
                break
            c = kids[rng.integers(len(kids))]
            TL[node, tr.tokens[c]] = TL[node].max() + 1.0
            node = c
        path, alen, bonus, _ = O.verify_greedy(TL, tr.tokens, tr.parents)
        bpath, bbonus = _brute_walk(TL, tr.tokens, tr.parents)
        assert path == bpath and alen == len(bpath) and bonus == bbonus


def test_expected_accept_length_matches_pages():
    """Chain drafts whose i-th token matches the target's argmax with
    probability alpha_i give E[accept_len] = 1 + sum_i prod_{j<=i} alpha_j
    ([P1] §8 and §14 exercise 2; 50 000 rounds as in §14 exercise 6)."""
    g = json.load(open(os.path.join(GOLDEN, "expected_accept_length.json")))
    rng = np.random.default_rng(19)
    V = 16
    for case in g["cases"]:
        alpha = case["alpha"]
        K = len(alpha)
        tokens = np.array([0] + list(range(1, K + 1)))
        parents = np.array([-1] + list(range(K)))
        total = 0
        hits = rng.random((g["rounds"], K)) < np.array(alpha)
        for r in range(g["rounds"]):
            TL = np.zeros((K + 1, V))
            for i in range(K):
                want = tokens[i + 1] if hits[r, i] else (tokens[i + 1] % (K + 1)) + K + 1
                TL[i, want] = 1.0
            TL[K, 0] = 1.0
            _, alen, _, _ = O.verify_greedy(TL, tokens, parents)
            total += alen
        mean = total / g["rounds"]
        assert abs(mean - case["E_N"]) < 0.02, (case, mean)


def test_first_draft_token_is_always_accepted_when_q_equals_p():
    # [P1] §7.1: same feature + same LM head => q == p; greedily, the target's argmax
    # at the root is the draft's top-1 child, which is always in the tree
    cfg = tiny_cfg(D=3, k=2, V=25, m=5)
    for seed in range(20):
        model, st = _random_model(cfg, 200 + seed)
        root_logits = O.lm_logits(model, st.root_feat)[0]
        srt = np.sort(root_logits)
        if srt[-1] - srt[-2] < O.NEAR_TIE:
            continue
        pool, _, _, _ = _levels(model, st, cfg.D, cfg.k)
        sel, _ = O.rerank(pool, cfg.m)
        tr = O.build_tree(pool, sel, st.root_token, st.P)
        TL = np.random.default_rng(seed).normal(0, 3, (cfg.m, cfg.V))
        TL[0] = root_logits
        _, alen, _, _ = O.verify_greedy(TL, tr.tokens, tr.parents)
        assert alen >= 2


# ------------------------------------------------------------------ extend

def test_extend_shift_and_state_update():
    # FC = [0 | I] and no attention/MLP output: h_i = e(token carried by row i), i.e.
    # the next path token and the bonus for the last row (R2, R10)
    cfg = tiny_cfg(D=4, k=2, V=13, m=5)
    d = cfg.d
    rng = np.random.default_rng(20)
    t = tensors(cfg, rng, fc_w=np.hstack([np.zeros((d, d)), np.eye(d)]), fc_b=np.zeros(d),
                wo=np.zeros((d, d)), w_down=np.zeros((d, cfg.F)))
    model = O.Model(cfg, t)
    st = seq_state(cfg, rng)
    tokens = np.array([st.root_token, 4, 9, 2, 6])
    true_feat = rng.normal(size=(5, d))
    P0 = st.P
    h, kn, vn = O.draft_extend(model, st, true_feat, tokens, [0, 2, 3], bonus=11)
    assert np.allclose(h, model.embed_rows([9, 2, 11]), atol=1e-12)
    assert st.P == P0 + 3 and st.root_token == 11 and np.allclose(st.root_feat, h[-1])
    assert st.K.shape[0] == P0 + 3 and np.allclose(st.K[P0:], kn)
    # FC = [I | 0]: rows carry the true features of path nodes 0..a
    t["fc_w"] = np.hstack([np.eye(d), np.zeros((d, d))]).astype(np.float32)
    model = O.Model(cfg, t)
    st = seq_state(cfg, np.random.default_rng(20))
    h, _, _ = O.draft_extend(model, st, true_feat, tokens, [0, 2, 3], bonus=11)
    assert np.allclose(h, true_feat[[0, 2, 3]], atol=1e-12)


def test_extend_attention_is_prefix_plus_causal():
    # reduces to library attention with a [prefix visible | causal] boolean mask
    cfg = tiny_cfg(D=4, k=2, V=13, m=5, H=4, Hkv=2, d=16, hd=4)
    rng = np.random.default_rng(21)
    model = O.Model(cfg, tensors(cfg, rng))
    st = seq_state(cfg, rng, P=6)
    tokens = np.array([st.root_token, 4, 9, 2, 6])
    true_feat = rng.normal(size=(5, cfg.d))
    path, bonus = [0, 1, 3, 4], 8
    P0, K0, V0 = st.P, st.K.copy(), st.V.copy()
    h, kn, vn = O.draft_extend(model, st, true_feat, tokens, path, bonus)
    a = len(path)
    x0, q, k2, v2 = O.draft_rows(model, true_feat[path],
                                 [tokens[path[1]], tokens[path[2]], tokens[path[3]], bonus],
                                 [P0 + i for i in range(a)])
    K = np.concatenate([K0, k2]).repeat(2, axis=1)   # GQA: expand KV heads to H
    V = np.concatenate([V0, v2]).repeat(2, axis=1)
    mask = np.zeros((a, P0 + a), dtype=bool)
    mask[:, :P0] = True
    mask[:, P0:] = np.tril(np.ones((a, a), dtype=bool))
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(K).permute(1, 0, 2),
        torch.from_numpy(V).permute(1, 0, 2), attn_mask=torch.from_numpy(mask))
    attn = o.permute(1, 0, 2).reshape(a, -1).numpy()
    assert np.allclose(h, O.finish_rows(model, x0, attn), atol=1e-12)


# ------------------------------------------------------------------ whole rounds

@pytest.mark.parametrize("name", ["tiny", "ragged_f32", "chain_small", "hd128_bf16"])
def test_round_invariants_on_synthetic_configs(name):
    cfg = synth.config_by_name(name)
    inp = synth.make_inputs(cfg, 0)
    model = O.Model(cfg, inp)
    for b in range(cfg.B):
        W = lambda a: O.widen(a, cfg.dtype)
        st = O.SeqState(W(inp["k_cache"][b]), W(inp["v_cache"][b]), int(inp["prefix_len"][b]),
                        W(inp["root_feat"][b]), int(inp["root_token"][b]))
        P0 = st.P
        r = O.run_round(model, st, W(inp["true_feat"][b]),
                        inp["target_logits"][b].astype(np.float64))
        assert len(r.pool) == cfg.pool_size and len(r.tree.tokens) == cfg.m
        assert 1 <= r.accept_len <= cfg.D + 1 and st.P == P0 + r.accept_len
        assert np.all(r.tree.positions == P0 - 1 + r.tree.depth)
        if cfg.k == 1:
            assert list(r.tree.parents) == [-1] + list(range(cfg.m - 1))
