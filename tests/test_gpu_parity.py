"""GPU parity of the HIP draft round against the fp64 oracle, through the C ABI.

Gate (stage-isolated): each stage's inputs come from the generator or from
the oracle's earlier stages, rounded to the GPU's storage types and written
into the GPU workspace; both sides then compute that stage.
  * features, in-tree K/V, extend rows: relative L2 <= 1e-4 (fp32), 2e-2 (bf16)
  * top-k child probabilities |delta| <= 1e-3; node log-scores |delta| <= 1e-3
  * token ids, parents, frontier, pool, tree, mask, positions, accept length,
    path, bonus: bit-exact wherever the oracle's selection margins exceed
    1e-3 (log domain); rows below are counted as near-tie and reported.
End-to-end (gated for fp32 shapes, reported for bf16): whole rounds from the
generated inputs, three rounds in a row.
"""
from __future__ import annotations

import gc
import math

import numpy as np
import pytest

import synth
from oracle import eagle_oracle as O
from tests._gpu import (FEAT_TOL, HAVE_GPU, NEAR, PROB_TOL, SCORE_TOL, OracleSeqs, gpu_feats, logit_scale,
                        score_tol,
                        gpu_frontier, gpu_pool, gpu_rows, gpu_tree_kv, handover, pool_records,
                        quant, rel_l2, say, seed_workspace, store, to_host)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not HAVE_GPU, reason="needs a GPU")]

FAST = ["tiny", "tiny_bf16", "ragged_f32", "ragged_bf16", "hd128_bf16", "chain_small", "wide_bf16",
        "deep_bf16", "batch_bf16", "short_f32", "heads_bf16", "heads_f32", "rows64_bf16", "deep16_f32", "deep16_bf16"]
FULL = ["7b", "13b", "70b", "chain"]
# sequences the oracle checks at full size (the GPU runs the whole batch)
SAMPLE = {"13b": [0, 7, 15], "70b": [0, 3], "chain": [0, 31, 63]}

_CACHE: dict = {}


def get(name):
    import torch
    from eagle_draft_trees_amd.round import DraftRound
    if name not in _CACHE:
        _CACHE.clear()
        gc.collect()
        torch.cuda.empty_cache()
        cfg = synth.config_by_name(name)
        say(f"  generating inputs for {name}")
        inp = synth.make_inputs(cfg, seed=11)
        r = DraftRound(cfg, inp)
        _CACHE[name] = (cfg, inp, r, O.Model(cfg, inp), SAMPLE.get(name))
    cfg, inp, r, model, seqs = _CACHE[name]
    r.reset_state(inp)
    torch.cuda.synchronize()
    return cfg, inp, r, model, seqs


def oracle_for(cfg, inp, model, seqs):
    o = OracleSeqs.__new__(OracleSeqs)
    OracleSeqs.__init__(o, cfg, inp, seqs)
    o.model = model
    return o


def sync():
    import torch
    torch.cuda.synchronize()


def _check_children(cfg, gp_seq, o_entries, base, tails, strict, lscale):
    """Pool entries of one sequence's level: probabilities and scores within
    tolerance always (scores: score_tol of the row's logit scale lscale[j]);
    ids bit-exact where the row's tail margin is clear."""
    k = cfg.k
    g = gp_seq[base:base + len(o_entries)]
    n_rows = len(o_entries) // k
    near_rows = 0
    for j in range(n_rows):
        og = o_entries[j * k:(j + 1) * k]
        gg = g[j * k:(j + 1) * k]
        assert np.allclose(np.exp(gg["logp"]), [math.exp(e.logp) for e in og], atol=PROB_TOL, rtol=0)
        assert np.allclose(gg["score"], [e.score for e in og], atol=score_tol(cfg.d, lscale[j]), rtol=0)
        if tails[j] > NEAR:
            assert list(gg["token"]) == [e.token for e in og], f"row {j} ids"
            assert list(gg["parent"]) == [e.parent for e in og]
            assert list(gg["depth"]) == [e.depth for e in og]
            assert list(gg["pslot"]) == [e.pslot for e in og]
        else:
            near_rows += 1
    return near_rows


def _check_frontier(gf_seq, o_front):
    assert list(gf_seq["token"][:len(o_front)]) == [x.token for x in o_front]
    assert list(gf_seq["pool_idx"][:len(o_front)]) == [x.pool_idx for x in o_front]
    assert list(gf_seq["pslot"][:len(o_front)]) == [x.pslot for x in o_front]
    for j, x in enumerate(o_front):
        assert list(gf_seq[j]["anc"][:len(x.anc)]) == list(x.anc)


# ------------------------------------------------------------------ level 1

@pytest.mark.parametrize("name", FAST + FULL)
def test_level1_tail(name):
    cfg, inp, r, model, seqs = get(name)
    say(f"[level1 tail] {name}")
    orc = oracle_for(cfg, inp, model, seqs)
    r.level(1)
    sync()
    orc.level1()
    gp, gf = gpu_pool(r), gpu_frontier(r, 1)
    near = 0
    clear = []
    for b in orc.seqs:
        n = _check_children(cfg, gp[b], orc.pool[b], 0, orc.tail_margin[b], True,
                            logit_scale(orc.model, orc.st[b].root_feat))
        near += n
        if n == 0:
            _check_frontier(gf[b], orc.F[b][0])
            clear.append(b)
    say(f"  level1 {name}: {len(orc.seqs)} sequences, {near} near-tie rows")
    if handover(cfg):
        # level 1's merge launch formed level 2's FC input: each depth-1 node's
        # row is [root feature || e(its token)] ([P1] §4.1)
        from eagle_draft_trees_amd import _lib as L
        gx0 = gpu_rows(r, L.WS_X0, cfg.d)
        worst = 0.0
        for b in clear:
            F = orc.F[b][0]
            x0_o = O.draft_rows(orc.model, np.stack([orc.st[b].root_feat] * len(F)),
                                [x.token for x in F], [0] * len(F))[0]
            for j in range(cfg.k):
                e = rel_l2(gx0[b * cfg.k + j], x0_o[j])
                worst = max(worst, e)
                assert e <= FEAT_TOL["f32"], (b, j, e)
        say(f"  FC hand-over {name} level 1: {len(clear)} sequences, worst x0 rel L2 {worst:.2e}")


# ------------------------------------------------------------------ levels >= 2

def _levels_for(name):
    return list(range(2, synth.config_by_name(name).D + 1))


@pytest.mark.parametrize("name,level", [(n, L) for n in FAST + FULL for L in _levels_for(n)])
def test_level_forward_then_tail(name, level):
    import torch
    from eagle_draft_trees_amd import _lib as L
    cfg, inp, r, model, seqs = get(name)
    say(f"[level {level}] {name}")
    orc = oracle_for(cfg, inp, model, seqs)
    orc.level1()
    for lv in range(2, level):
        h = orc.forward(lv)
        orc.tail(lv, h)
    for dep in range(1, level - 1):
        orc.quantize_state(dep)
    orc.quantize_scores()
    seed_workspace(r, orc, upto_depth=level - 1)
    sync()
    # the workspace was written here, so this level forms its own FC input
    r.level(level, L.EAGLE_LEVEL_FULL_FC)
    sync()
    parts = {}
    h_o = orc.forward(level, parts)  # the same (rounded) stage inputs
    depth = level - 1
    gfeat = gpu_feats(r, depth)
    gtk, gtv = gpu_tree_kv(r)
    g_mid = {"x0": gpu_rows(r, L.WS_X0, cfg.d), "attn": gpu_rows(r, L.WS_ATTN, cfg.H * cfg.hd),
             "y": gpu_rows(r, L.WS_Y, cfg.d)}
    tol = FEAT_TOL[cfg.dtype]
    worst, mid = 0.0, {key: 0.0 for key in g_mid}
    for b in orc.seqs:
        for j in range(cfg.k):
            e = rel_l2(gfeat[b, j], h_o[b][j])
            worst = max(worst, e)
            assert e <= tol, (b, j, e)
            ok, ov = orc.intree[b][(depth, j)]
            assert rel_l2(gtk[b, depth, j], ok) <= tol
            assert rel_l2(gtv[b, depth, j], ov) <= tol
            for key, g in g_mid.items():   # per-intermediate errors, reported
                if key == "x0" and handover(cfg) and level < cfg.D:
                    continue  # the merge launch has already formed the next level's x0
                mid[key] = max(mid[key], rel_l2(g[b * cfg.k + j], parts[b][key][j]))
    say(f"  forward {name} level {level}: worst feature rel L2 {worst:.2e} (tol {tol}); "
        f"intermediates x0 {mid['x0']:.2e}, attention {mid['attn']:.2e}, y {mid['y']:.2e}")

    # tail-only stage on the oracle's features, rounded as the GPU stores them
    orc.quantize_state(depth)
    es = 2 if cfg.dtype == "bf16" else 4
    for b in orc.seqs:
        for j in range(cfg.k):
            r.ws_write(L.WS_FEAT, store(orc.feats[b][(depth, j)], cfg.dtype),
                       (((depth * cfg.B) + b) * cfg.k + j) * cfg.d * es)
    sync()
    r.level(level, L.EAGLE_LEVEL_TAIL_ONLY)
    sync()
    hq = {b: np.stack([orc.feats[b][(depth, j)] for j in range(cfg.k)]) for b in orc.seqs}
    orc.tail(level, hq)
    gp, gf = gpu_pool(r), gpu_frontier(r, level)
    base = cfg.k + (level - 2) * cfg.k * cfg.k
    near = 0
    clear = []
    for b in orc.seqs:
        tails = orc.tail_margin[b][-cfg.k:]
        ls = logit_scale(orc.model, hq[b])
        n = _check_children(cfg, gp[b], orc.pool[b][base:base + cfg.k * cfg.k], base, tails, True, ls)
        near += n
        if n == 0 and orc.sel_margin[b][-1] > NEAR:
            _check_frontier(gf[b], orc.F[b][-1])
            assert np.allclose(gf[b]["score"][:cfg.k], [x.score for x in orc.F[b][-1]],
                               atol=score_tol(cfg.d, ls.max()), rtol=0)
            clear.append(b)
    say(f"  tail {name} level {level}: {near} near-tie rows")
    if handover(cfg) and level < cfg.D:
        # the merge launch also formed the next level's FC input from the seeded
        # features and the frontier it chose: x0 of each next-frontier node x is
        # FC([feature of x's parent || e(token of x)]) ([P1] §4.1)
        gx0 = gpu_rows(r, L.WS_X0, cfg.d)
        worst = 0.0
        for b in clear:
            F = orc.F[b][-1]
            pf = np.stack([orc.feats[b][(depth, x.pslot)] for x in F])
            x0_o = O.draft_rows(orc.model, pf, [x.token for x in F], [0] * len(F))[0]
            for j in range(cfg.k):
                e = rel_l2(gx0[b * cfg.k + j], x0_o[j])
                worst = max(worst, e)
                assert e <= FEAT_TOL["f32"], (b, j, e)
        say(f"  FC hand-over {name} level {level}: {len(clear)} sequences, worst x0 rel L2 {worst:.2e}")


# ------------------------------------------------------------------ static tree

STATIC = ["tiny", "ragged_f32", "hd128_bf16", "wide_bf16", "7b"]


@pytest.mark.parametrize("name", STATIC)
def test_static_tree(name):
    """Static (fixed-shape) tree, reading R16: per level, the oracle's
    frontier and random features are seeded and the template's tail-only
    level runs (children and the template-picked frontier compared); then all
    the oracle's static frontiers are seeded and the built tree is compared
    exactly."""
    import torch
    from eagle_draft_trees_amd import _lib as L
    cfg, inp, r, model, seqs = get(name)
    say(f"[static] {name}")
    orc = oracle_for(cfg, inp, model, seqs)
    orc.level1()
    k, D, B, d = cfg.k, cfg.D, cfg.B, cfg.d
    es = 2 if cfg.dtype == "bf16" else 4
    rng = np.random.default_rng(31)
    tm = np.zeros((D, k, 2), dtype=np.int32)
    for lv in range(2, D + 1):
        pairs = rng.choice(k * k, size=k, replace=False)
        tm[lv - 1, :, 0], tm[lv - 1, :, 1] = pairs // k, pairs % k
    tmpl = torch.from_numpy(tm).to(r.device)
    near = 0
    for level in range(2, D + 1):
        depth = level - 1
        h = {b: quant(rng.normal(size=(k, d)), cfg.dtype) for b in orc.seqs}
        orc.quantize_scores()
        seed_workspace(r, orc, upto_depth=depth)
        for b in orc.seqs:
            for j in range(k):
                r.ws_write(L.WS_FEAT, store(h[b][j], cfg.dtype), (((depth * B) + b) * k + j) * d * es)
        sync()
        r.level_static(level, tmpl, L.EAGLE_LEVEL_TAIL_ONLY)
        sync()
        for b in orc.seqs:
            F, tails = O.level_step_tail_static(orc.model, level, orc.F[b][-1], h[b], orc.pool[b], k,
                                                tm[level - 1, :, 0], tm[level - 1, :, 1])
            orc.F[b].append(F)
            orc.tail_margin[b] += tails
        gp, gf = gpu_pool(r), gpu_frontier(r, level)
        base = k + (level - 2) * k * k
        for b in orc.seqs:
            ls = logit_scale(orc.model, h[b])
            n = _check_children(cfg, gp[b], orc.pool[b][base:base + k * k], base, orc.tail_margin[b][-k:], True,
                                ls)
            near += n
            if n == 0:
                _check_frontier(gf[b], orc.F[b][-1])
                assert np.allclose(gf[b]["score"][:k], [x.score for x in orc.F[b][-1]],
                                   atol=score_tol(d, ls.max()), rtol=0)
    orc.quantize_scores()
    seed_workspace(r, orc, upto_depth=D)
    sync()
    r.build_static()
    sync()
    tok, par = r.tokens.cpu().numpy(), r.parents.cpu().numpy()
    dep, pos = r.depth.cpu().numpy(), r.positions.cpu().numpy()
    msk, lsc = r.mask.cpu().numpy(), r.logscore.cpu().numpy()
    for b in orc.seqs:
        tr = O.build_static_tree(orc.F[b], orc.st[b].root_token, orc.st[b].P, cfg.m)
        assert list(tok[b]) == list(tr.tokens) and list(par[b]) == list(tr.parents)
        assert list(dep[b]) == list(tr.depth) and list(pos[b]) == list(tr.positions)
        assert np.array_equal(msk[b], tr.mask)
        assert np.allclose(lsc[b], tr.logscore, atol=SCORE_TOL, rtol=0)  # seeded fp32 scores
    say(f"  static {name}: levels 2..{D} ({near} near-tie rows), tree of {cfg.m} nodes")


# ------------------------------------------------------------------ rerank, verify, extend

def _oracle_pool(cfg, inp, model, seqs, seed=5):
    """A full-depth candidate pool from the oracle (tails on random features)."""
    orc = oracle_for(cfg, inp, model, seqs)
    orc.level1()
    rng = np.random.default_rng(seed)
    for lv in range(2, cfg.D + 1):
        h = {b: rng.normal(size=(cfg.k, cfg.d)) for b in orc.seqs}
        orc.tail(lv, h)
    orc.quantize_scores()
    return orc


def _trees(cfg, orc):
    out = {}
    for b in orc.seqs:
        sel, margin = O.rerank(orc.pool[b], cfg.m)
        out[b] = (O.build_tree(orc.pool[b], sel, orc.st[b].root_token, orc.st[b].P), margin)
    return out


@pytest.mark.parametrize("name", FAST + FULL)
def test_rerank_build(name):
    from eagle_draft_trees_amd import _lib as L
    cfg, inp, r, model, seqs = get(name)
    say(f"[rerank/build] {name}")
    orc = _oracle_pool(cfg, inp, model, seqs)
    for b in orc.seqs:
        r.ws_write(L.WS_POOL, pool_records(orc.pool[b]), b * cfg.pool_size * L.POOL_DTYPE.itemsize)
    sync()
    r.rerank()
    sync()
    trees = _trees(cfg, orc)
    for name_, t in (("tokens", r.tokens), ("parents", r.parents), ("depth", r.depth),
                     ("positions", r.positions)):
        g = t.cpu().numpy()
        for b in orc.seqs:
            want = getattr(trees[b][0], name_)
            assert list(g[b]) == list(want), (name_, b)
    gm, gs = r.mask.cpu().numpy(), r.logscore.cpu().numpy()
    for b in orc.seqs:
        tr = trees[b][0]
        assert np.array_equal(gm[b], tr.mask)
        assert np.array_equal(gs[b], tr.logscore.astype(np.float32))
    say(f"  rerank {name}: min margin {min(m for _, m in trees.values()):.2e} (exact on equal keys)")


def _plant(cfg, inp, trees, seqs, seed=3, p=0.8):
    """Target logits with planted accepted paths: along a random root-to-leaf
    walk, each step's child token gets the row's top logit with prob p."""
    TL = inp["target_logits"].copy()
    rng = np.random.default_rng(seed)
    for b in seqs:
        tr = trees[b][0]
        node = 0
        while True:
            kids = [c for c in range(cfg.m) if tr.parents[c] == node]
            if not kids or rng.random() > p:
                break
            c = kids[rng.integers(len(kids))]
            TL[b, node, tr.tokens[c]] = TL[b, node].max() + 1.0
            node = c
    return TL


def _upload_tree(r, trees, seqs):
    import torch
    tok, par = r.tokens.cpu().numpy(), r.parents.cpu().numpy()
    for b in seqs:
        tok[b], par[b] = trees[b][0].tokens, trees[b][0].parents
    r.tokens.copy_(torch.from_numpy(tok))
    r.parents.copy_(torch.from_numpy(par))


@pytest.mark.parametrize("name", FAST + FULL)
def test_verify_walk(name):
    import torch
    cfg, inp, r, model, seqs = get(name)
    say(f"[verify] {name}")
    orc = _oracle_pool(cfg, inp, model, seqs)
    trees = _trees(cfg, orc)
    TL = _plant(cfg, inp, trees, orc.seqs)
    _upload_tree(r, trees, orc.seqs)
    r.target_logits.copy_(torch.from_numpy(TL))
    sync()
    r.verify()
    sync()
    al, ap, bo = r.accept_len.cpu().numpy(), r.accept_path.cpu().numpy(), r.bonus.cpu().numpy()
    near, lens = 0, []
    for b in orc.seqs:
        tr = trees[b][0]
        path, alen, bonus, wm = O.verify_greedy(TL[b].astype(np.float64), tr.tokens, tr.parents)
        if min(wm) <= NEAR:
            near += 1
            continue
        assert al[b] == alen and bo[b] == bonus, (b, al[b], alen, bo[b], bonus)
        assert list(ap[b][:alen]) == path and all(x == -1 for x in ap[b][alen:])
        lens.append(alen)
    say(f"  verify {name}: accept lengths {lens}, near-tie {near}")


@pytest.mark.parametrize("name", FAST + FULL)
def test_extend(name):
    _extend_case(name, "random")


@pytest.mark.parametrize("name", ["tiny", "tiny_bf16", "hd128_bf16", "7b", "70b"])
def test_extend_full_length(name):
    """accept_len = min(m, depth+1), the most the extend forwards per sequence,
    with the accepted path set directly to flat nodes 0, 1, 2, ... (the extend
    reads only the path, its tokens and the bonus), so that every extend row,
    the last included, carries real inputs and the last is the next root."""
    _extend_case(name, "full")


def _extend_case(name, plant):
    import torch
    cfg, inp, r, model, seqs = get(name)
    say(f"[extend:{plant}] {name}")
    orc = _oracle_pool(cfg, inp, model, seqs)
    trees = _trees(cfg, orc)
    TL = _plant(cfg, inp, trees, orc.seqs, p=0.9)
    _upload_tree(r, trees, orc.seqs)
    al, ap, bo = (r.accept_len.cpu().numpy(), r.accept_path.cpu().numpy(), r.bonus.cpu().numpy())
    ores = {}
    rng = np.random.default_rng(23)
    for b in orc.seqs:
        tr = trees[b][0]
        if plant == "full":
            alen = min(cfg.m, cfg.D + 1)
            path, bonus = list(range(alen)), int(rng.integers(0, cfg.V))
        else:
            path, alen, bonus, _ = O.verify_greedy(TL[b].astype(np.float64), tr.tokens, tr.parents)
        al[b], bo[b] = alen, bonus
        ap[b] = path + [-1] * (cfg.D + 1 - alen)
        ores[b] = (path, alen, bonus)
    r.accept_len.copy_(torch.from_numpy(al))
    r.accept_path.copy_(torch.from_numpy(ap))
    r.bonus.copy_(torch.from_numpy(bo))
    P0 = inp["prefix_len"].copy()
    sync()
    r.extend()
    sync()
    tol = FEAT_TOL[cfg.dtype]
    tf = O.widen(inp["true_feat"], cfg.dtype)
    g_root = to_host(r.root_feat)
    g_ext = to_host(r.ws_typed(6).view(cfg.B, min(cfg.m, cfg.D + 1), cfg.d))
    g_k, g_v = to_host(r.k_cache), to_host(r.v_cache)
    g_plen, g_rtok = r.prefix_len.cpu().numpy(), r.root_token.cpu().numpy()
    worst, lens = 0.0, []
    for b in orc.seqs:
        path, alen, bonus = ores[b]
        st = orc.st[b]
        h, kn, vn = O.draft_extend(model, st, tf[b], trees[b][0].tokens, path, bonus)
        lens.append(alen)
        assert g_plen[b] == P0[b] + alen and g_rtok[b] == bonus
        for i in range(alen):
            e = rel_l2(g_ext[b, i], h[i])
            worst = max(worst, e)
            assert e <= tol, (b, i, e)
            assert rel_l2(g_k[b, P0[b] + i], kn[i]) <= tol
            assert rel_l2(g_v[b, P0[b] + i], vn[i]) <= tol
        assert rel_l2(g_root[b], h[alen - 1]) <= tol
    say(f"  extend {name}: accept lengths {lens}, worst rel L2 {worst:.2e} (tol {tol})")


# ------------------------------------------------------------------ whole rounds

def _oracle_draft(model, st, cfg, info=None):
    """The oracle's tree and its smallest decision margin; `info` (a dict, if
    given) receives the stage of that margin and the level-2 feature rows."""
    k, D = cfg.k, cfg.D
    pool, F, mg = O.level_one(model, st, k)
    margins = [(x, "level 1 top-k", 1) for x in mg["tail"]]
    feats, intree = {}, {}
    for level in range(2, D + 1):
        h = O.level_step_forward(model, st, level, F, feats, intree)
        if info is not None and level == 2:
            info["h2"] = np.array(h)
        F, tails, sm = O.level_step_tail(model, level, F, h, pool, k)
        margins += [(x, f"level {level} top-k", level) for x in tails] + [(sm, f"level {level} k^2->k select", level)]
    sel, rm = O.rerank(pool, cfg.m)
    margins.append((rm, "rerank", D + 1))
    if info is not None:
        info["margins"] = margins
    return O.build_tree(pool, sel, st.root_token, st.P), min(x[0] for x in margins)


def _margin_at(info, depth):
    """The oracle's smallest decision margin among the decisions that can
    change a node at `depth`: every level up to it, and the rerank."""
    ms = [x for x in info.get("margins", []) if x[2] <= depth or x[1] == "rerank"]
    return min(ms, key=lambda x: x[0])[:2] if ms else (float("nan"), "?")


def _bf16_logit_error(model, cfg, h):
    """Largest change of a top-k log-probability when feature rows h (fp64) are
    stored in bf16: the scale of score noise that bf16 features alone put on
    the drafting decisions."""
    def logp(z):
        mx = z.max(axis=1, keepdims=True)
        return z - (mx + np.log(np.exp(z - mx).sum(axis=1, keepdims=True)))
    h = np.atleast_2d(h)
    lp = logp(O.lm_logits(model, h))
    lq = logp(O.lm_logits(model, quant(h, "bf16")))
    top = np.argsort(-lp, axis=1)[:, :cfg.k]
    return float(np.max(np.abs(np.take_along_axis(lp, top, 1) - np.take_along_axis(lq, top, 1))))


def _run_rounds(name, rounds, gate):
    import torch
    cfg, inp, r, model, seqs = get(name)
    seqs = list(range(cfg.B)) if seqs is None else seqs
    W = lambda a: O.widen(a, cfg.dtype)
    states = {b: O.SeqState(W(inp["k_cache"][b]), W(inp["v_cache"][b]), int(inp["prefix_len"][b]),
                            W(inp["root_feat"][b]), int(inp["root_token"][b])) for b in seqs}
    tf = W(inp["true_feat"])
    alive = set(seqs)
    stats = {"match": 0, "compared": 0, "near": 0, "feat": [], "path_differs": 0, "diffs": [],
             "diverged": [], "lerr": 0.0, "cmp": []}
    rng = np.random.default_rng(99)
    for rd in range(rounds):
        trees = {}
        for b in sorted(alive):
            info = {}
            tr, mmin = _oracle_draft(model, states[b], cfg, info)
            trees[b] = (tr, mmin, info)
            if not gate and "h2" in info:
                stats["lerr"] = max(stats["lerr"], _bf16_logit_error(model, cfg, info["h2"]))
        TL = inp["target_logits"].copy()
        for b in sorted(alive):   # plant a path so that accept lengths vary
            tr = trees[b][0]
            node = 0
            while rng.random() < 0.85:
                kids = [c for c in range(cfg.m) if tr.parents[c] == node]
                if not kids:
                    break
                c = kids[rng.integers(len(kids))]
                TL[b, node, tr.tokens[c]] = TL[b, node].max() + 1.0
                node = c
        r.target_logits.copy_(torch.from_numpy(TL))
        r.run_round()
        sync()
        err = int(r.ws_region(0).view(torch.int32)[0].item())
        assert err == 0, f"device error word {err:#x} after round {rd}"
        g_tok, g_par = r.tokens.cpu().numpy(), r.parents.cpu().numpy()
        g_mask, g_pos = r.mask.cpu().numpy(), r.positions.cpu().numpy()
        g_al, g_bo = r.accept_len.cpu().numpy(), r.bonus.cpu().numpy()
        g_path = r.accept_path.cpu().numpy()
        g_root = to_host(r.root_feat)
        g_plen = r.prefix_len.cpu().numpy()
        for b in sorted(alive):
            tr, mmin, info = trees[b]
            P0 = states[b].P
            path, alen, bonus, wm = O.verify_greedy(TL[b].astype(np.float64), tr.tokens, tr.parents)
            O.draft_extend(model, states[b], tf[b], tr.tokens, path, bonus)
            near = min(mmin, min(wm)) <= NEAR
            if near:
                stats["near"] += 1
                if gate:  # gated comparisons skip near-tie rounds; reports compare them too
                    alive.discard(b)
                    continue
            stats["compared"] += 1
            diff = [f for f, ok in (
                ("tokens", list(g_tok[b]) == list(tr.tokens)),
                ("parents", list(g_par[b]) == list(tr.parents)),
                ("mask", np.array_equal(g_mask[b], tr.mask)),
                ("positions", list(g_pos[b]) == list(tr.positions)),
                ("accept_len", g_al[b] == alen), ("bonus", g_bo[b] == bonus),
                ("prefix_len", g_plen[b] == P0 + alen)) if not ok]
            same = not diff
            stats["cmp"].append((min(mmin, min(wm)), same, rd, b))
            # the next root feature is comparable only when the extend consumed the
            # same accepted nodes (indices and tokens) and bonus as the oracle's
            path_same = (g_al[b] == alen and g_bo[b] == bonus
                         and list(g_path[b][:alen]) == list(path[:alen])
                         and all(g_tok[b][i] == tr.tokens[i] for i in path[:alen]))
            fe = rel_l2(g_root[b], states[b].root_feat)
            if path_same:
                stats["feat"].append(fe)
            else:
                stats["path_differs"] += 1
            stats["diffs"].append(diff)
            if gate:
                assert same, (name, rd, b, diff, list(g_tok[b]), list(tr.tokens))
                assert fe <= FEAT_TOL[cfg.dtype], (name, rd, b, fe)
            if same:
                stats["match"] += 1
            else:
                # first flat node where the drafted tree differs, and the oracle's
                # smallest decision margin of the round with its stage
                first = next((i for i in range(cfg.m) if g_tok[b][i] != tr.tokens[i] or g_par[b][i] != tr.parents[i]),
                             None)
                if first is None:  # same tree: the walk decided differently
                    stats["diverged"].append((rd, b, first, min(wm), "verify walk"))
                else:
                    mg_, st_ = _margin_at(info, int(tr.depth[first]))
                    stats["diverged"].append((rd, b, first, mg_, st_))
                alive.discard(b)  # the states have diverged
    return stats


@pytest.mark.parametrize("name", ["tiny", "ragged_f32", "chain_small"])
def test_round_end_to_end_fp32(name):
    say(f"[end-to-end fp32] {name}")
    s = _run_rounds(name, 3, gate=True)
    say(f"  {name}: {s['match']}/{s['compared']} sequence-rounds identical, {s['near']} near-tie, "
        f"worst root feature rel L2 {max(s['feat'], default=0):.2e}")
    assert s["compared"] > 0


BF16_GATE = 4.0  # margin factor over the bf16 logit-error estimate above which a round is gated


@pytest.mark.parametrize("name", ["tiny_bf16", "ragged_bf16", "hd128_bf16", "wide_bf16", "7b", "13b", "70b",
                                  "chain"])
def test_round_end_to_end_bf16_reported(name):
    say(f"[end-to-end bf16, reported] {name}")
    s = _run_rounds(name, 2, gate=False)
    say(f"  {name}: {s['match']}/{s['compared']} sequence-rounds identical to the oracle "
        f"({s['near']} of them with an oracle margin at or below {NEAR}), "
        f"{s['path_differs']} with another accepted path, "
        f"root feature rel L2 max {max(s['feat'], default=0):.2e} (same path); "
        f"bf16 logit-error estimate (largest top-k log-prob change from storing the level-2 "
        f"features in bf16) {s['lerr']:.2e}")
    for rd, b, first, margin, stage in s["diverged"]:
        say(f"    diverged: round {rd} sequence {b}: first differing flat node {first}, oracle's smallest "
            f"margin among the decisions that shape it {margin:.2e} ({stage})")
    # every sequence-round is compared (near-tie ones included), so this is
    # never vacuous; bf16 storage moves logits by more than the near-tie margin,
    # so the drafted tree may differ from the fp64 one, and where the accepted
    # path is the same the extend's next root feature must still agree
    assert s["compared"] >= 1
    assert all(f <= FEAT_TOL["bf16"] for f in s["feat"])
    # where every decision of the round (drafting and the verify walk) clears
    # the bf16 score-noise scale by a wide factor, the round must be the
    # oracle's exactly
    gate = BF16_GATE * s["lerr"]
    clear = [(mg, same, rd, b) for mg, same, rd, b in s["cmp"] if mg > gate]
    say(f"    {len(clear)} sequence-round(s) with every margin above {BF16_GATE} x the logit-error "
        f"estimate ({gate:.2e}): all must match")
    for mg, same, rd, b in clear:
        assert same, (name, rd, b, mg, gate)


# ------------------------------------------------------------------ determinism, data errors

@pytest.mark.parametrize("name", ["ragged_bf16", "7b"])
def test_repeat_runs_are_bit_identical(name):
    cfg, inp, r, model, seqs = get(name)
    say(f"[determinism] {name}")
    outs = []
    for rep in range(2):
        r.reset_state(inp)
        r.run_round()
        sync()
        outs.append([t.cpu().numpy().copy() for t in (r.tokens, r.parents, r.mask, r.logscore,
                                                      r.accept_len, r.bonus, r.prefix_len)]
                    + [to_host(r.root_feat).copy(), r.ws.cpu().numpy().copy()])
    for a, b in zip(*outs[:2]):
        assert np.array_equal(a, b)


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


@pytest.mark.parametrize("name", ["tiny", "ragged_bf16", "hd128_bf16", "wide_bf16", "7b", "70b"])
def test_tree_verify_attention(name):
    """Target-side tree-verify attention through the C ABI against the oracle:
    seeded post-RoPE queries, the tree rows' K/V written right after each
    prefix, ancestor masks of random trees; relative L2 per sequence."""
    import torch
    from eagle_draft_trees_amd import _lib as L
    from eagle_draft_trees_amd.round import to_device
    cfg, inp, r, model, seqs = get(name)
    say(f"[tree verify attention] {name}")
    dt = cfg.dtype
    rng = np.random.default_rng(1000 + cfg.uid)
    B, m, H, Hkv, hd = cfg.B, cfg.m, cfg.H, cfg.Hkv, cfg.hd
    q = rng.normal(size=(B, m, H, hd)).astype(np.float32)
    kc = np.array(inp["k_cache"], copy=True)
    vc = np.array(inp["v_cache"], copy=True)
    P = np.asarray(inp["prefix_len"], np.int32)
    for b in range(B):
        kc[b, P[b]:P[b] + m] = store(rng.normal(size=(m, Hkv, hd)), dt)
        vc[b, P[b]:P[b] + m] = store(rng.normal(size=(m, Hkv, hd)), dt)
    mask = np.stack([_random_tree_mask(rng, m) for _ in range(B)])
    out = torch.zeros(B, m, H * hd, dtype=torch.bfloat16 if dt == "bf16" else torch.float32,
                      device="cuda")
    L.eagle_tree_verify_attention(r.dims, r.tcfg, torch.from_numpy(q).cuda(), to_device(kc, dt, "cuda"),
                                  to_device(vc, dt, "cuda"), to_device(P, dt, "cuda"),
                                  torch.from_numpy(mask).cuda(), out, r.ws)
    sync()
    got = to_host(out)
    worst = 0.0
    for b in (seqs if seqs is not None else range(B)):
        o = O.tree_verify_attention(q[b].astype(np.float64), O.widen(kc[b], dt), O.widen(vc[b], dt),
                                    int(P[b]), mask[b])
        e = rel_l2(got[b], o)
        worst = max(worst, e)
        assert e <= FEAT_TOL[dt], (b, e)
    say(f"  tree verify attention {name}: worst rel L2 {worst:.2e} (tol {FEAT_TOL[dt]})")


@pytest.mark.parametrize("name", ["ragged_bf16", "7b"])
def test_graph_replay_matches_eager(name):
    """A round captured in a HIP graph and replayed several times, each replay
    after the state is reloaded eagerly, gives the eager round's results bit
    for bit every time."""
    import torch
    cfg, inp, r, model, seqs = get(name)
    say(f"[graph replay] {name}")
    snap = lambda: ([t.cpu().numpy().copy() for t in (r.tokens, r.parents, r.mask, r.logscore,
                                                       r.accept_len, r.bonus, r.prefix_len,
                                                       r.root_token)]
                    + [to_host(r.root_feat).copy()])
    r.run_round()
    sync()
    ref = snap()
    stream = torch.cuda.Stream()
    r.reset_state(inp)
    sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        r.run_round(stream=stream)
    sync()
    for rep in range(3):
        r.reset_state(inp)
        sync()
        g.replay()
        sync()
        for a_, b_ in zip(ref, snap()):
            assert np.array_equal(a_, b_), f"replay {rep}"


@pytest.mark.parametrize("name", ["ragged_bf16", "7b"])
def test_timed_level_matches_plain(name):
    """eagle_draft_level_timed drafts the same tree as eagle_draft_level, and the
    events it hands to the LM-head launch bracket a positive time that lies
    inside ordinary events queued around the same call."""
    import torch
    from eagle_draft_trees_amd import _lib as L
    cfg, inp, r, model, seqs = get(name)
    say(f"[timed level] {name}")
    outs = lambda: [t.cpu().numpy().copy() for t in (r.tokens, r.parents, r.mask, r.logscore)]
    r.draft()
    sync()
    ref = outs()
    r.reset_state(inp)
    ev = []
    for level in range(1, cfg.D + 1):
        q = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        for e in q:          # torch creates an event on its first record
            e.record()
        sync()
        q[0].record()
        r.level_timed(level, L.EAGLE_LEVEL_FULL, q[1], q[2])
        q[3].record()
        ev.append(q)
    r.rerank()
    sync()
    for a, b in zip(ref, outs()):
        assert np.array_equal(a, b)
    for m0, k0, k1, m1 in ev:
        assert k0.elapsed_time(k1) > 0
        assert m0.elapsed_time(k0) >= -1e-3 and k1.elapsed_time(m1) >= -1e-3


@pytest.mark.parametrize("name", ["rows64_bf16", "13b", "chain"])
def test_packed_lm_input_matches_in_place(name):
    """At 17..64 bf16 level rows the streaming LM head reads the level's
    features from the copy the down projection's epilogue writes in MFMA
    fragment order; an LM-head-only call (TAIL_ONLY) reads the same features in
    place.  The two must give bit-identical records: drafting every level in
    full, then re-running each level's tail on the features it wrote, builds
    the same tree."""
    from eagle_draft_trees_amd import _lib as L
    cfg, inp, r, model, seqs = get(name)
    say(f"[packed LM input] {name}")
    outs = lambda: [t.cpu().numpy().copy() for t in (r.tokens, r.parents, r.mask, r.logscore)]
    r.draft()
    sync()
    ref = outs()
    r.reset_state(inp)
    r.level(1)
    for level in range(2, cfg.D + 1):
        r.level(level)
        r.level(level, L.EAGLE_LEVEL_TAIL_ONLY)
    r.rerank()
    sync()
    for a, b in zip(ref, outs()):
        assert np.array_equal(a, b)


def test_out_of_range_token_is_clamped_and_flagged():
    import torch
    cfg, inp, r, model, seqs = get("ragged_f32")
    say("[data errors] ragged_f32")
    r.root_token[1] = cfg.V + 5
    sync()
    r.run_round()
    sync()
    err = r.ws_region(0).view(torch.int32)[0].item()
    assert err & 1, err
    assert int(r.tokens[1, 0]) == cfg.V - 1


def test_out_of_range_prefix_is_clamped_and_flagged():
    """A prefix length that leaves no room for the round's rows (above
    max_prefix - m) or that is not positive is clamped to the nearest valid
    one and flagged (error word bit 1); the round still completes, every
    drafted token is a vocabulary id, and the extend advances from the clamped
    length."""
    import torch
    cfg, inp, r, model, seqs = get("ragged_f32")
    say("[data errors] prefix lengths out of range, ragged_f32")
    hi = cfg.max_prefix - cfg.m
    r.ws_region(0).zero_()
    r.prefix_len[0] = 0
    r.prefix_len[2] = cfg.max_prefix
    p1 = int(r.prefix_len[1])
    sync()
    r.run_round()
    sync()
    err = r.ws_region(0).view(torch.int32)[0].item()
    assert err & 2, err
    toks = r.tokens.cpu().numpy()
    assert ((toks >= 0) & (toks < cfg.V)).all()
    alen = [int(x) for x in r.accept_len.cpu()]
    rows = min(cfg.m, cfg.D + 1)
    assert all(1 <= x <= rows for x in alen), alen
    plen = [int(x) for x in r.prefix_len.cpu()]
    assert plen == [1 + alen[0], p1 + alen[1], hi + alen[2]], (plen, alen, hi)
