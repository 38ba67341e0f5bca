"""CPU pins of the oracle's level forward (``level_step_forward``): the
position a tree row is rotated at and the set of keys it attends.

* At topk = 1 the tree is a chain, its ancestor-only mask is the causal mask,
  and drafting the chain level by level must give what one causal pass over
  the same rows gives ([P1] §12 item 5: the tree mask sees only ancestors and
  positions are shared per level; [P3] "在 SGLang 里": the extend reruns the
  accepted positions causally).  ``draft_extend`` is pinned to library
  attention with a causal mask, so this ties the levels' position P-1+depth
  and their key set (prefix, ancestors, self) to it.
* At topk > 1 every forwarded row is recomputed from scratch with library
  primitives: torch linear layers, RoPE as a complex rotation, the mask
  derived from the pool's parent pointers (not from the frontier's ancestor
  slots) and torch's scaled_dot_product_attention.
"""
import copy

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

from oracle import eagle_oracle as O
from tests._tiny import seq_state, tensors, tiny_cfg


def _levels(model, st, D, k):
    pool, F, _ = O.level_one(model, st, k)
    frontiers, feats, intree = [F], {}, {}
    for level in range(2, D + 1):
        h = O.level_step_forward(model, st, level, F, feats, intree)
        F, _, _ = O.level_step_tail(model, level, F, h, pool, k)
        frontiers.append(F)
    return pool, frontiers, feats, intree


@pytest.mark.parametrize("D,H,Hkv,P", [(5, 2, 2, 3), (6, 4, 2, 7), (4, 4, 1, 1)])
def test_chain_levels_equal_one_causal_pass(D, H, Hkv, P):
    # topk = 1: level L forwards the depth-(L-1) node c with row
    # [feature of c's parent || e(token of c)].  Over the chain root -> c1 -> ...
    # this is the causal extend whose rows carry the drafted features as the
    # "true" ones: extend row i = [h_i || e(t_{i+1})] at position P+i sees the
    # prefix and rows 0..i, which is what the level of depth i+1 sees
    # (prefix, its ancestors, itself) at position P-1+(i+1).
    cfg = tiny_cfg(D=D, k=1, V=17, m=D, H=H, Hkv=Hkv, hd=4, d=4 * H, F=10, P_lo=P, P_hi=P)
    rng = np.random.default_rng(300 + D)
    model = O.Model(cfg, tensors(cfg, rng, scale=0.3))
    st = seq_state(cfg, rng)
    st_ext = copy.deepcopy(st)
    pool, frontiers, feats, intree = _levels(model, st, D, 1)
    toks = [F[0].token for F in frontiers]                      # t_1 .. t_D
    a = D - 2                                                  # extend rows 0..D-2
    tokens = np.array([st.root_token] + toks[:a], dtype=np.int64)
    true_feat = np.stack([st.root_feat] + [feats[(i, 0)] for i in range(1, a + 1)])
    h, kn, vn = O.draft_extend(model, st_ext, true_feat, tokens, list(range(a + 1)),
                               bonus=toks[a])
    for i in range(a + 1):
        assert np.allclose(h[i], feats[(i + 1, 0)], rtol=1e-12, atol=1e-12), i
        kk, vv = intree[(i + 1, 0)]
        assert np.allclose(kn[i], kk, rtol=1e-12, atol=1e-12), i
        assert np.allclose(vn[i], vv, rtol=1e-12, atol=1e-12), i


def _chain_matches_extend(model, st, D):
    pool, frontiers, feats, intree = _levels(model, copy.deepcopy(st), D, 1)
    toks = [F[0].token for F in frontiers]
    a = D - 2
    tokens = np.array([st.root_token] + toks[:a], dtype=np.int64)
    true_feat = np.stack([st.root_feat] + [feats[(i, 0)] for i in range(1, a + 1)])
    h, _, _ = O.draft_extend(model, copy.deepcopy(st), true_feat, tokens, list(range(a + 1)),
                             bonus=toks[a])
    return all(np.allclose(h[i], feats[(i + 1, 0)], rtol=1e-9, atol=1e-9) for i in range(a + 1))


def test_chain_pin_catches_planted_mistakes(monkeypatch):
    # plant plausible mistakes in the oracle's level forward (on the CPU) and check
    # that the chain equality above no longer holds: a level position one off,
    # and the row's own in-tree key dropped from its visible set
    cfg = tiny_cfg(D=5, k=1, V=17, m=5, H=2, Hkv=2, hd=4, d=8, F=10, P_lo=5, P_hi=5)
    rng = np.random.default_rng(311)
    model = O.Model(cfg, tensors(cfg, rng, scale=0.3))
    st = seq_state(cfg, rng)
    assert _chain_matches_extend(model, st, cfg.D)

    real_fwd = O.level_step_forward
    real_rows = O.draft_rows

    def fwd_pos_plus_one(*args, **kw):
        monkeypatch.setattr(O, "draft_rows",
                            lambda m_, f_, t_, pos: real_rows(m_, f_, t_, [p + 1 for p in pos]))
        try:
            return real_fwd(*args, **kw)
        finally:
            monkeypatch.setattr(O, "draft_rows", real_rows)

    monkeypatch.setattr(O, "level_step_forward", fwd_pos_plus_one)
    assert not _chain_matches_extend(model, st, cfg.D)
    monkeypatch.setattr(O, "level_step_forward", real_fwd)

    real_vis = O._visible_kv

    def without_self(st_, intree, node):
        ks, vs = real_vis(st_, intree, node)
        return ks[:-1], vs[:-1]

    monkeypatch.setattr(O, "_visible_kv", without_self)
    assert not _chain_matches_extend(model, st, cfg.D)


def _rope_complex(x, pos, theta):
    # rotate-half pairs (i, i+hd/2) as the complex number x_i + j*x_{i+hd/2},
    # turned by pos * theta^(-2i/hd)
    hd = x.shape[-1]
    half = hd // 2
    z = torch.complex(x[..., :half], x[..., half:])
    i = torch.arange(half, dtype=torch.float64)
    w = torch.polar(torch.ones(half, dtype=torch.float64), pos * theta ** (-2.0 * i / hd))
    r = z * w
    return torch.cat([r.real, r.imag], dim=-1)


@pytest.mark.parametrize("D,k,H,Hkv,P", [(4, 3, 2, 2, 5), (3, 4, 4, 2, 6), (5, 2, 4, 1, 2)])
def test_level_rows_match_library_layer_with_pool_ancestor_mask(D, k, H, Hkv, P):
    cfg = tiny_cfg(D=D, k=k, V=29, m=4, H=H, Hkv=Hkv, hd=4, d=4 * H, F=12, P_lo=P, P_hi=P)
    rng = np.random.default_rng(400 + 10 * D + k)
    raw = tensors(cfg, rng, scale=0.45)
    model = O.Model(cfg, raw)
    st = seq_state(cfg, rng)
    pool, frontiers, feats, _ = _levels(model, st, D, k)

    T = {n: torch.from_numpy(np.asarray(v, dtype=np.float64)) for n, v in raw.items()}
    Kp = torch.from_numpy(st.K[:P])
    Vp = torch.from_numpy(st.V[:P])
    g = H // Hkv
    theta, eps = cfg.rope_theta, cfg.rms_eps
    h_of = {-1: torch.from_numpy(st.root_feat)}   # pool index -> this test's feature
    kv_of = {}                                     # pool index -> (k, v) of its tree row
    for dd in range(1, D):                         # rows forwarded at level dd+1
        F = frontiers[dd - 1]
        pidx = [x.pool_idx for x in F]
        par = [pool[i].parent for i in pidx]
        u = torch.stack([torch.cat([h_of[pp], T["embed"][pool[i].token]])
                         for i, pp in zip(pidx, par)])
        x0 = Fn.linear(u, T["fc_w"], T["fc_b"])
        q = _rope_complex(Fn.linear(x0, T["wq"]).view(-1, H, 4), P - 1 + dd, theta)
        kk = _rope_complex(Fn.linear(x0, T["wk"]).view(-1, Hkv, 4), P - 1 + dd, theta)
        vv = Fn.linear(x0, T["wv"]).view(-1, Hkv, 4)
        for r, i in enumerate(pidx):
            kv_of[i] = (kk[r], vv[r])
        tree_nodes = sorted(kv_of)                 # every tree row written so far
        keys = torch.cat([Kp, torch.stack([kv_of[i][0] for i in tree_nodes])])
        vals = torch.cat([Vp, torch.stack([kv_of[i][1] for i in tree_nodes])])
        mask = torch.zeros(len(pidx), P + len(tree_nodes), dtype=torch.bool)
        mask[:, :P] = True
        for r, i in enumerate(pidx):
            chain, j = set(), i
            while j != -1:                         # ancestor-or-self by parent pointers
                chain.add(j)
                j = pool[j].parent
            for c, n in enumerate(tree_nodes):
                mask[r, P + c] = n in chain
        o = Fn.scaled_dot_product_attention(
            q.permute(1, 0, 2), keys.repeat_interleave(g, dim=1).permute(1, 0, 2),
            vals.repeat_interleave(g, dim=1).permute(1, 0, 2), attn_mask=mask)
        attn = o.permute(1, 0, 2).reshape(len(pidx), -1)
        y = x0 + Fn.linear(attn, T["wo"])
        z = y * torch.rsqrt((y * y).mean(-1, keepdim=True) + eps) * T["post_norm"]
        h = y + Fn.linear(Fn.silu(Fn.linear(z, T["w_gate"])) * Fn.linear(z, T["w_up"]),
                          T["w_down"])
        for r, i in enumerate(pidx):
            h_of[i] = h[r]
            assert np.allclose(feats[(dd, r)], h[r].numpy(), rtol=1e-11, atol=1e-11), (dd, r)
