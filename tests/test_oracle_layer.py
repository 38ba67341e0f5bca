"""CPU pins of the oracle's draft layer and LM-head tail.

Each test holds the oracle to something other than itself: closed forms,
invariants, special cases that reduce to an identity or to a library routine
(torch's CPU attention), or brute force on tiny inputs.
"""
import math

import numpy as np
import pytest
import torch

from oracle import eagle_oracle as O
from tests._tiny import seq_state, tensors, tiny_cfg


# ------------------------------------------------------------------ RoPE (reading R8)

def test_rope_identity_at_zero_and_norm_preserving():
    rng = np.random.default_rng(1)
    x = rng.normal(size=(3, 8))
    assert np.allclose(O.rope(x, 0, 1e4), x, atol=0, rtol=0)
    for p in (1, 7, 513, 4100):
        y = O.rope(x, p, 1e4)
        assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
        assert not np.allclose(y, x)


def test_rope_relative_position_and_composition():
    # <R(p)q, R(p')k> depends only on p - p'; R(a)R(b) = R(a+b)
    rng = np.random.default_rng(2)
    q, k = rng.normal(size=16), rng.normal(size=16)
    for p, pp, s in ((5, 2, 11), (100, 37, 900), (0, 0, 3)):
        a = O.rope(q, p, 1e4) @ O.rope(k, pp, 1e4)
        b = O.rope(q, p + s, 1e4) @ O.rope(k, pp + s, 1e4)
        assert abs(a - b) < 1e-9
    assert np.allclose(O.rope(O.rope(q, 17, 1e4), 40, 1e4), O.rope(q, 57, 1e4), atol=1e-12)


def test_rope_pairs_rotate_half():
    # position 1, dims (i, i+hd/2) form one plane each; the other halves stay zero
    hd = 8
    x = np.zeros(hd)
    x[1] = 1.0
    y = O.rope(x, 1, 1e4)
    nz = set(np.flatnonzero(np.abs(y) > 1e-15))
    assert nz <= {1, 1 + hd // 2} and len(nz) == 2


# ------------------------------------------------------------------ elementwise pieces

def test_silu_and_rmsnorm_closed_forms():
    x = np.linspace(-6, 6, 25)
    assert np.allclose(O.silu(x) - O.silu(-x), x, atol=1e-12)  # x*sig(x) - (-x)*sig(-x) = x
    assert O.silu(np.array([0.0]))[0] == 0.0
    rng = np.random.default_rng(3)
    y = rng.normal(size=(4, 32))
    g = 1 + rng.normal(0, .1, 32)
    z = O.rms_norm(y, np.ones(32), 0.0)
    assert np.allclose(np.sqrt(np.mean(z * z, axis=-1)), 1.0)
    assert np.allclose(O.rms_norm(7.5 * y, g, 0.0), O.rms_norm(y, g, 0.0))
    assert np.allclose(O.rms_norm(y, g, 0.0), z * g)
    tiny = np.full((1, 4), 1e-4)
    assert np.allclose(O.rms_norm(tiny, np.ones(4), 1e-6), 1e-4 / math.sqrt(1e-8 + 1e-6))


# ------------------------------------------------------------------ attention

def _sdpa(q, keys, vals):
    H, hd = q.shape
    g = H // keys.shape[1]
    kt = torch.from_numpy(np.repeat(keys, g, axis=1)).permute(1, 0, 2)  # [H, N, hd]
    vt = torch.from_numpy(np.repeat(vals, g, axis=1)).permute(1, 0, 2)
    qt = torch.from_numpy(q)[:, None, :]  # [H, 1, hd]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)
    return o[:, 0, :].reshape(-1).numpy()


@pytest.mark.parametrize("H,Hkv,hd,N", [(2, 2, 4, 5), (4, 2, 8, 9), (6, 1, 16, 33)])
def test_attend_row_matches_library_attention(H, Hkv, hd, N):
    rng = np.random.default_rng(H * 100 + N)
    q = rng.normal(size=(H, hd))
    keys, vals = rng.normal(size=(N, Hkv, hd)), rng.normal(size=(N, Hkv, hd))
    assert np.allclose(O.attend_row(q, keys, vals), _sdpa(q, keys, vals), atol=1e-12)


def test_attend_row_single_key_and_gqa_grouping():
    rng = np.random.default_rng(5)
    q = rng.normal(size=(4, 8))
    keys, vals = rng.normal(size=(1, 2, 8)), rng.normal(size=(1, 2, 8))
    out = O.attend_row(q, keys, vals).reshape(4, 8)
    assert np.allclose(out[:2], vals[0, 0]) and np.allclose(out[2:], vals[0, 1])
    keys, vals = rng.normal(size=(6, 2, 8)), rng.normal(size=(6, 2, 8))
    base = O.attend_row(q, keys, vals).reshape(4, 8)
    vals2 = vals.copy()
    vals2[:, 1] += 3.0
    pert = O.attend_row(q, keys, vals2).reshape(4, 8)
    assert np.allclose(pert[:2], base[:2]) and not np.allclose(pert[2:], base[2:])


# ------------------------------------------------------------------ draft layer special cases

def test_fc_input_is_feature_then_next_token_embedding():
    # [P1] §4.1: input = [f_j || e(t_{j+1})]; feature first, then the embedding
    cfg = tiny_cfg()
    rng = np.random.default_rng(6)
    d = cfg.d
    eye, zero = np.eye(d), np.zeros((d, d))
    feats = rng.normal(size=(3, d))
    toks = [1, 5, 11]
    for fc, want in ((np.hstack([eye, zero]), feats),
                     (np.hstack([zero, eye]), None)):
        m = O.Model(cfg, tensors(cfg, rng, fc_w=fc, fc_b=np.zeros(d)))
        x0, _, _, _ = O.draft_rows(m, feats.astype(np.float32).astype(np.float64), toks, [0, 0, 0])
        w = m.embed_rows(toks) if want is None else feats.astype(np.float32)
        assert np.allclose(x0, w, atol=1e-6)
    m = O.Model(cfg, tensors(cfg, rng, fc_w=np.zeros((d, 2 * d))))
    x0, _, _, _ = O.draft_rows(m, feats, toks, [0, 0, 0])
    assert np.allclose(x0, m.w("fc_b")[None, :])


def test_first_input_norm_is_identity_and_v_is_not_rotated():
    # [P3]: the first layer's input_layernorm is replaced by the identity
    cfg = tiny_cfg()
    d = cfg.d
    rng = np.random.default_rng(7)
    t = tensors(cfg, rng, fc_w=np.hstack([np.eye(d), np.zeros((d, d))]), fc_b=np.zeros(d),
                wq=np.eye(d))
    m = O.Model(cfg, t)
    feats = 5.0 * rng.normal(size=(2, d)).astype(np.float32).astype(np.float64)
    x0, q, k0, v0 = O.draft_rows(m, feats, [0, 1], [0, 0])
    assert np.allclose(q.reshape(2, d), feats, atol=1e-12)  # not normalised
    _, q9, k9, v9 = O.draft_rows(m, feats, [0, 1], [9, 9])
    assert np.allclose(v9, v0) and not np.allclose(k9, k0)
    for r in range(2):
        assert np.allclose(k9[r], O.rope(k0[r], 9, cfg.rope_theta))


def test_residuals_and_no_final_norm():
    cfg = tiny_cfg()
    d = cfg.d
    rng = np.random.default_rng(8)
    m = O.Model(cfg, tensors(cfg, rng, wo=np.eye(d), w_down=np.zeros((d, cfg.F))))
    x0, attn = rng.normal(size=(3, d)), rng.normal(size=(3, d))
    assert np.allclose(O.finish_rows(m, x0, attn), x0 + attn, atol=1e-12)


def test_swiglu_closed_form_with_gain():
    cfg = tiny_cfg(F=8)
    d = cfg.d
    rng = np.random.default_rng(9)
    t = tensors(cfg, rng, wo=np.zeros((d, d)), w_gate=np.eye(d), w_up=2 * np.eye(d),
                w_down=np.eye(d))
    m = O.Model(cfg, t)
    x0 = rng.normal(size=(2, d))
    g = m.w("post_norm")
    z = x0 / np.sqrt(np.mean(x0 ** 2, axis=1, keepdims=True) + cfg.rms_eps) * g
    want = x0 + (z / (1 + np.exp(-z))) * (2 * z)
    assert np.allclose(O.finish_rows(m, x0, np.zeros((2, d))), want, atol=1e-12)


# ------------------------------------------------------------------ LM-head tail

def _brute_tail(W, h, k):
    V, d = len(W), len(h)
    z = [sum(W[v][i] * h[i] for i in range(d)) for v in range(V)]
    mx = max(z)
    lse = mx + math.log(sum(math.exp(x - mx) for x in z))
    left = list(range(V))
    ids = []
    for _ in range(k):
        best = left[0]
        for v in left[1:]:
            if z[v] > z[best]:
                best = v  # strict: the lowest id wins a tie
        ids.append(best)
        left.remove(best)
    return ids, [z[i] - lse for i in ids]


@pytest.mark.parametrize("k", [1, 3, 7])
def test_tail_matches_brute_force(k):
    cfg = tiny_cfg(V=37, d=6, H=2, Hkv=2, hd=3)
    rng = np.random.default_rng(10 + k)
    t = tensors(cfg, rng)
    m = O.Model(cfg, t)
    h = rng.normal(size=cfg.d)
    ids, logp, _ = O.lm_tail(m, h, k)
    W = m.w("lm_head").tolist()
    bids, blogp = _brute_tail(W, h.tolist(), k)
    assert list(ids) == bids
    assert np.allclose(logp, blogp, atol=1e-12)


def test_tail_ties_normalisation_and_margin():
    cfg = tiny_cfg(V=9, d=4)
    rng = np.random.default_rng(11)
    lm = rng.normal(size=(9, 4))
    h = np.array([1.0, 0.5, -0.25, 2.0])
    top = int(np.argmax(lm @ h))
    lm[7] = lm[top]  # exact tie at the maximum
    lo, hi = min(top, 7), max(top, 7)
    m = O.Model(cfg, tensors(cfg, rng, lm_head=lm))
    ids, logp, margin = O.lm_tail(m, h, 2)
    assert list(ids) == [lo, hi] and margin == 0.0
    ids, logp, _ = O.lm_tail(m, h, 9)
    assert abs(np.exp(logp).sum() - 1.0) < 1e-12
    assert np.all(np.diff(logp) <= 0)
