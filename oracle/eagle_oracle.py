"""fp64 CPU oracle for one round of EAGLE feature-level drafting with EAGLE-2
dynamic draft trees.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or run this module.  It shares no
code, header, table or helper with the HIP library; its inputs come from the
seeded generator (``synth``) or from the oracle's own earlier stages.

Sources (cited by title and section throughout):
  [P1] "EAGLE 推测解码为什么比 Medusa 快？（含 EAGLE-2 动态草稿树）" (study notes)
  [P2] "(EAGLE 1)EAGLE: Speculative Sampling Requires Rethinking Feature Uncertainty"
       (paper-reading notes)
  [P3] Medusa -> EAGLE -> EAGLE-2 blog notes, zdszero.github.io "spec_medusa_eagle"
  [P4] "投机解码：从eagle1到dflash" (news article; EAGLE-2 flow diagram)

What one round computes (readings where the pages are silent are marked R#):
  * Level 1 is only the LM-head tail on the root's draft feature, because
    the first level's top-k comes from the previous round's draft extend
    ([P3] section "在 SGLang 里").
  * Levels 2..D run the draft head on the k frontier nodes: the row of node x
    is [feature of x's parent || embedding of x's token] ([P1] §4.1 input
    equation; [P2] Core Idea), FC 2d->d with bias, one Llama decoder layer
    whose first input norm is the identity and which has no final norm
    ([P3] "在 SGLang 里"), then the frozen LM head, softmax and top-k.
  * A node's value is the product of draft probabilities along its root
    path ([P1] §10.3 value equation); it is kept here as a sum of
    log-probabilities.  Each level keeps the best k of the k*k children
    ([P1] §10.3 expansion; [P3] select_top_k_tokens).
  * After the last level every scored candidate competes in the rerank;
    the best m-1 join the root (R3: m counts the root, as SGLang's
    num_draft_tokens does, [P3]).  Ties prefer the shallower node ([P1]
    §10.3 property 2).
  * The tree is flattened (root, then depth-major, then by parent's flat
    index, then child rank; [P4] EAGLE-2 diagram), with an ancestor-only
    mask and per-depth positions ([P1] §12 item 5).
  * Greedy verification walks from the root while the target's argmax token
    is a child of the current node; the argmax at the stop is the bonus
    token ([P4] EAGLE-2 diagram: accept the longest path, back off to the
    last accepted node).
  * The draft extend reruns the draft head over the accepted path with the
    target's true features and appends the draft KV ([P3] "在 SGLang 里";
    [P2] Core Idea; [P1] §6.2 and §12 item 3).

Readings of what the pages leave open:
  R1  round = level-1 tail + (D-1) forwards + rerank/build + verify + extend.
  R2  shift direction: the feature is paired with the NEXT token's embedding
      ([P1] §4.1, [P3]); [P4]'s "e_{t-1}" is read as garbled.
  R3  m includes the root.
  R4  every scored candidate (k + (D-1)k^2) competes in the rerank.
  R5  confidence = softmax probability at temperature 1.
  R6  ties: top-k by (logit desc, id asc); k*k->k by (score desc, pool index
      asc); rerank by (score desc, depth asc, pool index asc).
  R7  flatten order as above.
  R8  position of a node at depth L is P-1+L (the root row is the last of the
      P prefix rows); RoPE theta = 10000, rotate-half pairs (i, i+hd/2).
  R9  RMSNorm eps = 1e-6; no biases except the FC; scale 1/sqrt(hd); SiLU;
      GQA head h reads KV head h // (H/Hkv).
  R10 extend row i (i = 0..accept_len-1) carries [true feature of path node
      i || embedding of path node i+1 (or the bonus for the last row)] at
      position P+i, attends the prefix and extend rows 0..i only.
  R11 accept_len counts the root, i.e. accepted drafts + 1 (the bonus);
      this is the E[N] = 1 + ... convention of [P1] §8.
  R12 greedy verification (argmax, lowest id on exact ties).
  R13 exactly one decoder layer.
  R14 target-side tree verify (the next step after the round, [P1] §6.2,
      [P4] EAGLE-2 diagram stage two): the tree tokens' keys and values sit in
      the target's cache right after the prefix, in flat order; query i sees
      every prefix row and tree row j iff mask[i, j] is set.
  R15 relaxed acceptance (the SGLang variant in [P2]'s closing notes: target
      probabilities and a probability threshold decide acceptance, and only
      when every candidate of a level fails is one rejection-sampling draw
      made there for the bonus): at node x, p = softmax(target logits / T);
      x's children are tried in flat order and the walk descends to the first
      child c with p(c) >= threshold.  When none passes (or x is a leaf) the
      bonus is drawn from the residual: p with x's children removed and the
      rest renormalised (rejection sampling with the rejected candidates as
      point-mass proposals), by inverse CDF over token ids with one uniform
      u in [0, 1) supplied per sequence.  If the children hold all of p's
      mass the draw is from p itself.
  R17 strict verification by recursive rejection sampling ([P1] §6.2): at
      node x, p = softmax(target logits / T) and q = softmax(draft logits / T)
      (the draft's distribution at x, supplied by the caller as logits at
      every tree node); x's children are tried in flat order, child c
      accepted iff p(t_c) > 0 and u_c * q(t_c) <= p(t_c), i.e. u_c <=
      min(1, p/q) (u_c the uniform of flat node c; a token without target
      mass is never accepted, whatever q is); after each rejection
      p <- norm(max(0, p - q)); when every child is rejected (or x is a leaf)
      the bonus is drawn from the current p by inverse CDF with the
      sequence's last uniform.  If max(0, p - q) has no mass, p is kept.
      Lossless when the children were drawn from q (a sampled tree).
  R18 strict verification of deterministic candidates ([P1] §6.2 read with
      each drafted child as a point-mass proposal, since EAGLE-2's top-k
      children and a static template's are a fixed list, not draws from q;
      accepting a point mass at t with probability min(1, p(t)/1) and
      resampling from norm(max(0, p - delta_t)) is the same rule): at node x
      the children are tried in flat order, child c accepted iff u_c <= r(t_c)
      with r = p less the tokens rejected so far, renormalised; a rejection
      removes t_c from r; at the stop the bonus is drawn from r by inverse CDF
      (p with x's children removed, as in R15's draw).  R17's rule is kept for
      trees whose children were sampled from q.
  R16 static tree (EAGLE-1 / Medusa, [P1] §10.1: a fixed-shape tree with a
      fixed number of candidates per level, its shape set once for every
      input; [P3]: EAGLE-1 drafts on one static tree): a template of k slots
      per depth.  Depth 1 is the root's top-k in rank order; slot j of depth
      L >= 2 is the child of rank rank[L][j] (in the parent's top-k order) of
      slot parent[L][j] of depth L-1.  The draft forward, LM head and top-k
      are those of the dynamic tree; the tree is every template node, root
      first, then depth-major, then slot order (its first m nodes).

Parity pins: every function below is pinned by a CPU test (tests/
test_oracle_*.py) against brute force, closed forms, special cases or the
pages' worked numbers.  The layer's absolute values at random weights have
no printed example on the pages; they are pinned through special cases
(zeroed sublayers, identity FC, single-key attention, library attention
under an equivalent mask) rather than end to end.  The level forward
(level_step_forward: R8's position P-1+depth and the visible keys prefix,
ancestors and self) is pinned two ways in tests/test_oracle_level.py: at
topk = 1 the levels over a chain equal one causal pass of the layer over
the same rows (draft_extend, itself pinned to library causal attention),
and at any topk the level rows equal a library layer under a mask built in
the test from the pool's parent links.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "widen", "Model", "SeqState", "PoolEntry", "FrontierNode", "rope", "rms_norm", "silu",
    "attend_row", "draft_rows", "finish_rows", "lm_logits", "lm_tail", "level_one",
    "level_step_forward", "level_step_tail", "rerank", "build_tree", "verify_greedy",
    "draft_extend", "run_round", "RoundResult", "NEAR_TIE", "tree_verify_attention",
    "target_probs", "sample_residual", "verify_relaxed", "level_step_tail_static",
    "build_static_tree", "verify_rejection", "verify_rejection_topk",
]

NEAR_TIE = 1e-3  # a selection whose margin (log domain) is below this is "near-tie"


# --------------------------------------------------------------------------- storage

def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of stored data: bf16 bit patterns (uint16) or float32."""
    if dtype == "bf16":
        a = np.ascontiguousarray(a, dtype=np.uint16)
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


class Model:
    """Draft-head weights plus the frozen target embedding and LM head.

    Draft head = FC(2d->d, bias) + one Llama decoder layer; embedding and LM
    head are the target's, shared and frozen ([P1] §4.1 components; [P3]
    draft structure).  Values are widened to fp64 on first use.
    """

    _CACHE_LIMIT = 1 << 28  # elements; larger matrices are widened in row blocks

    def __init__(self, cfg, tensors: Dict[str, np.ndarray]):
        self.cfg = cfg
        self.dtype = cfg.dtype
        self.raw = {n: tensors[n] for n in ("fc_w", "fc_b", "wq", "wk", "wv", "wo",
                                            "post_norm", "w_gate", "w_up", "w_down",
                                            "embed", "lm_head")}
        self._w: Dict[str, np.ndarray] = {}

    def w(self, name: str) -> np.ndarray:
        if name not in self._w:
            self._w[name] = widen(self.raw[name], self.dtype)
        return self._w[name]

    def linear(self, name: str, x: np.ndarray) -> np.ndarray:
        """x @ W^T for a [N][K] weight (the Linear convention)."""
        raw = self.raw[name]
        if raw.size <= self._CACHE_LIMIT:
            return x @ self.w(name).T
        n = raw.shape[0]
        out = np.empty(x.shape[:-1] + (n,), dtype=np.float64)
        step = max(1, (1 << 24) // raw.shape[1])
        for r0 in range(0, n, step):
            out[..., r0:r0 + step] = x @ widen(raw[r0:r0 + step], self.dtype).T
        return out

    def embed_rows(self, tokens: Sequence[int]) -> np.ndarray:
        return widen(self.raw["embed"][np.asarray(tokens, dtype=np.int64)], self.dtype)


@dataclasses.dataclass
class SeqState:
    """Per-sequence decoding state: the draft's prefix KV (post-RoPE, rows
    0..P-1, the last being the root row), the root's draft feature and the
    root token."""
    K: np.ndarray          # [P, Hkv, hd] fp64
    V: np.ndarray          # [P, Hkv, hd] fp64
    P: int
    root_feat: np.ndarray  # [d] fp64
    root_token: int


@dataclasses.dataclass
class PoolEntry:
    score: float       # log value: sum of log-probabilities along the root path
    logp: float        # this node's own draft log-probability
    token: int
    parent: int        # pool index of the parent, -1 for children of the root
    depth: int
    pslot: int         # frontier slot of the parent at its level, -1 for the root


@dataclasses.dataclass
class FrontierNode:
    token: int
    score: float
    pool_idx: int
    pslot: int                 # frontier slot of the parent (-1: the root)
    anc: Tuple[int, ...]       # frontier slot of the ancestor at depth 1..self


# --------------------------------------------------------------------------- layer pieces

def rope(x: np.ndarray, pos: float, theta: float) -> np.ndarray:
    """Rotary embedding of one head vector (or a stack of them) at position
    ``pos``: rotate-half pairs (i, i+hd/2) by angle pos * theta^(-2i/hd).
    The pages fix only that the position is shared per tree level ([P1] §12
    item 5); the base and pairing are reading R8."""
    hd = x.shape[-1]
    half = hd // 2
    i = np.arange(half, dtype=np.float64)
    ang = float(pos) * np.power(float(theta), -2.0 * i / hd)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def rms_norm(y: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    return y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps) * g


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def attend_row(q: np.ndarray, keys: np.ndarray, vals: np.ndarray) -> np.ndarray:
    """Softmax attention of one query row over an explicit list of visible
    keys.  q [H, hd]; keys/vals [N, Hkv, hd]; returns [H*hd].  Head h reads
    KV head h // (H/Hkv) (R9)."""
    H, hd = q.shape
    Hkv = keys.shape[1]
    g = H // Hkv
    out = np.empty((H, hd), dtype=np.float64)
    for h in range(H):
        kv = h // g
        s = keys[:, kv, :] @ q[h] / math.sqrt(hd)
        s = s - s.max()
        p = np.exp(s)
        p /= p.sum()
        out[h] = p @ vals[:, kv, :]
    return out.reshape(H * hd)


def draft_rows(model: Model, feats: np.ndarray, tokens: Sequence[int],
               positions: Sequence[float]):
    """Input fusion, FC and the QKV projections of the draft layer.

    Row r is u_r = [feats[r] || e(tokens[r])] ([P1] §4.1 input equation;
    [P2] Core Idea: 2d-wide fused sequence), x0 = W_fc u + b ([P3]: FC with
    bias).  The first decoder layer's input norm is the identity ([P3]), so
    q/k/v project x0 directly; q and k are rotated at the row's position.
    Returns x0 [R,d], q [R,H,hd], k [R,Hkv,hd], v [R,Hkv,hd].
    """
    c = model.cfg
    u = np.concatenate([np.asarray(feats, dtype=np.float64), model.embed_rows(tokens)], axis=1)
    x0 = model.linear("fc_w", u) + model.w("fc_b")
    q = model.linear("wq", x0).reshape(-1, c.H, c.hd)
    k = model.linear("wk", x0).reshape(-1, c.Hkv, c.hd)
    v = model.linear("wv", x0).reshape(-1, c.Hkv, c.hd)
    for r, p in enumerate(positions):
        q[r] = rope(q[r], p, c.rope_theta)
        k[r] = rope(k[r], p, c.rope_theta)
    return x0, q, k, v


def finish_rows(model: Model, x0: np.ndarray, attn: np.ndarray,
                parts: Optional[dict] = None) -> np.ndarray:
    """Rest of the Llama decoder layer: output projection with the residual
    on x0, post-attention RMSNorm, SwiGLU MLP with its residual.  No final
    norm ([P3]).  Returns the predicted feature rows [R, d]; ``parts`` (if
    given) receives the post-attention stream y."""
    c = model.cfg
    y = x0 + model.linear("wo", attn)
    if parts is not None:
        parts["y"] = y
    z = rms_norm(y, model.w("post_norm"), c.rms_eps)
    a = silu(model.linear("w_gate", z)) * model.linear("w_up", z)
    return y + model.linear("w_down", a)


def lm_logits(model: Model, h: np.ndarray) -> np.ndarray:
    """Frozen target LM head on draft features ([P1] §4.1: draft
    distribution = LM_Head(f-hat))."""
    return model.linear("lm_head", np.atleast_2d(h))


def lm_tail(model: Model, h: np.ndarray, k: int):
    """Top-k of softmax(LM_Head(h)) for one feature row.

    Returns (ids[k], logp[k], margin): ids ordered by (logit desc, id asc),
    logp = logit - logsumexp(logits), and the smallest gap among the first
    k+1 sorted logits (inf when V == k).  [P1] §4.1 draft distribution;
    [P2] Core Idea; EAGLE-2 keeps the top-k instead of sampling ([P3]).
    """
    z = lm_logits(model, h)[0]
    mx = z.max()
    lse = mx + math.log(np.exp(z - mx).sum())
    order = np.lexsort((np.arange(z.size), -z))
    ids = order[:k]
    top = z[order[:k + 1]]
    margin = float(np.min(top[:-1] - top[1:])) if top.size > k else math.inf
    return ids.astype(np.int64), z[ids] - lse, margin


# --------------------------------------------------------------------------- tree levels

def _order_key_select(e: PoolEntry, idx: int):
    return (-e.score, idx)


def level_one(model: Model, st: SeqState, k: int):
    """Level 1: LM-head tail on the root's draft feature; its k children
    enter the pool and all of them form the first frontier ([P3] "在 SGLang
    里": the first level's top-k comes from the previous extend)."""
    ids, logp, margin = lm_tail(model, st.root_feat, k)
    pool = [PoolEntry(float(lp), float(lp), int(t), -1, 1, -1) for t, lp in zip(ids, logp)]
    order = sorted(range(len(pool)), key=lambda i: _order_key_select(pool[i], i))
    frontier = [FrontierNode(pool[i].token, pool[i].score, i, -1, (j,))
                for j, i in enumerate(order)]
    return pool, frontier, {"tail": [margin], "select": [math.inf]}


def _visible_kv(st: SeqState, intree: Dict[Tuple[int, int], Tuple[np.ndarray, np.ndarray]],
                node: FrontierNode):
    """Keys a tree row sees: every prefix row, then the in-tree rows of its
    ancestors and itself, never a sibling or cousin (ancestor-only mask,
    [P1] §12 item 5; [P4] EAGLE-2 diagram)."""
    ks = [st.K[:st.P]]
    vs = [st.V[:st.P]]
    for depth, slot in enumerate(node.anc, start=1):
        kk, vv = intree[(depth, slot)]
        ks.append(kk[None])
        vs.append(vv[None])
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def level_step_forward(model: Model, st: SeqState, level: int,
                       frontier: List[FrontierNode],
                       feats: Dict[Tuple[int, int], np.ndarray],
                       intree: Dict[Tuple[int, int], Tuple[np.ndarray, np.ndarray]],
                       parts: Optional[dict] = None):
    """Draft forward of level ``level`` >= 2 over the frontier of depth
    level-1.  Node x's row pairs its parent's draft feature with x's own
    token and sits at position P-1+depth(x) (R8).  Writes in-tree K/V for
    slot (level-1, j) and the predicted features feats[(level-1, j)].
    ``parts`` (if given) receives the rows' intermediates x0, attn and y."""
    c = model.cfg
    depth = level - 1
    pf = np.stack([st.root_feat if depth == 1 else feats[(depth - 1, x.pslot)]
                   for x in frontier])
    toks = [x.token for x in frontier]
    pos = [st.P - 1 + depth] * len(frontier)
    x0, q, kn, vn = draft_rows(model, pf, toks, pos)
    for j in range(len(frontier)):
        intree[(depth, j)] = (kn[j], vn[j])
    attn = np.stack([attend_row(q[j], *_visible_kv(st, intree, x))
                     for j, x in enumerate(frontier)])
    if parts is not None:
        parts["x0"], parts["attn"] = x0, attn
    h = finish_rows(model, x0, attn, parts)
    for j in range(len(frontier)):
        feats[(depth, j)] = h[j]
    return h


def level_step_tail(model: Model, level: int, frontier: List[FrontierNode],
                    h_rows: np.ndarray, pool: List[PoolEntry], k: int):
    """Tail of level >= 2: each frontier node's top-k children get score =
    parent score + log p ([P1] §10.3 value as a product along the path;
    [P3] select_top_k_tokens multiplies the running score by this level's
    probabilities).  All k*k children join the pool in (frontier slot,
    child rank) order; the best k by (score desc, pool index asc) form the
    next frontier ([P1] §10.3 expansion)."""
    base = len(pool)
    assert base == k + (level - 2) * k * k
    tails = []
    for j, x in enumerate(frontier):
        ids, logp, margin = lm_tail(model, h_rows[j], k)
        tails.append(margin)
        for t, lp in zip(ids, logp):
            pool.append(PoolEntry(x.score + float(lp), float(lp), int(t), x.pool_idx, level, j))
    cand = list(range(base, len(pool)))
    cand.sort(key=lambda i: _order_key_select(pool[i], i))
    nxt = []
    for j2, i in enumerate(cand[:k]):
        e = pool[i]
        nxt.append(FrontierNode(e.token, e.score, i, e.pslot, frontier[e.pslot].anc + (j2,)))
    # membership and order of the new frontier hang on the gaps among the
    # best k+1 candidate scores
    sc = [pool[i].score for i in cand[:k + 1]]
    sel_margin = min((sc[i] - sc[i + 1] for i in range(len(sc) - 1)), default=math.inf)
    return nxt, tails, sel_margin


def level_step_tail_static(model: Model, level: int, frontier: List[FrontierNode],
                           h_rows: np.ndarray, pool: List[PoolEntry], k: int,
                           parent: Sequence[int], rank: Sequence[int]):
    """Tail of level >= 2 on a static tree (R16; [P1] §10.1): each frontier
    node's top-k children are scored and pooled exactly as in the dynamic
    tail, in (frontier slot, child rank) order; the next frontier's slot j is
    the child of rank rank[j] of slot parent[j], whatever its score."""
    base = len(pool)
    assert base == k + (level - 2) * k * k
    tails = []
    for j, x in enumerate(frontier):
        ids, logp, margin = lm_tail(model, h_rows[j], k)
        tails.append(margin)
        for t, lp in zip(ids, logp):
            pool.append(PoolEntry(x.score + float(lp), float(lp), int(t), x.pool_idx, level, j))
    nxt = []
    for j2 in range(k):
        pj, rk = int(parent[j2]), int(rank[j2])
        if not (0 <= pj < k and 0 <= rk < k):
            raise ValueError("template slot out of range")
        i = base + pj * k + rk
        e = pool[i]
        nxt.append(FrontierNode(e.token, e.score, i, pj, frontier[pj].anc + (j2,)))
    return nxt, tails


def build_static_tree(frontiers: Sequence[Sequence[FrontierNode]], root_token: int, P: int,
                      m: int) -> "Tree":
    """Flatten a static tree (R16): the root, then depth 1..D, each in slot
    order; node (L, j) has flat index 1 + (L-1)*k + j and its parent is the
    root (L = 1) or slot pslot of depth L-1.  Positions P-1+depth ([P1] §12
    item 5), ancestor-or-self mask.  The first m nodes are kept (parents
    precede children, so the kept set is ancestor-closed)."""
    k = len(frontiers[0])
    n = min(m, 1 + len(frontiers) * k)
    tokens = np.empty(n, dtype=np.int64)
    parents = np.empty(n, dtype=np.int64)
    depth = np.empty(n, dtype=np.int64)
    logscore = np.zeros(n, dtype=np.float64)
    tokens[0], parents[0], depth[0] = root_token, -1, 0
    for f in range(1, n):
        L, j = 1 + (f - 1) // k, (f - 1) % k
        x = frontiers[L - 1][j]
        tokens[f], depth[f], logscore[f] = x.token, L, x.score
        parents[f] = 0 if L == 1 else 1 + (L - 2) * k + x.pslot
    mask = np.zeros((n, n), dtype=np.uint8)
    for f in range(n):
        a = f
        while a != -1:
            mask[f, a] = 1
            a = parents[a]
    pool_idx = np.array([-1] + [frontiers[(f - 1) // k][(f - 1) % k].pool_idx for f in range(1, n)],
                        dtype=np.int64)
    return Tree(tokens, parents, depth, P - 1 + depth, mask, logscore, pool_idx)


# --------------------------------------------------------------------------- rerank, build

def rerank(pool: List[PoolEntry], m: int):
    """The best m-1 of every scored candidate by (score desc, depth asc,
    pool index asc) ([P1] §10.3 rerank and property 2; [P3] organize_draft_
    results takes num_draft_tokens-1).  Returns (selected pool indices,
    margin between the (m-1)-th and m-th scores)."""
    order = sorted(range(len(pool)), key=lambda i: (-pool[i].score, pool[i].depth, i))
    sel = order[:m - 1]
    if len(order) > m - 1 and m - 1 > 0:
        margin = pool[order[m - 2]].score - pool[order[m - 1]].score
    else:
        margin = math.inf
    return sel, margin


@dataclasses.dataclass
class Tree:
    tokens: np.ndarray     # [m] int
    parents: np.ndarray    # [m] int, -1 for the root
    depth: np.ndarray      # [m] int
    positions: np.ndarray  # [m] int
    mask: np.ndarray       # [m, m] uint8, 1 iff column is an ancestor of row or the row itself
    logscore: np.ndarray   # [m] float, 0 for the root
    pool_idx: np.ndarray   # [m] int, -1 for the root


def build_tree(pool: List[PoolEntry], sel: Sequence[int], root_token: int, P: int) -> Tree:
    """Flatten root + selected nodes: root first, then depth-major, then by
    parent's flat index, then by child rank (pool index) ([P4] EAGLE-2
    diagram lists x1, x2, x3, x1a, x1b, ...).  Positions are P-1+depth
    (shared per level, [P1] §12 item 5); the mask admits only ancestors and
    self ([P4] tree causal mask; [P3] ancestor-only mask)."""
    sel_set = set(sel)
    flat_of = {-1: 0}
    flat: List[int] = [-1]
    maxd = max((pool[i].depth for i in sel), default=0)
    for dd in range(1, maxd + 1):
        nodes = [i for i in sel if pool[i].depth == dd]
        for i in nodes:
            if pool[i].parent != -1 and pool[i].parent not in sel_set:
                raise ValueError("selected set is not ancestor-closed")
        nodes.sort(key=lambda i: (flat_of[pool[i].parent], i))
        for i in nodes:
            flat_of[i] = len(flat)
            flat.append(i)
    n = len(flat)
    tokens = np.empty(n, dtype=np.int64)
    parents = np.empty(n, dtype=np.int64)
    depth = np.empty(n, dtype=np.int64)
    logscore = np.zeros(n, dtype=np.float64)
    tokens[0], parents[0], depth[0] = root_token, -1, 0
    for f, i in enumerate(flat[1:], start=1):
        e = pool[i]
        tokens[f], parents[f], depth[f], logscore[f] = e.token, flat_of[e.parent], e.depth, e.score
    mask = np.zeros((n, n), dtype=np.uint8)
    for f in range(n):
        a = f
        while a != -1:
            mask[f, a] = 1
            a = parents[a]
    return Tree(tokens, parents, depth, P - 1 + depth, mask, logscore,
                np.array(flat, dtype=np.int64))


# --------------------------------------------------------------------------- verify

def verify_greedy(target_logits: np.ndarray, tokens: np.ndarray, parents: np.ndarray):
    """Greedy longest-accepted-path walk ([P4] EAGLE-2 diagram: accept the
    longest consistent path, back off to the last accepted node; R12).
    target_logits [m, V] are the target's logits at each tree node.
    Returns (path of flat indices starting at the root, accept_len = len(path),
    bonus token, margins of each argmax)."""
    node, path, margins = 0, [0], []
    while True:
        row = target_logits[node]
        best = int(np.argmax(row))  # numpy returns the lowest index among equal maxima
        srt = np.sort(row)
        margins.append(float(srt[-1] - srt[-2]) if row.size > 1 else math.inf)
        child = [c for c in range(len(tokens)) if parents[c] == node and tokens[c] == best]
        if not child:
            return path, len(path), best, margins
        node = child[0]
        path.append(node)


def target_probs(row: np.ndarray, temperature: float) -> np.ndarray:
    """Target distribution at a tree node: softmax(logits / T) in fp64 (R15)."""
    z = np.asarray(row, dtype=np.float64) / float(temperature)
    e = np.exp(z - z.max())
    return e / e.sum()


def sample_residual(p: np.ndarray, removed: Sequence[int], u: float):
    """One rejection-sampling draw at a node whose candidates `removed` were all
    rejected ([P1] §6.2: resample from the normalised positive part of the
    target minus the proposal; with point-mass proposals on the candidates that
    is p with those tokens taken out, renormalised; R15).  Inverse CDF over
    token ids: the smallest id x whose cumulative residual probability exceeds
    u.  Returns (token, margin): the distance of u from the nearer end of the
    drawn token's CDF interval (normalised units) that another token lies
    beyond; the ends of [0, 1) have none, so the first and last tokens with
    mass get an infinite margin on that side."""
    r = np.array(p, dtype=np.float64)
    r[list(removed)] = 0.0
    if not r.sum() > 0.0:  # the candidates held all the mass: draw from p
        r = np.array(p, dtype=np.float64)
    c = np.cumsum(r) / r.sum()
    x = int(np.searchsorted(c, u, side="right"))
    x = min(x, int(np.nonzero(r)[0][-1]))  # u at the very top: the last token with mass
    nz = np.nonzero(r)[0]
    lo_m = u - c[x - 1] if x > int(nz[0]) else math.inf
    hi_m = c[x] - u if x < int(nz[-1]) else math.inf
    return x, float(min(lo_m, hi_m))


def verify_relaxed(target_logits: np.ndarray, tokens: np.ndarray, parents: np.ndarray,
                   temperature: float, threshold: float, u: float):
    """Relaxed acceptance walk (R15; [P2] closing notes on SGLang).  From the
    root, descend to the first child in flat order whose target probability is
    at least `threshold`; at the stop, draw the bonus from the residual with
    the uniform u.  target_logits [m, V].  Returns (path of flat indices from
    the root, accept_len = len(path), bonus, margins): |p(c) - threshold| for
    every child tried, then the draw's margin."""
    m = len(tokens)
    node, path, margins = 0, [0], []
    while True:
        p = target_probs(target_logits[node], temperature)
        kids = [c for c in range(m) if parents[c] == node and c != node]
        nxt = None
        for c in kids:
            pc = float(p[int(tokens[c])])
            margins.append(abs(pc - threshold))
            if pc >= threshold:
                nxt = c
                break
        if nxt is None:
            bonus, mg = sample_residual(p, [int(tokens[c]) for c in kids], u)
            margins.append(mg)
            return path, len(path), bonus, margins
        node = nxt
        path.append(node)


def _rel_margin(a: float, b: float) -> float:
    """Distance of the comparison a <= b from flipping, relative to the larger
    side; 0 where both sides are below fp32's normal range."""
    hi = max(a, b)
    return abs(a - b) / hi if hi >= 1e-30 else 0.0


def verify_rejection(target_logits: np.ndarray, draft_logits: np.ndarray, tokens: np.ndarray,
                     parents: np.ndarray, temperature: float, u: Sequence[float]):
    """Recursive rejection sampling over the tree ([P1] §6.2: accept t-hat iff
    r <= min(1, p(t-hat)/q(t-hat)), otherwise resample from
    norm(max(0, p - q)), node by node; R17).  A token the current p gives no
    mass is never accepted (min(1, 0/q) = 0, also where q is 0).  Lossless when
    each child was drawn from q at its parent.  target_logits, draft_logits
    [m, V]; u [m + 1]: u[c] decides child c, u[m] draws the bonus.  Returns
    (path of flat indices from the root, accept_len, bonus, margins): for every
    child tried |u_c q(t_c) - p(t_c)| relative to the larger side (infinite
    where p(t_c) is 0), then the draw's margin."""
    m = len(tokens)
    node, path, margins = 0, [0], []
    while True:
        p = target_probs(target_logits[node], temperature)
        q = target_probs(draft_logits[node], temperature)
        nxt = None
        for c in [c for c in range(m) if parents[c] == node and c != node]:
            t = int(tokens[c])
            margins.append(_rel_margin(u[c] * q[t], p[t]) if p[t] > 0.0 else math.inf)
            if p[t] > 0.0 and u[c] * q[t] <= p[t]:
                nxt = c
                break
            r = np.maximum(p - q, 0.0)
            if r.sum() > 0.0:
                p = r / r.sum()
        if nxt is None:
            bonus, mg = sample_residual(p, [], u[m])
            margins.append(mg)
            return path, len(path), bonus, margins
        node = nxt
        path.append(node)


def verify_rejection_topk(target_logits: np.ndarray, tokens: np.ndarray, parents: np.ndarray,
                          temperature: float, u: Sequence[float]):
    """Rejection sampling of deterministic candidates (R18; [P1] §6.2 with each
    drafted child a point-mass proposal: the draft's top-k children are a fixed
    list, not draws from q).  At node x, p = softmax(target logits / T); the
    children are tried in flat order, child c accepted iff its token still has
    mass r(t_c) > 0 in the residual r = p with the rejected tokens removed and
    renormalised, and u_c <= r(t_c); a rejected token leaves r.  When every
    child is rejected (or x is a leaf) the bonus is drawn from r, i.e. p with
    x's children removed (sample_residual).  The emitted token is distributed
    as p for any fixed candidate list.  target_logits [m, V]; u [m + 1]: u[c]
    decides child c, u[m] draws the bonus.  Returns (path, accept_len, bonus,
    margins): for every child tried |u_c * left - p(t_c)| relative to the
    larger side (left = the residual's unnormalised mass; infinite for a token
    already removed), then the draw's margin."""
    m = len(tokens)
    node, path, margins = 0, [0], []
    while True:
        p = target_probs(target_logits[node], temperature)
        kids = [c for c in range(m) if parents[c] == node and c != node]
        keep = np.ones(p.size, dtype=bool)  # tokens still in the residual
        nxt = None
        for c in kids:
            t = int(tokens[c])
            left = float(p[keep].sum())
            if not keep[t] or not p[t] > 0.0:
                margins.append(math.inf)
            else:
                margins.append(_rel_margin(u[c] * left, p[t]))
                if u[c] * left <= p[t]:
                    nxt = c
                    break
            keep[t] = False
        if nxt is None:
            bonus, mg = sample_residual(p, [int(tokens[c]) for c in kids], u[m])
            margins.append(mg)
            return path, len(path), bonus, margins
        node = nxt
        path.append(node)


def tree_verify_attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, P: int,
                          mask: np.ndarray) -> np.ndarray:
    """Target-side tree-verify attention of one sequence ([P1] §6.2: the target
    scores every tree node in one forward with tree attention; [P4] EAGLE-2
    diagram, stage two: a node sees only its ancestors and itself; R14).
    q [m, H, hd] post-RoPE; k_cache/v_cache [>= P+m, Hkv, hd] with the prefix
    in rows 0..P-1 and the flat tree nodes in rows P..P+m-1; mask [m, m]
    (nonzero: visible).  Returns [m, H*hd]."""
    m = q.shape[0]
    out = np.empty((m, q.shape[1] * q.shape[2]), dtype=np.float64)
    for i in range(m):
        rows = list(range(P)) + [P + j for j in range(m) if mask[i, j]]
        out[i] = attend_row(q[i], k_cache[rows], v_cache[rows])
    return out


# --------------------------------------------------------------------------- extend

def draft_extend(model: Model, st: SeqState, true_feat: np.ndarray, tokens: np.ndarray,
                 path: Sequence[int], bonus: int):
    """Draft extend over the accepted path with the target's true features
    ([P3] "在 SGLang 里": rerun the draft over the accepted positions and
    take position accept_len-1 as the next start; [P2] Core Idea: restore
    the KV cache from the target's hidden states and the bonus token).
    Row i pairs the true feature of path node i with the next accepted
    token (the bonus for the last row), at position P+i (R10); rows see the
    prefix plus extend rows 0..i.  Returns (h rows, new K rows, new V rows)
    and updates ``st`` (K/V appended, P += accept_len, new root)."""
    c = model.cfg
    a = len(path) - 1
    feats = np.stack([true_feat[path[i]] for i in range(a + 1)])
    toks = [int(tokens[path[i + 1]]) if i < a else int(bonus) for i in range(a + 1)]
    pos = [st.P + i for i in range(a + 1)]
    x0, q, kn, vn = draft_rows(model, feats, toks, pos)
    K = np.concatenate([st.K[:st.P], kn], axis=0)
    V = np.concatenate([st.V[:st.P], vn], axis=0)
    attn = np.stack([attend_row(q[i], K[:st.P + i + 1], V[:st.P + i + 1])
                     for i in range(a + 1)])
    h = finish_rows(model, x0, attn)
    st.K, st.V, st.P = K, V, st.P + a + 1
    st.root_feat, st.root_token = h[a].copy(), int(bonus)
    return h, kn, vn


# --------------------------------------------------------------------------- one round

@dataclasses.dataclass
class RoundResult:
    tree: Tree
    path: List[int]
    accept_len: int
    bonus: int
    pool: List[PoolEntry]
    frontiers: List[List[FrontierNode]]
    feats: Dict[Tuple[int, int], np.ndarray]
    intree: Dict[Tuple[int, int], Tuple[np.ndarray, np.ndarray]]
    ext_h: np.ndarray
    ext_k: np.ndarray
    ext_v: np.ndarray
    margins: Dict[str, List[float]]

    def min_margin(self) -> float:
        return min((min(v) for v in self.margins.values() if v), default=math.inf)


def run_round(model: Model, st: SeqState, true_feat: np.ndarray, target_logits: np.ndarray
              ) -> RoundResult:
    """One steady-state round for one sequence (R1): level-1 tail, D-1
    draft forwards with expansion, rerank, build, greedy verify, extend.
    ``st`` is advanced in place."""
    c = model.cfg
    k, D, m = c.k, c.D, c.m
    pool, F, mg = level_one(model, st, k)
    margins = {"tail": list(mg["tail"]), "select": [], "rerank": [], "walk": []}
    frontiers = [F]
    feats: Dict[Tuple[int, int], np.ndarray] = {}
    intree: Dict[Tuple[int, int], Tuple[np.ndarray, np.ndarray]] = {}
    for level in range(2, D + 1):
        h = level_step_forward(model, st, level, F, feats, intree)
        F, tails, sm = level_step_tail(model, level, F, h, pool, k)
        margins["tail"] += tails
        margins["select"].append(sm)
        frontiers.append(F)
    sel, rm = rerank(pool, m)
    margins["rerank"].append(rm)
    tree = build_tree(pool, sel, st.root_token, st.P)
    path, alen, bonus, wm = verify_greedy(target_logits, tree.tokens, tree.parents)
    margins["walk"] += wm
    h, kn, vn = draft_extend(model, st, true_feat, tree.tokens, path, bonus)
    return RoundResult(tree, path, alen, bonus, pool, frontiers, feats, intree, h, kn, vn,
                       margins)
