"""Seeded synthetic inputs for one EAGLE-2 draft round.

This module only draws random numbers and rounds them to the storage type
(fp32 or bf16 bit patterns).  It holds none of the method's arithmetic, and
both the HIP path (through the tests and the bench) and the fp64 oracle take
their inputs from here.

Recipe (the pages give no value ranges; these are the fill-ins):
  * draft-layer weights fc_w, fc_b, wq, wk, wv, wo, w_gate, w_up, w_down and
    the embedding table ~ N(0, 0.02^2);
  * post-attention RMSNorm gain = 1 (or 1 + N(0, 0.1^2) when
    ``norm_gain_noise`` is set, to exercise the gain);
  * LM head = N(0, 1) * 3 / sqrt(d), so unit-variance features give logits
    of standard deviation about 3;
  * root feature and the target's true features ~ N(0, 1);
  * prefix K/V ~ N(0, 1), stored as if already rotated (post-RoPE);
  * target logits ~ N(0, 3^2), always fp32;
  * token ids uniform over the vocabulary;
  * prefix lengths fixed or uniform per sequence, per config.

Every tensor has its own stream:
``default_rng(SeedSequence([seed, config.uid, tensor_id]))``.  Draws are
float32 normals scaled in float32, then rounded once to bf16 with
round-to-nearest-even when the config is bf16.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import math
import os
from typing import Dict, Optional, Sequence, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class TreeConfig:
    """Shapes of one draft round.

    The tree triple (depth, topk, m) is the (num-steps, eagle-topk,
    num-draft-tokens) triple of the SGLang mapping; m counts the root.
    """
    name: str
    uid: int
    dtype: str          # "f32" or "bf16": weights, features and KV
    B: int              # sequences in the batch
    d: int              # hidden size
    H: int              # query heads
    Hkv: int            # key/value heads (GQA when Hkv < H)
    hd: int             # head dim
    F: int              # SwiGLU inner size
    V: int              # vocabulary (shared by embedding, LM head, target logits)
    P_lo: int           # prefix length range (inclusive); P_lo == P_hi is fixed
    P_hi: int
    D: int              # tree depth (levels per round)
    k: int              # top-k per node and frontier width
    m: int              # tree size including the root
    norm_gain_noise: bool = False
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0

    @property
    def max_prefix(self) -> int:
        # room for three draft extends, each appending up to m rows
        return self.P_hi + 3 * self.m

    @property
    def pool_size(self) -> int:
        return self.k + (self.D - 1) * self.k * self.k

    @property
    def qkv_out(self) -> int:
        return (self.H + 2 * self.Hkv) * self.hd


# The five workloads of the draft-round benchmark, then test-only variants.
CONFIGS: Dict[int, TreeConfig] = {}


def _add(c: TreeConfig) -> None:
    CONFIGS[c.uid] = c


_add(TreeConfig("tiny", 0, "f32", 1, 256, 4, 4, 64, 688, 4096, 64, 64, 3, 2, 6))
_add(TreeConfig("7b", 1, "bf16", 1, 4096, 32, 32, 128, 11008, 32000, 512, 512, 6, 10, 60))
_add(TreeConfig("13b", 2, "bf16", 16, 5120, 40, 40, 128, 13824, 32000, 512, 1024, 5, 4, 8))
_add(TreeConfig("70b", 3, "bf16", 4, 8192, 64, 8, 128, 28672, 32000, 2048, 2048, 6, 10, 48))
_add(TreeConfig("chain", 4, "bf16", 64, 4096, 32, 32, 128, 14336, 128256, 1024, 4096, 8, 1, 8))
# test-only shapes: ragged tails, GQA, hd=128, bf16 tiny, non-unit norm gain
_add(TreeConfig("tiny_bf16", 10, "bf16", 1, 256, 4, 4, 64, 688, 4096, 64, 64, 3, 2, 6))
_add(TreeConfig("ragged_f32", 11, "f32", 3, 192, 3, 1, 64, 400, 1003, 1, 40, 4, 3, 9,
                norm_gain_noise=True))
_add(TreeConfig("ragged_bf16", 12, "bf16", 3, 192, 3, 1, 64, 400, 1003, 1, 40, 4, 3, 9,
                norm_gain_noise=True))
_add(TreeConfig("hd128_bf16", 13, "bf16", 2, 256, 2, 2, 128, 264, 777, 3, 100, 5, 4, 12,
                norm_gain_noise=True))
_add(TreeConfig("chain_small", 14, "f32", 5, 128, 2, 2, 64, 256, 515, 7, 70, 6, 1, 6))
_add(TreeConfig("wide_bf16", 15, "bf16", 2, 256, 4, 2, 64, 512, 2048, 20, 90, 4, 16, 64,
                norm_gain_noise=True))
# a pool above 1024 entries (16 + 4*256): the rerank's LDS-sort path
_add(TreeConfig("deep_bf16", 16, "bf16", 2, 256, 4, 2, 64, 512, 2048, 20, 90, 5, 16, 64,
                norm_gain_noise=True))
# more than 64 LM-head rows (80 at level 1, 160 after): the tiled batched
# LM-head GEMM; a vocabulary that ends inside a 128-column block
_add(TreeConfig("batch_bf16", 17, "bf16", 80, 256, 4, 2, 64, 512, 3000, 8, 40, 3, 2, 6))
# a chain shorter than depth+1 (topk 1, m = 3 < D + 1 = 5): the extend's rows
# per sequence are limited by m, and a whole-tree path reaches that limit, on
# the weight-streaming kernels (3 sequences x 3 rows)
_add(TreeConfig("short_f32", 18, "f32", 3, 256, 4, 4, 64, 688, 4096, 64, 64, 4, 1, 3))
# 64 level rows (16 sequences x top-4) over a small vocabulary: the streaming
# LM head with one weight tile per wave, its features packed by the down
# epilogue; a vocabulary that ends inside a 16-column tile; at d 1280 the FC
# and O split K into uneven ranges (5 loop iterations over 2 workgroups)
_add(TreeConfig("rows64_bf16", 21, "bf16", 16, 1280, 10, 5, 128, 512, 3001, 8, 60, 4, 4, 12))
# the deepest tree the library takes (depth 16: every ancestor slot of a
# frontier record in use, 17 verify and extend rows per sequence)
_add(TreeConfig("deep16_f32", 22, "f32", 2, 256, 4, 2, 64, 512, 1000, 5, 60, 16, 2, 32))
_add(TreeConfig("deep16_bf16", 23, "bf16", 2, 256, 4, 2, 64, 512, 1000, 5, 60, 16, 2, 32))
# 320 (sequence, KV head) query tiles: the attention's four-wave workgroups
# (three per compute unit), bf16 at hd 128 and fp32 at hd 64
_add(TreeConfig("heads_bf16", 19, "bf16", 40, 1024, 8, 8, 128, 512, 2000, 8, 70, 4, 3, 9))
_add(TreeConfig("heads_f32", 20, "f32", 40, 512, 8, 8, 64, 512, 2000, 8, 70, 4, 3, 9))


def config_by_name(name: str) -> TreeConfig:
    for c in CONFIGS.values():
        if c.name == name:
            return c
    raise KeyError(name)


# ----------------------------------------------------------------- rounding

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


# ----------------------------------------------------------------- drawing

_TENSOR_IDS = {
    "fc_w": 1, "fc_b": 2, "wq": 3, "wk": 4, "wv": 5, "wo": 6, "post_norm": 7,
    "w_gate": 8, "w_up": 9, "w_down": 10, "embed": 11, "lm_head": 12,
    "k_cache": 20, "v_cache": 21, "prefix_len": 22, "root_feat": 23, "root_token": 24,
    "true_feat": 30, "target_logits": 31,
}


def _rng(seed: int, cfg: TreeConfig, name: str) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cfg.uid, _TENSOR_IDS[name]]))


def _normal(rng: np.random.Generator, shape: Tuple[int, ...], scale: float,
            store_bf16: bool, chunk_rows: int = 1 << 14) -> np.ndarray:
    """Draw N(0, scale^2) in float32 row-chunks, rounding each chunk once."""
    shape = tuple(int(s) for s in shape)
    rows = shape[0]
    inner = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    out = np.empty((rows, inner), dtype=np.uint16 if store_bf16 else np.float32)
    step = max(1, min(rows, chunk_rows * max(1, 4096 // max(1, inner))))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        z = rng.standard_normal((r1 - r0, inner), dtype=np.float32)
        if scale != 1.0:
            z *= np.float32(scale)
        out[r0:r1] = bf16_bits(z) if store_bf16 else z
    return out.reshape(shape)


def make_inputs(cfg: TreeConfig, seed: int = 0, *, with_weights: bool = True,
                with_state: bool = True, with_round: bool = True,
                only_seqs: Optional[Sequence[int]] = None) -> Dict[str, object]:
    """Build every input of one round for ``cfg``.

    Floating tensors of the config dtype are uint16 bf16 bit patterns (bf16)
    or float32 (f32); integer tensors are int32; target logits are float32.
    Weight layouts: fc_w [d][2d] (columns 0..d-1 take the feature, d..2d-1
    the token embedding), wq [H*hd][d], wk/wv [Hkv*hd][d], wo [d][H*hd],
    w_gate/w_up [F][d], w_down [d][F], embed/lm_head [V][d], fc_b and
    post_norm [d].  K/V cache [B][max_prefix][Hkv][hd]; rows at and beyond a
    sequence's prefix length are zero.

    ``only_seqs`` keeps the per-sequence state of the listed sequences only
    (the others' K/V rows stay zero); it draws the same values for those
    sequences as a full call does.
    """
    bf = cfg.dtype == "bf16"
    d, V, F = cfg.d, cfg.V, cfg.F
    out: Dict[str, object] = {"cfg": cfg, "seed": seed}
    # every tensor has its own stream, so they are drawn in parallel threads
    # (numpy's generators release the interpreter lock while filling arrays);
    # the values do not depend on the order
    jobs: Dict[str, object] = {}

    def normal(name, shape, scale):
        jobs[name] = lambda: _normal(_rng(seed, cfg, name), shape, scale, bf)

    if with_weights:
        normal("fc_w", (d, 2 * d), 0.02)
        normal("fc_b", (d,), 0.02)
        normal("wq", (cfg.H * cfg.hd, d), 0.02)
        normal("wk", (cfg.Hkv * cfg.hd, d), 0.02)
        normal("wv", (cfg.Hkv * cfg.hd, d), 0.02)
        normal("wo", (d, cfg.H * cfg.hd), 0.02)

        def gain():
            if cfg.norm_gain_noise:
                g = 1.0 + _normal(_rng(seed, cfg, "post_norm"), (d,), 0.1, False)
            else:
                g = np.ones((d,), dtype=np.float32)
            return bf16_bits(g) if bf else g.astype(np.float32)

        jobs["post_norm"] = gain
        normal("w_gate", (F, d), 0.02)
        normal("w_up", (F, d), 0.02)
        normal("w_down", (d, F), 0.02)
        normal("embed", (V, d), 0.02)
        normal("lm_head", (V, d), 3.0 / math.sqrt(d))
    if with_state:
        B, P = cfg.B, cfg.max_prefix
        rp = _rng(seed, cfg, "prefix_len")
        plen = rp.integers(cfg.P_lo, cfg.P_hi + 1, size=B, dtype=np.int64).astype(np.int32)
        if cfg.name.startswith("ragged") and B >= 1:
            plen[0] = 1  # a sequence whose only prefix row is the root row
        out["prefix_len"] = plen
        keep = set(range(B)) if only_seqs is None else set(int(b) for b in only_seqs)

        def cache(name):
            c = np.zeros((B, P, cfg.Hkv, cfg.hd), dtype=np.uint16 if bf else np.float32)
            r = _rng(seed, cfg, name)
            for b in range(B):
                # draw every sequence in order so that only_seqs reproduces the same values
                n = int(plen[b])
                if b in keep:
                    c[b, :n] = _normal(r, (n, cfg.Hkv, cfg.hd), 1.0, bf)
                else:
                    r.standard_normal((n, cfg.Hkv * cfg.hd), dtype=np.float32)
            return c

        jobs["k_cache"] = lambda: cache("k_cache")
        jobs["v_cache"] = lambda: cache("v_cache")
        normal("root_feat", (B, d), 1.0)
        jobs["root_token"] = lambda: _rng(seed, cfg, "root_token").integers(
            0, V, size=B, dtype=np.int64).astype(np.int32)
    if with_round:
        normal("true_feat", (cfg.B, cfg.m, d), 1.0)
        jobs["target_logits"] = lambda: _normal(_rng(seed, cfg, "target_logits"),
                                                (cfg.B, cfg.m, V), 3.0, False)
    # the largest draws first, so that they start at once
    order = sorted(jobs, key=lambda n: n not in ("k_cache", "v_cache", "embed", "lm_head", "w_gate",
                                                  "w_up", "w_down"))
    with cf.ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1))) as ex:
        futs = {n: ex.submit(jobs[n]) for n in order}
        for n, f in futs.items():
            out[n] = f.result()
    return out
