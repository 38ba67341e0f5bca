"""Parity of the many-row LM heads against the oracle's LM-head tail, through
the C ABI.

When a level puts more than 64 bf16 rows through the LM head (a large batch
at level 1, or a wide frontier), the library runs it as a tiled MFMA GEMM
with the per-slab softmax and top-k fused (logits never leave the chip);
at 17..64 rows with a large vocabulary, as a streaming MFMA kernel.
[P1] "EAGLE 推测解码为什么比 Medusa 快？（含 EAGLE-2 动态草稿树）" §4.1: the draft
distribution is softmax(LM_Head(f-hat)); EAGLE-2 keeps the top-k children of
each expanded row ([P3] zdszero.github.io spec_medusa_eagle, "在 SGLang 里").
Level 1 on a batch of B sequences is B such rows.

  * 300 rows, vocab 3000, d 256, top-4: every row compared.  Two 256-row
    tiles, the second ragged (44 rows), and a vocabulary that ends inside a
    256-column block (its last slab holds 56 columns, the block's fourth slab
    lies past the vocabulary);
  * 512 rows, vocab 128256, d 4096, top-4 (the large-vocabulary chain
    workload's vocabulary and hidden size; the shape the batched GEMM is timed
    at): rows sampled at both ends of both row tiles;
  * 40 rows, vocab 50003, d 256, top-4: the streaming kernel with two weight
    tiles per wave (the chain workload runs it with four), every row
    compared.

Gate as in the level tests: child probabilities within 1e-3, node scores
within the logit-scale tolerance, ids bit-exact where the oracle's tail margin
exceeds the near-tie threshold, and the level-1 frontier exact then.
"""
from __future__ import annotations

import gc

import numpy as np
import pytest

import synth
from tests._gpu import HAVE_GPU, OracleSeqs, gpu_frontier, gpu_pool, say
from tests.test_gpu_parity import _check_children, _check_frontier

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not HAVE_GPU, reason="needs a GPU")]

# name, uid, dtype, B, d, H, Hkv, hd, F, V, P_lo, P_hi, D, k, m
SHAPES = {
    "rows300_v3000": (synth.TreeConfig("batched_lm_300", 40, "bf16", 300, 256, 4, 2, 64, 512, 3000,
                                       8, 40, 3, 4, 8), None),
    "rows512_v128256": (synth.TreeConfig("batched_lm_512", 41, "bf16", 512, 4096, 32, 32, 128, 256,
                                         128256, 4, 4, 2, 4, 5),
                        [0, 1, 127, 255, 256, 383, 510, 511]),
    # 40 rows (17..64: the streaming LM head), vocab 50003: two 16-column
    # weight tiles per wave, rows past 40 padded, the last slab ragged
    "rows40_v50003": (synth.TreeConfig("streaming_lm_40", 42, "bf16", 40, 256, 4, 2, 64, 512, 50003,
                                       8, 40, 3, 4, 8), None),
}


@pytest.mark.parametrize("shape", list(SHAPES))
def test_batched_lmhead_level1(shape):
    import torch
    from oracle import eagle_oracle as O
    from eagle_draft_trees_amd.round import DraftRound
    cfg, seqs = SHAPES[shape]
    say(f"[many-row LM head] {shape}: {cfg.B} rows x vocab {cfg.V} x d {cfg.d}, top-{cfg.k}")
    inp = synth.make_inputs(cfg, seed=5, with_round=False)
    r = DraftRound(cfg, inp)
    r.reset_state(inp)
    r.level(1)
    torch.cuda.synchronize()
    gp, gf = gpu_pool(r), gpu_frontier(r, 1)
    del r
    gc.collect()
    torch.cuda.empty_cache()
    orc = OracleSeqs(cfg, inp, seqs)
    orc.model._CACHE_LIMIT = cfg.V * cfg.d  # widen the LM head once for all sampled rows
    orc.level1()
    feats = np.stack([orc.st[b].root_feat for b in orc.seqs])
    lscale = np.abs(O.lm_logits(orc.model, feats)).max(axis=1)
    near = 0
    for i, b in enumerate(orc.seqs):
        n = _check_children(cfg, gp[b], orc.pool[b], 0, orc.tail_margin[b], True, lscale[i:i + 1])
        near += n
        if n == 0:
            _check_frontier(gf[b], orc.F[b][0])
    say(f"  {len(orc.seqs)} rows compared, {near} near-tie rows")
    assert near < len(orc.seqs)
