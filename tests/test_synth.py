"""The seeded generator: bf16 rounding, determinism, and config shapes
against the pages' parameter counts."""
import json
import os

import numpy as np

import synth


def test_bf16_round_to_nearest_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)  # bf16 spacing at 1.0
    vals = np.array([one, one + ulp / 2, one + 3 * ulp / 2, one + ulp / 4, -2.5, 3.0e38],
                    dtype=np.float32)
    got = synth.bf16_bits_to_f32(synth.bf16_bits(vals))
    # ties go to the even mantissa: 1+ulp/2 -> 1, 1+3ulp/2 -> 1+2ulp
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == one + 2 * ulp and got[3] == 1.0
    assert got[4] == -2.5
    x = np.random.default_rng(0).normal(size=10000).astype(np.float32)
    r = synth.bf16_bits_to_f32(synth.bf16_bits(x))
    assert np.all(np.abs(r - x) <= np.abs(x) * 2.0 ** -8)


def test_generator_is_deterministic_and_per_tensor():
    cfg = synth.config_by_name("ragged_bf16")
    a = synth.make_inputs(cfg, 5)
    b = synth.make_inputs(cfg, 5)
    c = synth.make_inputs(cfg, 6)
    for n in ("fc_w", "embed", "k_cache", "target_logits", "root_token", "prefix_len"):
        assert np.array_equal(a[n], b[n])
    assert not np.array_equal(a["fc_w"], c["fc_w"])
    assert a["prefix_len"][0] == 1 and np.all(a["prefix_len"] <= cfg.P_hi)
    assert a["k_cache"].shape == (cfg.B, cfg.max_prefix, cfg.Hkv, cfg.hd)
    for bb in range(cfg.B):  # rows at and beyond the prefix stay zero
        assert not a["k_cache"][bb, a["prefix_len"][bb]:].any()
    s = synth.make_inputs(cfg, 5, with_weights=False, only_seqs=[2])
    assert np.array_equal(s["k_cache"][2], a["k_cache"][2]) and not s["k_cache"][1].any()


def test_config_shapes_reproduce_page_parameter_counts():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "draft_param_counts.json")))
    for name, billions in g["trainable_billions"].items():
        c = synth.config_by_name(name)
        d = c.d
        n = (2 * d * d + d                        # FC 2d->d with bias
             + d * (c.H + 2 * c.Hkv) * c.hd       # q, k, v
             + c.H * c.hd * d                     # o
             + 3 * d * c.F                        # SwiGLU
             + d)                                 # post-attention norm
        assert round(n / 1e9, 2) == billions, (name, n)


def test_logit_scale_recipe():
    cfg = synth.config_by_name("tiny")
    inp = synth.make_inputs(cfg, 0)
    z = inp["lm_head"].astype(np.float64) @ inp["root_feat"][0].astype(np.float64)
    assert 2.0 < z.std() < 4.0
