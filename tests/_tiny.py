"""Hand-built tiny models for the oracle's CPU pins (fp32 storage, exact in fp64)."""
import numpy as np

import synth


def tiny_cfg(**kw) -> synth.TreeConfig:
    base = dict(name="hand", uid=99, dtype="f32", B=1, d=8, H=2, Hkv=2, hd=4, F=6, V=12,
                P_lo=3, P_hi=3, D=3, k=2, m=4)
    base.update(kw)
    return synth.TreeConfig(**base)


def tensors(cfg, rng, scale=0.3, **over):
    d, F, V = cfg.d, cfg.F, cfg.V
    t = dict(
        fc_w=rng.normal(0, scale, (d, 2 * d)), fc_b=rng.normal(0, scale, d),
        wq=rng.normal(0, scale, (cfg.H * cfg.hd, d)), wk=rng.normal(0, scale, (cfg.Hkv * cfg.hd, d)),
        wv=rng.normal(0, scale, (cfg.Hkv * cfg.hd, d)), wo=rng.normal(0, scale, (d, cfg.H * cfg.hd)),
        post_norm=1.0 + rng.normal(0, 0.1, d), w_gate=rng.normal(0, scale, (F, d)),
        w_up=rng.normal(0, scale, (F, d)), w_down=rng.normal(0, scale, (d, F)),
        embed=rng.normal(0, 1.0, (V, d)), lm_head=rng.normal(0, 1.0, (V, d)))
    t.update(over)
    return {k: np.asarray(v, dtype=np.float32) for k, v in t.items()}


def seq_state(cfg, rng, P=None):
    from oracle import eagle_oracle as O
    P = cfg.P_lo if P is None else P
    K = rng.normal(0, 1, (P, cfg.Hkv, cfg.hd)).astype(np.float32).astype(np.float64)
    V = rng.normal(0, 1, (P, cfg.Hkv, cfg.hd)).astype(np.float32).astype(np.float64)
    return O.SeqState(K, V, P, rng.normal(0, 1, cfg.d).astype(np.float32).astype(np.float64),
                      int(rng.integers(0, cfg.V)))
