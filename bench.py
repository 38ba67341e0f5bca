"""Benchmark: EAGLE-2 draft-tree rounds/s on one MI355X at the Vicuna-7B shape.

A step is one whole steady-state round of the draft path on the synthetic
batch: level 1 (LM-head tail) + levels 2..depth (draft forward, LM head,
softmax, top-k, k*k->k select), rerank/build, greedy verify, draft extend.
Inputs are resident in HBM before timing starts; up to ten consecutive
rounds are captured into one HIP graph, which is replayed.  Between rounds
the prefix length is restored on the device so every round has the same
shape, while the root feature and root token advance (the extend writes
them).

Prints one JSON line (rank 0).  With --gpus N > 1 it exits: the benchmark
measures one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PROFILES = os.path.join(ROOT, "profiles")


def algorithmic_bytes(cfg) -> dict:
    """Bytes a round must move at minimum (weights once per pass, prefix KV
    once per level, verified target-logit rows), by component."""
    es = 2 if cfg.dtype == "bf16" else 4
    d, F, V = cfg.d, cfg.F, cfg.V
    layer = es * (2 * d * d + d * (cfg.H + 2 * cfg.Hkv) * cfg.hd + cfg.H * cfg.hd * d + 3 * d * F)
    lm = es * V * d
    P = (cfg.P_lo + cfg.P_hi) / 2.0
    kv_level = es * 2 * cfg.B * P * cfg.Hkv * cfg.hd
    passes = cfg.D  # (depth-1) level forwards + the extend
    return {
        "layer_weights": passes * layer,
        "lm_head": cfg.D * lm,
        # the extend reads the prefix plus its own rows (at most min(m, D+1))
        "prefix_kv": (cfg.D - 1) * kv_level + es * 2 * cfg.B * (P + min(cfg.m, cfg.D + 1)) * cfg.Hkv * cfg.hd,
        "verify_rows": 4 * cfg.B * 2 * V,   # about two target-logit rows per sequence
        "lm_head_per_launch": lm,
    }


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "eagle_draft_trees_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


LMHEAD_SOURCES = ("k_lmhead.hip", "skinny_core.h", "eagle_internal.h")


def stored_traffic(workload: str):
    """HBM bytes per LM-head launch from the committed counter summary (its
    `key: value` lines), if it was taken on the current kernel source and the
    same workload; else None."""
    path = os.path.join(PROFILES, "k_lmhead_7b_counters.md")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                rec[k.strip()] = v.strip().strip("`")
    if rec.get("source_hash") != source_hash(*LMHEAD_SOURCES) or rec.get("workload") != workload:
        return None
    try:
        return int(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def blas_info() -> dict:
    """The BLAS library NumPy runs on and its thread count."""
    try:
        import threadpoolctl
        info = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
    except Exception:
        info = []
    if not info:
        return {"vendor": "unknown", "threads": os.cpu_count() or 1}
    i = info[0]
    return {"vendor": f"{i.get('internal_api', '?')} {i.get('version', '')}".strip(),
            "threads": int(i.get("num_threads", 1))}


def cpu_baseline(cfg, inp, budget_s: float) -> dict:
    """The fp64 oracle, as it stands, on this host's cores: whole rounds of the
    same workload until about budget_s seconds of work.  A batch is sampled by
    sequence (one sequence-round at a time, in order); the rate is scaled to
    the whole batch and then labelled extrapolated."""
    import numpy as np
    from oracle import eagle_oracle as O
    blas = blas_info()
    model = O.Model(cfg, inp)
    W = lambda a: O.widen(a, cfg.dtype)
    # widen the weights once, outside the timed region
    for n in ("fc_w", "wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "lm_head"):
        if model.raw[n].size <= model._CACHE_LIMIT:
            model.w(n)
    done, t0 = 0, time.perf_counter()
    while True:
        b = done % cfg.B
        st = O.SeqState(W(inp["k_cache"][b]), W(inp["v_cache"][b]), int(inp["prefix_len"][b]),
                        W(inp["root_feat"][b]), int(inp["root_token"][b]))
        O.run_round(model, st, W(inp["true_feat"][b]), inp["target_logits"][b].astype(np.float64))
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s or done >= 50 * cfg.B:
            break
    rounds = done / cfg.B
    out = {"value": rounds / el, "unit": "rounds/s", "cores": blas["threads"], "kind": "oracle",
           "blas": blas["vendor"], "blas_threads": blas["threads"], "host_cpus": os.cpu_count(),
           "sample": f"{done} sequence-round(s) of the same workload ({cfg.B} sequence(s) per round), "
                     f"{el:.1f} s, fp64 NumPy"}
    if done % cfg.B:
        out["extrapolated"] = True
    return out


def batched_lmhead(torch, L, dev, stream, rows=512, vocab=128256, d=4096, reps=10) -> dict:
    """The LM-head GEMM batched over `rows` rows at the large-vocabulary chain
    workload's shape (vocab 128256, d 4096; 512 = its batch x tree rows): a
    level-1 LM-head-only call on a batch of `rows` sequences (the same kernel a
    level with more than 16 rows runs, logits reduced to slab records on chip),
    timed with kernel-stamped HIP events.  MFMA utilisation = 2*rows*vocab*d
    FLOP per launch over the dense bf16 MFMA peak."""
    import numpy as np
    H, hd, F = 32, 128, 14336
    dims = L.EagleDims(d, H, H, hd, F, vocab, L.EAGLE_BF16, 1e-6, 1e4)
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    bf = dict(dtype=torch.bfloat16, device=dev)
    shapes = {"fc_w": (d, 2 * d), "fc_b": (d,), "wq": (H * hd, d), "wk": (H * hd, d),
              "wv": (H * hd, d), "wo": (d, H * hd), "post_norm": (d,), "w_gate": (F, d),
              "w_up": (F, d), "w_down": (d, F), "embed": (vocab, d)}
    w = {n: torch.zeros(sh, **bf) for n, sh in shapes.items()}  # not read by an LM-head-only call
    w["lm_head"] = torch.randn(vocab, d, generator=gen, **bf) * (3.0 / d ** 0.5)
    wpack = torch.empty(L.eagle_packed_weights_bytes(dims), dtype=torch.uint8, device=dev)
    wts = L.eagle_pack_weights(dims, L.make_weights(w), wpack)
    tcfg = L.EagleTreeCfg(rows, 2, 1, 2, 4)
    kc = torch.zeros(rows, 4, H, hd, **bf)
    vc = torch.zeros(rows, 4, H, hd, **bf)
    plen = torch.full((rows,), 2, dtype=torch.int32, device=dev)
    feat = torch.randn(rows, d, generator=gen, **bf)
    tok = torch.zeros(rows, dtype=torch.int32, device=dev)
    state = L.make_state(kc, vc, plen, feat, tok)
    ws = torch.empty(L.eagle_workspace_bytes(dims, tcfg), dtype=torch.uint8, device=dev)
    L.eagle_workspace_init(dims, tcfg, ws)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    with torch.cuda.stream(stream):
        for q in ev:  # torch creates events on their first record
            for e in q:
                e.record(stream)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        L.eagle_draft_level(dims, wts, tcfg, state, 1, L.EAGLE_LEVEL_LMHEAD_ONLY, ws, stream)
        for e0, e1 in ev:
            L.eagle_draft_level_timed(dims, wts, tcfg, state, 1, L.EAGLE_LEVEL_LMHEAD_ONLY, ws,
                                      e0, e1, stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    tflops = 2.0 * rows * vocab * d / (ms * 1e-3) / 1e12
    return {"kernel": "k_lg_xpack + k_lmgemm (feature rows into fragment order, then the batched LM-head GEMM + per-slab softmax/top-k; bf16, rows > 64)",
            "rows": rows, "vocab": vocab, "d": d, "bound": "mfma",
            "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "avg_launch_us": round(ms * 1e3, 1),
            "launches": reps}


def tree_verify(torch, L, r, cfg, stream, reps=50, replays=10) -> dict:
    """Target-side tree-verify attention at the round's shape: the m flattened
    tree tokens of each sequence attend to its prefix and, through the mask the
    round just built, to their ancestors' rows (appended after the prefix).
    Timed with HIP events around `replays` replays of a graph of `reps`
    back-to-back calls (attention and its split merge), after two untimed
    replays; bytes = the K/V rows read plus q, mask and output."""
    es = 2 if cfg.dtype == "bf16" else 4
    gen = torch.Generator(device=r.device)
    gen.manual_seed(1)
    q = torch.randn(cfg.B, cfg.m, cfg.H, cfg.hd, generator=gen, device=r.device, dtype=torch.float32)
    out = torch.empty(cfg.B, cfg.m, cfg.H * cfg.hd, device=r.device,
                      dtype=torch.bfloat16 if cfg.dtype == "bf16" else torch.float32)
    call = lambda: L.eagle_tree_verify_attention(r.dims, r.tcfg, q, r.k_cache, r.v_cache, r.prefix_len,
                                                 r.mask, out, r.ws, stream)
    with torch.cuda.stream(stream):
        call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()  # launched as the round is: from a graph
    with torch.cuda.graph(g, stream=stream):
        for _ in range(reps):
            call()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        g.replay()
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(replays):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * replays)
    P = (cfg.P_lo + cfg.P_hi) / 2.0
    nbytes = cfg.B * ((P + cfg.m) * cfg.Hkv * cfg.hd * 2 * es + cfg.m * cfg.H * cfg.hd * (4 + es)
                      + cfg.m * cfg.m)
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"kernel": "k_attn + k_attn_merge (tree verify mode)", "bound": "hbm",
            "us_per_call": round(us, 2), "bytes_per_call": int(nbytes), "achieved": round(gbps, 1),
            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "timing": f"HIP events around {replays} replays of a graph of {reps} back-to-back calls"}


def relaxed_verify(torch, L, r, cfg, stream, reps=50, replays=10) -> dict:
    """Relaxed acceptance walk at the round's shape (temperature 1, threshold
    0.1) on the tree the round just built and the round's target logits.
    Timed like the tree-verify attention; bytes = every tree row's target
    logits (the softmax statistics of all m rows are taken in parallel before
    the walk) plus one sixteenth of the stop row, scanned again for the
    residual draw."""
    gen = torch.Generator(device=r.device)
    gen.manual_seed(2)
    uni = torch.rand(cfg.B, generator=gen, device=r.device, dtype=torch.float32)
    call = lambda: r.verify_relaxed(1.0, 0.1, uni, stream=stream)
    with torch.cuda.stream(stream):
        call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(reps):
            call()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        g.replay()
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(replays):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * replays)
    alen = r.accept_len.cpu().numpy()
    nbytes = cfg.B * cfg.m * cfg.V * 4 + cfg.B * (-(-cfg.V // 16)) * 4
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"kernel": "k_relaxed_stats + k_verify_relaxed", "bound": "hbm", "us_per_call": round(us, 2),
            "accept_len": [int(a) for a in alen], "bytes_per_call": nbytes,
            "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(gbps / HBM_PEAK_GBPS, 4), "temperature": 1.0, "threshold": 0.1,
            "timing": f"HIP events around {replays} replays of a graph of {reps} back-to-back calls"}


def rejection_verify(torch, L, r, cfg, stream, reps=50, replays=10) -> dict:
    """Strict recursive rejection sampling at the round's shape (temperature
    1) on the tree the round just built: target logits the round's, draft
    logits those plus N(0, 0.3^2) noise (a draft close to the target), random
    uniforms.  Timed like the tree-verify attention."""
    gen = torch.Generator(device=r.device)
    gen.manual_seed(3)
    dl = r.target_logits + 0.3 * torch.randn(r.target_logits.shape, generator=gen, device=r.device)
    uni = torch.rand(cfg.B, cfg.m + 1, generator=gen, device=r.device, dtype=torch.float32)
    scr = torch.empty(L.eagle_verify_rejection_scratch_bytes(r.tcfg, cfg.V), dtype=torch.uint8,
                      device=r.device)
    call = lambda: L.eagle_verify_rejection(r.tcfg, cfg.V, r.target_logits, dl, r.tokens, r.parents,
                                            1.0, uni, r.accept_len, r.accept_path, r.bonus, scr,
                                            stream)
    with torch.cuda.stream(stream):
        call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(reps):
            call()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        g.replay()
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(replays):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * replays)
    return {"kernel": "k_relaxed_stats (both arrays) + k_verify_rejection", "bound": "latency", "us_per_call": round(us, 2),
            "accept_len": [int(a) for a in r.accept_len.cpu().numpy()], "temperature": 1.0,
            "draft": "target logits + N(0, 0.3^2)",
            "timing": f"HIP events around {replays} replays of a graph of {reps} back-to-back calls"}


def static_round(torch, r, cfg, stream, saved_plen, rounds=50) -> dict:
    """A whole round on a static tree at the round's shape: the template's
    slot j of every depth >= 2 is the best child (rank 0) of slot j, i.e. the
    root's k children each extended greedily, m = min(1 + D*k, m) nodes.
    Captured and timed like the dynamic round."""
    k, D = cfg.k, cfg.D
    tm = torch.zeros(D, k, 2, dtype=torch.int32)
    tm[:, :, 0] = torch.arange(k, dtype=torch.int32)
    tmpl = tm.to(r.device)

    def one():
        r.run_static_round(tmpl, stream=stream)
        torch.add(saved_plen, 0, out=r.prefix_len)

    with torch.cuda.stream(stream):
        one()
    torch.cuda.synchronize()
    per = 10
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(per):
            one()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(rounds // per):
        g.replay()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    return {"rounds_per_s": round(rounds / el, 1), "ms_per_round": round(el * 1e3 / rounds, 4),
            "template": "slot j of every depth >= 2 = rank-0 child of slot j (k greedy chains)",
            "timing": f"{rounds} rounds from a graph of {per}, wall clock"}


def rejection_topk_verify(torch, L, r, cfg, stream, reps=50, replays=10) -> dict:
    """Rejection sampling of deterministic candidates (the draft's top-k
    children as point-mass proposals) at the round's shape, on the tree the
    round just built and the round's target logits, random uniforms.  Timed
    like the tree-verify attention."""
    gen = torch.Generator(device=r.device)
    gen.manual_seed(4)
    uni = torch.rand(cfg.B, cfg.m + 1, generator=gen, device=r.device, dtype=torch.float32)
    call = lambda: L.eagle_verify_rejection_topk(r.tcfg, cfg.V, r.target_logits, r.tokens, r.parents, 1.0, uni,
                                                 r.accept_len, r.accept_path, r.bonus, r._rv_scratch, stream)
    us = _graph_time(torch, call, stream, reps, replays)
    return {"kernel": "k_relaxed_stats + k_verify_relaxed<topk>", "bound": "latency", "us_per_call": round(us, 2),
            "accept_len": [int(a) for a in r.accept_len.cpu().numpy()], "temperature": 1.0,
            "timing": f"HIP events around {replays} replays of a graph of {reps} back-to-back calls"}


def _graph_time(torch, call, stream, reps, replays) -> float:
    """Microseconds per call: `reps` calls captured in a graph, two untimed
    replays, then `replays` replays between two HIP events on `stream`."""
    with torch.cuda.stream(stream):
        call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(reps):
            call()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        g.replay()
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(replays):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * replays)


def copy_bandwidth(torch, dev, stream, nbytes=1 << 30, reps=10) -> dict:
    """Device copy rate: a 1 GiB buffer copied `reps` times between HIP events;
    read plus written bytes over the time."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    with torch.cuda.stream(stream):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            dst.copy_(src)
        e1.record(stream)
    torch.cuda.synchronize()
    gbps = 2.0 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"gbps": round(gbps, 1), "bytes_copied": nbytes, "timing": f"{reps} copies of 1 GiB between HIP events"}


def measure_rounds(torch, r, stream, steps, warmup, graph=True) -> dict:
    """Whole rounds on the synthetic batch: R consecutive rounds per HIP graph
    (R the largest divisor of the step count up to 10; every round runs
    whole, and one graph launch's host latency is paid per R rounds), warm-up,
    then exactly `steps` rounds between two synchronisations (the wall-clock
    rate), each replay also bracketed by HIP events (the per-round spread).
    Between rounds the prefix length is restored on the device so that every
    round has the same shape; the root feature and token advance."""
    import numpy as np
    saved_plen = r.prefix_len.clone()

    def one_round():
        r.run_round(stream=stream)
        torch.add(saved_plen, 0, out=r.prefix_len)

    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        one_round()   # eager round: loads code objects, checks the path runs
    torch.cuda.synchronize()
    per = max(q for q in range(1, 11) if steps % q == 0) if graph else 1
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(per):
                one_round()
        torch.cuda.synchronize()
        run = g.replay
    else:
        def run():
            one_round()
    for _ in range(-(-warmup // per)):
        with torch.cuda.stream(stream):
            run()
    torch.cuda.synchronize()
    n = steps // per
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for e0, e1 in ev:
            e0.record(stream)
            run()
            e1.record(stream)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    per_round = np.array([e0.elapsed_time(e1) / per for e0, e1 in ev])
    out = {"rounds_per_s": steps / el, "ms_per_round": el * 1e3 / steps, "rounds_per_graph": per,
           "replays": n, "saved_plen": saved_plen}
    if n >= 1:
        out["round_ms"] = {"p10": round(float(np.percentile(per_round, 10)), 4),
                           "median": round(float(np.median(per_round)), 4),
                           "p90": round(float(np.percentile(per_round, 90)), 4),
                           "timing": f"HIP events around each of {n} graph replays of {per} rounds"}
    return out


def lm_kernel_name(cfg, rows) -> str:
    """The LM-head kernel the library's plan takes for `rows` rows: up to 16
    the skinny streaming kernel; bf16 with d a multiple of 128, the batched
    MFMA GEMM above 64 rows and, from 17 to 64 rows, the streaming MFMA
    kernel when the vocabulary gives each wave at least two 16-column weight
    tiles (more than 32768 columns), or at 49 to 64 rows with d a multiple of
    256; else k_lmhead."""
    if rows <= 16:
        return "k_lmskinny"
    tiled = cfg.dtype == "bf16" and cfg.d % 128 == 0
    if tiled and rows > 64:
        return "k_lg_xpack + k_lmgemm"
    if tiled and -(-cfg.V // 16) > 8 * 256:
        return "k_lmrows"
    if tiled and rows > 48 and cfg.d % 256 == 0:
        return "k_lmrows"
    return "k_lmhead"


def lmhead_roofline(torch, L, r, cfg, stream, steps, scrub) -> dict:
    """The dominant kernel, the LM-head GEMM with its fused per-slab softmax
    and top-k, timed live on the stream it runs on: a LMHEAD_ONLY level call
    launches exactly that one kernel, and the timed variant has the kernel's
    own dispatch stamp a pair of HIP events at its start and end.  A second
    pair of ordinary events, queued around the same call, shows what queue
    markers add.  Between launches a 512 MiB read (a reduction, outside the
    events) evicts the 256 MB memory-side Infinity Cache, which would
    otherwise keep part of the LM head warm across back-to-back launches;
    inside a round the layer weights stream through it in between.  A read,
    not a copy: a copy's dirty lines would be written back during the timed
    launch."""
    import numpy as np
    scrub_out = torch.empty((), dtype=torch.float32, device=r.device)
    n_lm = max(5, steps // 5) * (cfg.D - 1)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_lm)]
    with torch.cuda.stream(stream):
        for q in ev:            # torch creates events on their first record
            for e in q:
                e.record(stream)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i, (m0, k0, k1, m1) in enumerate(ev):
            torch.sum(scrub, dim=0, out=scrub_out)
            m0.record(stream)
            r.level_timed(2 + i % (cfg.D - 1), L.EAGLE_LEVEL_LMHEAD_ONLY, k0, k1, stream=stream)
            m1.record(stream)
    torch.cuda.synchronize()
    lm_ms = float(np.mean([k0.elapsed_time(k1) for _, k0, k1, _ in ev]))
    lm_marker_ms = float(np.mean([m0.elapsed_time(m1) for m0, _, _, m1 in ev]))
    es = 2 if cfg.dtype == "bf16" else 4
    nbytes = es * cfg.V * cfg.d
    rows = cfg.B * cfg.k
    gbps = nbytes / (lm_ms * 1e-3) / 1e9
    kname = lm_kernel_name(cfg, rows)
    scope = "the LM-head GEMM (the largest share of the 7B-shaped round's time)"
    if kname == "k_lmrows":
        scope += ("; an LM-head-only call has no down projection to pack its X, so these launches "
                  "read the features in place, where the round's levels read the copy the down "
                  "epilogue writes in MFMA fragment order")
    return {"kernel": f"{kname} (LM-head GEMM + per-slab softmax/top-k, {rows} rows)",
            "scope": scope,
            "bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(gbps / HBM_PEAK_GBPS, 4), "avg_launch_us": round(lm_ms * 1e3, 2),
            "timing": f"{n_lm} launches, HIP events stamped by the kernel's dispatch "
                      f"(hipExtLaunchKernel); queued marker events around the same launches: "
                      f"{lm_marker_ms * 1e3:.2f} us",
            "bytes_per_launch": int(nbytes),
            "mfma_frac": round(2.0 * rows * cfg.V * cfg.d / (lm_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}


def workload_name(cfg) -> str:
    return (f"EAGLE-2 draft round, {cfg.name}-shaped draft head, {cfg.dtype}, batch {cfg.B}, "
            f"d {cfg.d}, heads {cfg.H}/{cfg.Hkv}x{cfg.hd}, ffn {cfg.F}, vocab {cfg.V}, "
            f"prefix {cfg.P_lo}-{cfg.P_hi}, depth {cfg.D}, topk {cfg.k}, m {cfg.m}")


def round_hbm(cfg, rounds_s, copy_gbps) -> dict:
    ab = algorithmic_bytes(cfg)
    nbytes = ab["layer_weights"] + ab["lm_head"] + ab["prefix_kv"] + ab["verify_rows"]
    gbps = nbytes * rounds_s / 1e9
    out = {"algorithmic_bytes": int(nbytes), "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
           "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4)}
    if copy_gbps:
        out["copy_gbps"] = copy_gbps
        out["frac_of_copy"] = round(gbps / copy_gbps, 4)
    return out


def other_config(torch, L, name, dev, stream, seed, steps, warmup, cpu_budget, copy_gbps, scrub) -> dict:
    """One more workload of the benchmark table: rounds/s, tree tokens/s, the
    round's share of the HBM roofline, the LM head's roofline, and the oracle
    on a sample of its sequences."""
    import synth
    from eagle_draft_trees_amd.round import DraftRound
    cfg = synth.config_by_name(name)
    inp = synth.make_inputs(cfg, seed=seed)
    r = DraftRound(cfg, inp, dev)
    m = measure_rounds(torch, r, stream, steps, warmup)
    out = {"workload": workload_name(cfg), "rounds_per_s": round(m["rounds_per_s"], 2),
           "ms_per_round": round(m["ms_per_round"], 4), "round_ms": m.get("round_ms"),
           "rounds_timed": steps, "rounds_per_graph": m["rounds_per_graph"],
           "tree_tokens_per_s": round(m["rounds_per_s"] * cfg.B * cfg.m, 1)}
    if cfg.dtype == "bf16":
        out["round_hbm"] = round_hbm(cfg, m["rounds_per_s"], copy_gbps)
        out["lmhead_roofline"] = lmhead_roofline(torch, L, r, cfg, stream, steps, scrub)
    else:
        out["note"] = ("fp32 and about 12 MB of weights: the round lives in the 256 MB Infinity Cache and "
                       "is bound by launch latency, not HBM")
    del r
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if cpu_budget > 0:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, cpu_budget)
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="7b")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-batched", action="store_true",
                    help="skip the batched LM-head GEMM measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads of the table (13b, 70b, chain, tiny)")
    ap.add_argument("--configs-cpu-budget", type=float, default=8.0)
    ap.add_argument("--lmhead-only", type=int, default=0,
                    help="only launch the LM-head kernel this many times (counter runs)")
    ap.add_argument("--rounds-only", type=int, default=0,
                    help="only run this many eager rounds after the calibration copies (counter runs)")
    ap.add_argument("--batched-only", action="store_true",
                    help="only the batched LM-head GEMM measurement (counter runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              f"(the path would shard by sequence with no per-round communication)",
              file=sys.stderr)
        return 2

    import torch

    import synth
    from eagle_draft_trees_amd import _lib as L
    from eagle_draft_trees_amd.round import DraftRound

    dev = torch.device("cuda:0")
    if args.batched_only:
        print(json.dumps(batched_lmhead(torch, L, dev, torch.cuda.Stream(device=dev))), flush=True)
        return 0
    cfg = synth.config_by_name(args.config)
    inp = synth.make_inputs(cfg, seed=args.seed)
    r = DraftRound(cfg, inp, "cuda:0")
    stream = torch.cuda.Stream(device=dev)
    workload = workload_name(cfg)

    if args.lmhead_only:
        # counter runs: a copy of known size (calibration), then the LM head alone
        src = torch.empty(64 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        with torch.cuda.stream(stream):
            r.level(1, stream=stream)
            for _ in range(args.lmhead_only):
                r.level(2, L.EAGLE_LEVEL_LMHEAD_ONLY, stream=stream)
        torch.cuda.synchronize()
        print(json.dumps({"lmhead_only": args.lmhead_only, "copy_bytes": src.numel()}))
        return 0

    if args.rounds_only:
        # counter runs: a copy of known size (calibration), then whole rounds, one by one
        src = torch.empty(64 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        saved = r.prefix_len.clone()
        with torch.cuda.stream(stream):
            for _ in range(args.rounds_only):
                r.run_round(stream=stream)
                torch.add(saved, 0, out=r.prefix_len)
        torch.cuda.synchronize()
        print(json.dumps({"rounds_only": args.rounds_only, "copy_bytes": src.numel(), "workload": workload}))
        return 0

    m = measure_rounds(torch, r, stream, args.steps, args.warmup, graph=not args.no_graph)
    rounds_s = m["rounds_per_s"]
    scrub = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    roof = lmhead_roofline(torch, L, r, cfg, stream, args.steps, scrub)
    roof["traffic"] = stored_traffic(workload)
    copy = copy_bandwidth(torch, dev, stream)

    out = {
        "metric": "EAGLE-2 draft-tree rounds/s + tree tokens/s at 7B shape; % HBM roofline",
        "value": round(rounds_s, 3),
        "unit": "rounds/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_per_round"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; weights N(0,0.02^2), LM head N(0,1)*3/sqrt(d), features N(0,1), "
                "target logits N(0,9))",
        "config": {"workload": workload, "batch": cfg.B, "tree_tokens_per_round": cfg.B * cfg.m,
                   "graph": not args.no_graph, "rounds_per_graph": m["rounds_per_graph"]},
        "tree_tokens_per_s": round(rounds_s * cfg.B * cfg.m, 1),
        "round_ms": m.get("round_ms"),
        "round_hbm": round_hbm(cfg, rounds_s, copy["gbps"]),
        "roofline": roof,
        "hbm_copy": copy,
    }
    out["tree_verify_attention"] = tree_verify(torch, L, r, cfg, stream)
    out["relaxed_verify"] = relaxed_verify(torch, L, r, cfg, stream)
    out["rejection_verify"] = rejection_verify(torch, L, r, cfg, stream)
    out["rejection_topk_verify"] = rejection_topk_verify(torch, L, r, cfg, stream)
    if 1 + cfg.D * cfg.k >= cfg.m:
        out["static_round"] = static_round(torch, r, cfg, stream, m["saved_plen"])
    del r
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_batched:
        out["mfma_batched_lmhead"] = batched_lmhead(torch, L, dev, stream)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_budget)
    if not args.no_configs:
        others = {}
        for name in ("tiny", "13b", "70b", "chain"):
            if name == args.config:
                continue
            print(f"bench: {name}", file=sys.stderr, flush=True)
            others[name] = other_config(torch, L, name, dev, stream, args.seed, 20, 5,
                                        0.0 if args.no_cpu_baseline else args.configs_cpu_budget,
                                        copy["gbps"], scrub)
        out["configs"] = others
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
