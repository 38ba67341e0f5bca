"""Round driver: device buffers for one configuration and the four C-ABI
calls in round order (level 1..depth, rerank/build, verify, extend).

Order of a steady-state decode round ([P3] zdszero.github.io
spec_medusa_eagle, "在 SGLang 里": one verify, steps-1 draft forwards, one
draft extend; the first level's top-k comes from the previous extend).
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import _lib as L


def to_device(a, dtype: str, device) -> torch.Tensor:
    """Host array -> device tensor.  bf16 arrays arrive as uint16 bit patterns."""
    if isinstance(a, torch.Tensor):
        return a.to(device)
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


PACKED_NAMES = ("fc_w", "wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "lm_head")


class DraftRound:
    """Owns the device state of one configuration and runs rounds."""

    def __init__(self, cfg, inputs: Dict[str, object], device: str = "cuda:0"):
        self.cfg = cfg
        self.device = torch.device(device)
        dev = self.device
        dt = cfg.dtype
        self.w = {n: to_device(inputs[n], dt, dev) for n in L.WEIGHT_NAMES}
        self.k_cache = to_device(inputs["k_cache"], dt, dev)
        self.v_cache = to_device(inputs["v_cache"], dt, dev)
        self.prefix_len = to_device(np.asarray(inputs["prefix_len"], np.int32), dt, dev)
        self.root_feat = to_device(inputs["root_feat"], dt, dev)
        self.root_token = to_device(np.asarray(inputs["root_token"], np.int32), dt, dev)
        self.true_feat = to_device(inputs["true_feat"], dt, dev) if "true_feat" in inputs else None
        self.target_logits = (to_device(inputs["target_logits"], dt, dev)
                              if "target_logits" in inputs else None)
        B, m, D = cfg.B, cfg.m, cfg.D
        i32 = dict(dtype=torch.int32, device=dev)
        self.tokens = torch.zeros(B, m, **i32)
        self.parents = torch.zeros(B, m, **i32)
        self.depth = torch.zeros(B, m, **i32)
        self.positions = torch.zeros(B, m, **i32)
        self.mask = torch.zeros(B, m, m, dtype=torch.uint8, device=dev)
        self.logscore = torch.zeros(B, m, dtype=torch.float32, device=dev)
        self.accept_len = torch.zeros(B, **i32)
        self.accept_path = torch.zeros(B, D + 1, **i32)
        self.bonus = torch.zeros(B, **i32)
        self.dims = L.make_dims(cfg)
        self.tcfg = L.make_tree_cfg(cfg)
        # the streamed matrices go to the packed tile layout once; the
        # row-major copies of those are released
        self.wpack = torch.empty(L.eagle_packed_weights_bytes(self.dims), dtype=torch.uint8, device=dev)
        self.wts = L.eagle_pack_weights(self.dims, L.make_weights(self.w), self.wpack)
        torch.cuda.synchronize(dev)
        for n in PACKED_NAMES:
            del self.w[n]
        self.state = L.make_state(self.k_cache, self.v_cache, self.prefix_len, self.root_feat,
                                  self.root_token)
        nbytes = L.eagle_workspace_bytes(self.dims, self.tcfg)
        if nbytes == 0:
            raise L.EagleError(L.EAGLE_ERR_SHAPE, "eagle_workspace_bytes", L.eagle_last_error())
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        L.eagle_workspace_init(self.dims, self.tcfg, self.ws)
        # per-segment softmax statistics of the relaxed verify (allocated here,
        # so that a call captured into a graph allocates nothing)
        self._rv_scratch = torch.empty(L.eagle_verify_relaxed_scratch_bytes(self.tcfg),
                                       dtype=torch.uint8, device=dev)

    def reset_state(self, inputs: Dict[str, object]) -> None:
        """Reload the sequence state from host arrays and zero the workspace."""
        dt = self.cfg.dtype
        self.k_cache.copy_(to_device(inputs["k_cache"], dt, self.device))
        self.v_cache.copy_(to_device(inputs["v_cache"], dt, self.device))
        self.prefix_len.copy_(to_device(np.asarray(inputs["prefix_len"], np.int32), dt,
                                        self.device))
        self.root_feat.copy_(to_device(inputs["root_feat"], dt, self.device))
        self.root_token.copy_(to_device(np.asarray(inputs["root_token"], np.int32), dt,
                                        self.device))
        if self.target_logits is not None and "target_logits" in inputs:
            self.target_logits.copy_(to_device(inputs["target_logits"], dt, self.device))
        L.eagle_workspace_init(self.dims, self.tcfg, self.ws)

    # -------------------------------------------------------------- calls
    def level(self, level: int, flags: int = L.EAGLE_LEVEL_FULL, stream=None) -> None:
        L.eagle_draft_level(self.dims, self.wts, self.tcfg, self.state, level, flags, self.ws,
                            stream)

    def level_timed(self, level: int, flags: int, start_event, stop_event, stream=None) -> None:
        L.eagle_draft_level_timed(self.dims, self.wts, self.tcfg, self.state, level, flags,
                                  self.ws, start_event, stop_event, stream)

    def level_static(self, level: int, tmpl: torch.Tensor, flags: int = L.EAGLE_LEVEL_FULL,
                     stream=None) -> None:
        L.eagle_draft_level_static(self.dims, self.wts, self.tcfg, self.state, level, flags, tmpl,
                                   self.ws, stream)

    def build_static(self, stream=None) -> None:
        L.eagle_build_static_tree(self.dims, self.tcfg, self.state, self.ws, self.tokens,
                                  self.parents, self.depth, self.positions, self.mask,
                                  self.logscore, stream)

    def rerank(self, stream=None) -> None:
        L.eagle_rerank_build_tree(self.dims, self.tcfg, self.state, self.ws, self.tokens,
                                  self.parents, self.depth, self.positions, self.mask,
                                  self.logscore, stream)

    def verify(self, target_logits: Optional[torch.Tensor] = None, stream=None) -> None:
        tl = self.target_logits if target_logits is None else target_logits
        L.eagle_verify_greedy(self.tcfg, self.cfg.V, tl, self.tokens, self.parents,
                              self.accept_len, self.accept_path, self.bonus, stream)

    def verify_relaxed(self, temperature: float, threshold: float, uniforms: torch.Tensor,
                       target_logits: Optional[torch.Tensor] = None, stream=None) -> None:
        tl = self.target_logits if target_logits is None else target_logits
        L.eagle_verify_relaxed(self.tcfg, self.cfg.V, tl, self.tokens, self.parents, temperature,
                               threshold, uniforms, self.accept_len, self.accept_path, self.bonus,
                               self._rv_scratch, stream)

    def extend(self, true_feat: Optional[torch.Tensor] = None, stream=None) -> None:
        tf = self.true_feat if true_feat is None else true_feat
        L.eagle_draft_extend(self.dims, self.wts, self.tcfg, self.state, tf, self.tokens,
                             self.accept_len, self.accept_path, self.bonus, self.ws, stream)

    def run_static_round(self, tmpl: torch.Tensor, stream=None) -> None:
        """A round on a static tree: the template's levels, the static build,
        greedy verify and the extend."""
        self.level(1, stream=stream)
        for level in range(2, self.cfg.D + 1):
            self.level_static(level, tmpl, stream=stream)
        self.build_static(stream)
        self.verify(stream=stream)
        self.extend(stream=stream)

    def draft(self, stream=None) -> None:
        for level in range(1, self.cfg.D + 1):
            self.level(level, stream=stream)
        self.rerank(stream)

    def run_round(self, stream=None) -> None:
        self.draft(stream)
        self.verify(stream=stream)
        self.extend(stream=stream)

    # -------------------------------------------------------------- workspace views
    def ws_region(self, what: int) -> torch.Tensor:
        off, n = L.eagle_ws_view(self.dims, self.tcfg, self.ws, what)
        return self.ws[off:off + n]

    def ws_typed(self, what: int) -> torch.Tensor:
        """Feature/KV regions as tensors of the config dtype."""
        t = self.ws_region(what)
        return t.view(torch.bfloat16 if self.cfg.dtype == "bf16" else torch.float32)

    def ws_records(self, what: int) -> np.ndarray:
        """Pool / frontier regions copied to host as numpy records."""
        dt = L.POOL_DTYPE if what == L.WS_POOL else L.FRONTIER_DTYPE
        return self.ws_region(what).cpu().numpy().view(dt)

    def ws_write(self, what: int, host: np.ndarray, byte_offset: int = 0) -> None:
        """Copy host bytes into a workspace region (tests seed stage inputs this way)."""
        raw = np.ascontiguousarray(host).view(np.uint8).reshape(-1)
        reg = self.ws_region(what)
        reg[byte_offset:byte_offset + raw.size].copy_(torch.from_numpy(raw).to(self.device))
