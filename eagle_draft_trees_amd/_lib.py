"""ctypes binding of libeagle_mi355x.so (include/eagle_mi355x.h).

Argument marshalling only: every step of the draft round runs in the HIP
library.  torch provides device memory (tensors' data_ptr) and the stream.
Importing this module fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int32, c_size_t, c_void_p, POINTER

import numpy as np

LIB_NAME = "libeagle_mi355x.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

EAGLE_OK = 0
EAGLE_ERR_ARG = -1
EAGLE_ERR_SHAPE = -2
EAGLE_ERR_UNSUPPORTED = -3
EAGLE_ERR_WORKSPACE = -4
EAGLE_ERR_HIP = -5
EAGLE_F32 = 0
EAGLE_BF16 = 1
EAGLE_LEVEL_FULL = 0
EAGLE_LEVEL_TAIL_ONLY = 1
EAGLE_LEVEL_LMHEAD_ONLY = 2
EAGLE_LEVEL_FULL_FC = 3
EAGLE_MAX_DEPTH = 16
EAGLE_NOALLOC_MAX_ROWS = 4096
EAGLE_PACKED_WEIGHTS = 0x45505731

(WS_ERROR, WS_POOL, WS_FRONTIER, WS_FEAT, WS_TREE_K, WS_TREE_V, WS_EXT_H, WS_X0, WS_ATTN,
 WS_Y) = range(10)


class EagleError(RuntimeError):
    def __init__(self, status: int, what: str, msg: str):
        super().__init__(f"{what}: status {status} ({msg})")
        self.status = status


class EagleDims(ctypes.Structure):
    _fields_ = [("d", c_int32), ("n_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("ffn", c_int32), ("vocab", c_int32),
                ("dtype", c_int32), ("rms_eps", c_float), ("rope_theta", c_float)]


WEIGHT_NAMES = ("fc_w", "fc_b", "wq", "wk", "wv", "wo", "post_norm", "w_gate", "w_up",
                "w_down", "embed", "lm_head")


class EagleWeights(ctypes.Structure):
    _fields_ = ([(n, c_void_p) for n in WEIGHT_NAMES] + [("tok_proj", c_void_p)]
                + [("packed", c_int32)])


class EagleTreeCfg(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("depth", c_int32), ("topk", c_int32), ("m", c_int32),
                ("max_prefix", c_int32)]


class EagleSeqState(ctypes.Structure):
    _fields_ = [("k_cache", c_void_p), ("v_cache", c_void_p), ("prefix_len", c_void_p),
                ("root_feat", c_void_p), ("root_token", c_void_p)]


# numpy views of the workspace records
POOL_DTYPE = np.dtype([("score", "<f4"), ("logp", "<f4"), ("token", "<i4"), ("parent", "<i4"),
                       ("depth", "<i4"), ("pslot", "<i4")])
FRONTIER_DTYPE = np.dtype([("token", "<i4"), ("score", "<f4"), ("pool_idx", "<i4"),
                           ("pslot", "<i4"), ("anc", "<i4", (EAGLE_MAX_DEPTH,))])

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it first (__graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P = POINTER
        sig = {
            "eagle_workspace_bytes": (c_size_t, [P(EagleDims), P(EagleTreeCfg)]),
            "eagle_packed_weights_bytes": (c_size_t, [P(EagleDims)]),
            "eagle_pack_weights": (c_int32, [P(EagleDims), P(EagleWeights), c_void_p, c_size_t,
                                             P(EagleWeights), c_void_p]),
            "eagle_workspace_init": (c_int32, [P(EagleDims), P(EagleTreeCfg), c_void_p, c_size_t,
                                               c_void_p]),
            "eagle_draft_level": (c_int32, [P(EagleDims), P(EagleWeights), P(EagleTreeCfg),
                                            P(EagleSeqState), c_int32, c_int32, c_void_p, c_size_t,
                                            c_void_p]),
            "eagle_draft_level_timed": (c_int32, [P(EagleDims), P(EagleWeights), P(EagleTreeCfg),
                                                  P(EagleSeqState), c_int32, c_int32, c_void_p,
                                                  c_size_t, c_void_p, c_void_p, c_void_p]),
            "eagle_tree_verify_attention": (c_int32, [P(EagleDims), P(EagleTreeCfg), c_void_p,
                                                      c_void_p, c_void_p, c_void_p, c_void_p,
                                                      c_void_p, c_void_p, c_size_t, c_void_p]),
            "eagle_rerank_build_tree": (c_int32, [P(EagleDims), P(EagleTreeCfg), P(EagleSeqState),
                                                  c_void_p, c_size_t, c_void_p, c_void_p, c_void_p,
                                                  c_void_p, c_void_p, c_void_p, c_void_p]),
            "eagle_draft_level_static": (c_int32, [P(EagleDims), P(EagleWeights), P(EagleTreeCfg),
                                                   P(EagleSeqState), c_int32, c_int32, c_void_p,
                                                   c_void_p, c_size_t, c_void_p]),
            "eagle_build_static_tree": (c_int32, [P(EagleDims), P(EagleTreeCfg), P(EagleSeqState),
                                                  c_void_p, c_size_t, c_void_p, c_void_p, c_void_p,
                                                  c_void_p, c_void_p, c_void_p, c_void_p]),
            "eagle_verify_greedy": (c_int32, [P(EagleTreeCfg), c_int32, c_void_p, c_void_p,
                                              c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
            "eagle_verify_rejection_scratch_bytes": (c_size_t, [P(EagleTreeCfg), c_int32]),
            "eagle_verify_rejection": (c_int32, [P(EagleTreeCfg), c_int32, c_void_p, c_void_p,
                                                 c_void_p, c_void_p, c_float, c_void_p, c_void_p,
                                                 c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
            "eagle_verify_rejection_topk": (c_int32, [P(EagleTreeCfg), c_int32, c_void_p, c_void_p,
                                                      c_void_p, c_float, c_void_p, c_void_p,
                                                      c_void_p, c_void_p, c_void_p, c_size_t,
                                                      c_void_p]),
            "eagle_verify_rejection_topk_noalloc": (c_int32, [P(EagleTreeCfg), c_int32, c_void_p,
                                                              c_void_p, c_void_p, c_float, c_void_p,
                                                              c_void_p, c_void_p, c_void_p,
                                                              c_void_p]),
            "eagle_verify_relaxed_scratch_bytes": (c_size_t, [P(EagleTreeCfg)]),
            "eagle_verify_relaxed": (c_int32, [P(EagleTreeCfg), c_int32, c_void_p, c_void_p,
                                               c_void_p, c_float, c_float, c_void_p,
                                               c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                               c_void_p]),
            "eagle_draft_extend": (c_int32, [P(EagleDims), P(EagleWeights), P(EagleTreeCfg),
                                             P(EagleSeqState), c_void_p, c_void_p, c_void_p,
                                             c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
            "eagle_status_str": (ctypes.c_char_p, [c_int32]),
            "eagle_last_error": (ctypes.c_char_p, []),
            "eagle_ws_view": (c_int32, [P(EagleDims), P(EagleTreeCfg), c_void_p, c_int32,
                                        P(c_void_p), P(c_size_t)]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _check(status: int, what: str) -> None:
    if status != EAGLE_OK:
        msg = lib().eagle_last_error().decode(errors="replace")
        raise EagleError(status, what, msg)


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t if isinstance(t, int) else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def make_dims(cfg) -> EagleDims:
    return EagleDims(cfg.d, cfg.H, cfg.Hkv, cfg.hd, cfg.F, cfg.V,
                     EAGLE_BF16 if cfg.dtype == "bf16" else EAGLE_F32, cfg.rms_eps, cfg.rope_theta)


def make_tree_cfg(cfg) -> EagleTreeCfg:
    return EagleTreeCfg(cfg.B, cfg.D, cfg.k, cfg.m, cfg.max_prefix)


def make_weights(t: dict) -> EagleWeights:
    return EagleWeights(*[_ptr(t.get(n)) for n in WEIGHT_NAMES])


def make_state(k_cache, v_cache, prefix_len, root_feat, root_token) -> EagleSeqState:
    return EagleSeqState(_ptr(k_cache), _ptr(v_cache), _ptr(prefix_len), _ptr(root_feat),
                         _ptr(root_token))


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


# ------------------------------------------------------------------ entry points

def eagle_packed_weights_bytes(dims: EagleDims) -> int:
    return int(lib().eagle_packed_weights_bytes(ctypes.byref(dims)))


def eagle_pack_weights(dims, src: EagleWeights, dst, stream=None) -> EagleWeights:
    """Packs the row-major weights of `src` into the device buffer `dst`;
    returns the weights struct the drafting calls take."""
    out = EagleWeights()
    _check(lib().eagle_pack_weights(ctypes.byref(dims), ctypes.byref(src), _ptr(dst), _nbytes(dst),
                                    ctypes.byref(out), _stream(stream)), "eagle_pack_weights")
    return out


def eagle_workspace_bytes(dims: EagleDims, cfg: EagleTreeCfg) -> int:
    return int(lib().eagle_workspace_bytes(ctypes.byref(dims), ctypes.byref(cfg)))


def eagle_workspace_init(dims, cfg, ws, stream=None) -> None:
    _check(lib().eagle_workspace_init(ctypes.byref(dims), ctypes.byref(cfg), _ptr(ws), _nbytes(ws),
                                      _stream(stream)), "eagle_workspace_init")


def eagle_draft_level(dims, weights, cfg, state, level, flags, ws, stream=None) -> None:
    _check(lib().eagle_draft_level(ctypes.byref(dims), ctypes.byref(weights), ctypes.byref(cfg),
                                   ctypes.byref(state), level, flags, _ptr(ws), _nbytes(ws),
                                   _stream(stream)), f"eagle_draft_level({level})")


def _event(e) -> int:
    """Raw hipEvent_t of a torch.cuda.Event (which must have been recorded once,
    since torch creates the event lazily) or an int handle."""
    return e if isinstance(e, int) else e.cuda_event


def eagle_draft_level_timed(dims, weights, cfg, state, level, flags, ws, start_event, stop_event,
                            stream=None) -> None:
    _check(lib().eagle_draft_level_timed(ctypes.byref(dims), ctypes.byref(weights),
                                         ctypes.byref(cfg), ctypes.byref(state), level, flags,
                                         _ptr(ws), _nbytes(ws), _event(start_event),
                                         _event(stop_event), _stream(stream)),
           f"eagle_draft_level_timed({level})")


def eagle_tree_verify_attention(dims, cfg, q, k_cache, v_cache, prefix_len, mask, out, ws,
                                stream=None) -> None:
    _check(lib().eagle_tree_verify_attention(ctypes.byref(dims), ctypes.byref(cfg), _ptr(q),
                                             _ptr(k_cache), _ptr(v_cache), _ptr(prefix_len),
                                             _ptr(mask), _ptr(out), _ptr(ws), _nbytes(ws),
                                             _stream(stream)), "eagle_tree_verify_attention")


def eagle_rerank_build_tree(dims, cfg, state, ws, tokens, parents, depth=None, positions=None,
                            mask=None, node_logscore=None, stream=None) -> None:
    _check(lib().eagle_rerank_build_tree(ctypes.byref(dims), ctypes.byref(cfg), ctypes.byref(state),
                                         _ptr(ws), _nbytes(ws), _ptr(tokens), _ptr(parents),
                                         _ptr(depth), _ptr(positions), _ptr(mask),
                                         _ptr(node_logscore), _stream(stream)),
           "eagle_rerank_build_tree")


def eagle_draft_level_static(dims, weights, cfg, state, level, flags, tmpl, ws, stream=None) -> None:
    _check(lib().eagle_draft_level_static(ctypes.byref(dims), ctypes.byref(weights),
                                          ctypes.byref(cfg), ctypes.byref(state), level, flags,
                                          _ptr(tmpl), _ptr(ws), _nbytes(ws), _stream(stream)),
           "eagle_draft_level_static")


def eagle_build_static_tree(dims, cfg, state, ws, tokens, parents, depth=None, positions=None,
                            mask=None, node_logscore=None, stream=None) -> None:
    _check(lib().eagle_build_static_tree(ctypes.byref(dims), ctypes.byref(cfg), ctypes.byref(state),
                                         _ptr(ws), _nbytes(ws), _ptr(tokens), _ptr(parents),
                                         _ptr(depth), _ptr(positions), _ptr(mask),
                                         _ptr(node_logscore), _stream(stream)),
           "eagle_build_static_tree")


def eagle_verify_greedy(cfg, vocab, target_logits, tokens, parents, accept_len, accept_path, bonus,
                        stream=None) -> None:
    _check(lib().eagle_verify_greedy(ctypes.byref(cfg), vocab, _ptr(target_logits), _ptr(tokens),
                                     _ptr(parents), _ptr(accept_len), _ptr(accept_path),
                                     _ptr(bonus), _stream(stream)), "eagle_verify_greedy")


def eagle_verify_rejection_scratch_bytes(cfg, vocab) -> int:
    return int(lib().eagle_verify_rejection_scratch_bytes(ctypes.byref(cfg), vocab))


def eagle_verify_rejection(cfg, vocab, target_logits, draft_logits, tokens, parents, temperature,
                           uniforms, accept_len, accept_path, bonus, scratch, stream=None) -> None:
    _check(lib().eagle_verify_rejection(ctypes.byref(cfg), vocab, _ptr(target_logits),
                                        _ptr(draft_logits), _ptr(tokens), _ptr(parents),
                                        float(temperature), _ptr(uniforms), _ptr(accept_len),
                                        _ptr(accept_path), _ptr(bonus), _ptr(scratch),
                                        _nbytes(scratch), _stream(stream)), "eagle_verify_rejection")


def eagle_verify_rejection_topk(cfg, vocab, target_logits, tokens, parents, temperature, uniforms,
                                accept_len, accept_path, bonus, scratch, stream=None) -> None:
    _check(lib().eagle_verify_rejection_topk(ctypes.byref(cfg), vocab, _ptr(target_logits),
                                             _ptr(tokens), _ptr(parents), float(temperature),
                                             _ptr(uniforms), _ptr(accept_len), _ptr(accept_path),
                                             _ptr(bonus), _ptr(scratch), _nbytes(scratch),
                                             _stream(stream)), "eagle_verify_rejection_topk")


def eagle_verify_rejection_topk_noalloc(cfg, vocab, target_logits, tokens, parents, temperature,
                                        uniforms, accept_len, accept_path, bonus, stream=None) -> None:
    _check(lib().eagle_verify_rejection_topk_noalloc(ctypes.byref(cfg), vocab, _ptr(target_logits),
                                                     _ptr(tokens), _ptr(parents), float(temperature),
                                                     _ptr(uniforms), _ptr(accept_len),
                                                     _ptr(accept_path), _ptr(bonus), _stream(stream)),
           "eagle_verify_rejection_topk_noalloc")


def eagle_verify_relaxed_scratch_bytes(cfg) -> int:
    return int(lib().eagle_verify_relaxed_scratch_bytes(ctypes.byref(cfg)))


def eagle_verify_relaxed(cfg, vocab, target_logits, tokens, parents, temperature, threshold,
                         uniforms, accept_len, accept_path, bonus, scratch, stream=None) -> None:
    _check(lib().eagle_verify_relaxed(ctypes.byref(cfg), vocab, _ptr(target_logits), _ptr(tokens),
                                      _ptr(parents), float(temperature), float(threshold),
                                      _ptr(uniforms), _ptr(accept_len), _ptr(accept_path),
                                      _ptr(bonus), _ptr(scratch), _nbytes(scratch),
                                      _stream(stream)), "eagle_verify_relaxed")


def eagle_draft_extend(dims, weights, cfg, state, true_feat, tokens, accept_len, accept_path, bonus,
                       ws, stream=None) -> None:
    _check(lib().eagle_draft_extend(ctypes.byref(dims), ctypes.byref(weights), ctypes.byref(cfg),
                                    ctypes.byref(state), _ptr(true_feat), _ptr(tokens),
                                    _ptr(accept_len), _ptr(accept_path), _ptr(bonus), _ptr(ws),
                                    _nbytes(ws), _stream(stream)), "eagle_draft_extend")


def eagle_ws_view(dims, cfg, ws, what: int):
    """(byte offset into the workspace tensor, bytes) of a workspace region."""
    p, n = c_void_p(), c_size_t()
    _check(lib().eagle_ws_view(ctypes.byref(dims), ctypes.byref(cfg), _ptr(ws), what,
                               ctypes.byref(p), ctypes.byref(n)), "eagle_ws_view")
    return int(p.value) - _ptr(ws), int(n.value)


def eagle_status_str(status: int) -> str:
    return lib().eagle_status_str(status).decode()


def eagle_last_error() -> str:
    return lib().eagle_last_error().decode(errors="replace")
