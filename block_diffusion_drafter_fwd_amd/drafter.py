"""Python binding of the DFlash drafter's C ABI (include/dflash.h).

PyTorch supplies device memory and the stream; every computation happens in
libdflash.so.  The names mirror the C calls: ``Drafter`` wraps a dflash_ctx,
``Session`` a dflash_session, ``propose_batch`` and ``sample`` the batched
calls.
"""
from __future__ import annotations

import ctypes
from ctypes import byref, c_int32, c_int64, c_void_p
from typing import Dict, Optional, Sequence, Tuple

import numpy as np
import torch

from . import abi
from .abi import check

_CFG_INT_FIELDS = ("hidden", "layers", "q_heads", "kv_heads", "head_dim", "taps", "target_hidden", "vocab",
                   "block_size", "mask_id", "window", "intermediate", "flush_rows")
_CFG_OPT_FIELDS = ("sel_candidates", "sel_dim")
_CFG_FLAG_FIELDS = ("causal", "qk_norm", "gate", "aux_norms", "ctx_input_norm", "fused_qkv", "attention_bias")


def make_config(cfg) -> abi.Config:
    """dflash_config from any object carrying the same field names."""
    c = abi.Config()
    dt = getattr(cfg, "dtype")
    c.dtype = abi.BF16 if dt in ("bf16", abi.BF16, torch.bfloat16) else abi.FP32
    for n in _CFG_INT_FIELDS:
        setattr(c, n, int(getattr(cfg, n)))
    for n in _CFG_FLAG_FIELDS:
        setattr(c, n, int(bool(getattr(cfg, n, False))))
    for n in _CFG_OPT_FIELDS:
        setattr(c, n, int(getattr(cfg, n, 0)))
    c.rope_theta = float(cfg.rope_theta)
    c.rms_eps = float(cfg.rms_eps)
    return c


def _tensor(t: Optional[torch.Tensor]) -> abi.Tensor:
    out = abi.Tensor()
    if t is None:
        return out
    if not t.is_contiguous():
        raise ValueError("weights must be contiguous")
    out.data = t.data_ptr()
    out.ndim = t.dim()
    for i, s in enumerate(t.shape[:2]):
        out.shape[i] = int(s)
    return out


def _stream_handle(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


class Drafter:
    """A drafter: configuration + borrowed device weights + a shared workspace.

    ``weights`` maps the tensor names of ``dflash_weights`` / ``layers.{l}.*``
    to contiguous device tensors of the configuration's dtype.
    """

    def __init__(self, cfg, weights: Dict[str, torch.Tensor], max_sessions: int = 1,
                 device: str = "cuda"):
        self.lib = abi.load("hip")
        self.cfg = cfg
        self.device = torch.device(device)
        self._weights = weights
        self._c = make_config(cfg)
        W = abi.Weights()
        for n in ("embed", "lm_head", "fc", "hidden_norm", "norm", "aux_norms", "sel_prev", "sel_next"):
            setattr(W, n, _tensor(weights.get(n)))
        L = self._c.layers
        self._layers = (abi.LayerWeights * L)()
        for l in range(L):
            for n in abi.LAYER_FIELDS:
                setattr(self._layers[l], n, _tensor(weights.get(f"layers.{l}.{n}")))
        W.layers = ctypes.cast(self._layers, ctypes.POINTER(abi.LayerWeights))
        self._W = W
        ctx = c_void_p()
        check(self.lib, self.lib.dflash_create(byref(self._c), byref(W), byref(ctx)))
        self.ctx = ctx
        self.max_sessions = int(max_sessions)
        ws = self.lib.dflash_workspace_bytes(ctx, self.max_sessions)
        if ws == 0:
            raise abi.DFlashError(abi.E_ARG, "workspace size")
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=self.device)
        self.feature_dtype = torch.bfloat16 if self._c.dtype == abi.BF16 else torch.float32

    @property
    def draft_limit(self) -> int:
        return self.lib.dflash_draft_limit(self.ctx)

    def session_bytes(self, capacity: int) -> int:
        return int(self.lib.dflash_session_bytes(self.ctx, capacity))

    def session(self, capacity: int, seed: int = 0, stream_id: int = 0, restored_offset: int = 0,
                arena: Optional[torch.Tensor] = None, stream=None) -> "Session":
        return Session(self, capacity, seed, stream_id, restored_offset, arena, stream)

    def close(self):
        if self.ctx:
            self.lib.dflash_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Session:
    def __init__(self, drafter: Drafter, capacity: int, seed: int, stream_id: int, restored_offset: int,
                 arena: Optional[torch.Tensor], stream):
        self.d = drafter
        self.lib = drafter.lib
        nbytes = self.lib.dflash_session_bytes(drafter.ctx, capacity)
        if nbytes == 0:
            raise abi.DFlashError(abi.E_ARG, "session size")
        if arena is None:
            arena = torch.empty(nbytes, dtype=torch.uint8, device=drafter.device)
        self.arena = arena
        self.capacity = capacity
        h = c_void_p()
        check(self.lib, self.lib.dflash_session_open(
            drafter.ctx, arena.data_ptr(), arena.numel() * arena.element_size(), capacity,
            drafter.workspace.data_ptr(), drafter.workspace.numel(), drafter.max_sessions,
            restored_offset, seed, stream_id, _stream_handle(stream), byref(h)))
        self.h = h

    # -- the session calls ---------------------------------------------------
    def committed(self, tokens, features: torch.Tensor, position: int) -> None:
        tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        T = int(tok.shape[0])
        if T and (features.dtype != self.d.feature_dtype or not features.is_contiguous()
                  or features.shape[0] < T or features.device.type != "cuda"):
            raise ValueError("features must be a contiguous device tensor [T, taps*Ht] of the drafter dtype")
        ptr = features.data_ptr() if T else None
        check(self.lib, self.lib.dflash_committed(
            self.h, tok.ctypes.data_as(ctypes.POINTER(c_int32)), ptr, T, int(position)))

    def flush(self) -> None:
        check(self.lib, self.lib.dflash_flush(self.h))

    def commit_block(self) -> None:
        check(self.lib, self.lib.dflash_commit_block(self.h))

    def propose(self, current: int, max_tokens: int, logits: Optional[torch.Tensor] = None,
                hidden: bool = False) -> Tuple[int, torch.Tensor, Optional[torch.Tensor]]:
        cfg = self.d._c
        if logits is None:
            logits = torch.empty((cfg.block_size - 1, cfg.vocab), dtype=torch.float32, device=self.d.device)
        hid = torch.empty((cfg.block_size, cfg.hidden), dtype=torch.float32, device=self.d.device) if hidden else None
        n = c_int32()
        check(self.lib, self.lib.dflash_propose(self.h, int(current), int(max_tokens), logits.data_ptr(),
                                                hid.data_ptr() if hid is not None else None, byref(n)))
        n = n.value
        return n, logits[:n], (hid[:n + 1] if hid is not None else None)

    def state(self) -> Tuple[int, int, int, int]:
        a, b, c, d = c_int32(), c_int32(), c_int32(), c_int32()
        e = c_int64()
        check(self.lib, self.lib.dflash_session_state(self.h, byref(a), byref(b), byref(c), byref(d), byref(e)))
        self._rows_written = e.value
        return a.value, b.value, c.value, d.value

    @property
    def rows_written(self) -> int:
        self.state()
        return self._rows_written

    def cache_read(self, layer: int, position0: int, count: int) -> Tuple[torch.Tensor, torch.Tensor]:
        cfg = self.d._c
        k = torch.empty((count, cfg.kv_heads, cfg.head_dim), dtype=torch.float32, device=self.d.device)
        v = torch.empty_like(k)
        check(self.lib, self.lib.dflash_cache_read(self.h, layer, position0, count, k.data_ptr(), v.data_ptr()))
        return k, v

    def close(self) -> None:
        if self.h:
            h, self.h = self.h, None
            check(self.lib, self.lib.dflash_session_close(h))


def committed_batch(sessions: Sequence[Session], runs: Sequence, features: Sequence[torch.Tensor],
                    positions: Sequence[int]) -> None:
    """dflash_committed_batch: session k commits tokens runs[k] with feature
    rows features[k] (device, [T_k, taps*Ht]) at positions[k]."""
    d = sessions[0].d
    n = len(sessions)
    toks = [np.asarray(r, dtype=np.int32).reshape(-1) for r in runs]
    offs = np.zeros(n + 1, dtype=np.int32)
    offs[1:] = np.cumsum([len(t) for t in toks])
    flat = np.ascontiguousarray(np.concatenate(toks) if offs[-1] else np.zeros(1, dtype=np.int32))
    ptrs = (c_void_p * n)()
    for k, (t, f) in enumerate(zip(toks, features)):
        if len(t) and (f.dtype != d.feature_dtype or not f.is_contiguous() or f.shape[0] < len(t)
                       or f.device.type != "cuda"):
            raise ValueError("features must be contiguous device tensors [T, taps*Ht] of the drafter dtype")
        ptrs[k] = f.data_ptr() if len(t) else None
    hs = (c_void_p * n)(*[s.h for s in sessions])
    pos = (c_int32 * n)(*[int(p) for p in positions])
    check(d.lib, d.lib.dflash_committed_batch(hs, n, flat.ctypes.data_as(ctypes.POINTER(c_int32)),
                                              offs.ctypes.data_as(ctypes.POINTER(c_int32)), ptrs, pos))


def flush_batch(sessions: Sequence[Session]) -> None:
    """dflash_flush_batch: every session's pending rows in one context pass."""
    d = sessions[0].d
    hs = (c_void_p * len(sessions))(*[s.h for s in sessions])
    check(d.lib, d.lib.dflash_flush_batch(hs, len(sessions)))


def propose_batch(sessions: Sequence[Session], current: Sequence[int], max_tokens: Sequence[int],
                  logits: Optional[torch.Tensor] = None) -> Tuple[list, torch.Tensor]:
    d = sessions[0].d
    cfg = d._c
    n = len(sessions)
    if logits is None:
        logits = torch.empty((n * (cfg.block_size - 1), cfg.vocab), dtype=torch.float32, device=d.device)
    hs = (c_void_p * n)(*[s.h for s in sessions])
    cur = (c_int32 * n)(*[int(x) for x in current])
    mt = (c_int32 * n)(*[int(x) for x in max_tokens])
    offs = (c_int32 * (n + 1))()
    check(d.lib, d.lib.dflash_propose_batch(hs, n, cur, mt, logits.data_ptr(), offs))
    return list(offs), logits


def verify(sessions: Sequence[Session], draft_offsets: Sequence[int], target_logits: torch.Tensor,
           draft_ids: Optional[torch.Tensor], draft_probs: Optional[torch.Tensor], temperature: float,
           round: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Speculative verification (dflash_verify): per session, the number of
    accepted drafts and the next token (correction or bonus).  target_logits
    holds n_k + 1 rows per session, draft_ids / draft_probs n_k rows."""
    d = sessions[0].d
    n = len(sessions)
    acc = torch.empty((n,), dtype=torch.int32, device=d.device)
    nxt = torch.empty((n,), dtype=torch.int32, device=d.device)
    for t, dt in ((target_logits, torch.float32), (draft_ids, torch.int32), (draft_probs, torch.float32)):
        if t is not None and (not t.is_contiguous() or t.device.type != "cuda" or t.dtype != dt):
            raise ValueError("verify operands: contiguous device tensors, fp32 logits / probabilities, int32 ids")
    hs = (c_void_p * n)(*[s.h for s in sessions])
    offs = (c_int32 * (n + 1))(*[int(x) for x in draft_offsets])
    p = abi.VerifyParams(float(temperature), int(round))
    check(d.lib, d.lib.dflash_verify(hs, n, offs, target_logits.data_ptr(),
                                     draft_ids.data_ptr() if draft_ids is not None else None,
                                     draft_probs.data_ptr() if draft_probs is not None else None,
                                     byref(p), acc.data_ptr(), nxt.data_ptr()))
    return acc, nxt


def select(sessions: Sequence[Session], row_offsets: Sequence[int], logits: torch.Tensor, current: Sequence[int],
           temperature: float, round: int = 0, dense: bool = False):
    """dflash_select (the DFlash2 candidate selector): per session, its rows'
    tokens chosen in order, each conditioned on the one before (the anchor
    first), with the candidates and their probabilities.  Returns (tokens
    [R], candidate ids [R, K], candidate probabilities [R, K] or None, dense
    probability rows [R, V] or None)."""
    d = sessions[0].d
    n = len(sessions)
    K = d._c.sel_candidates
    R = int(row_offsets[n])
    tok = torch.empty((max(R, 1),), dtype=torch.int32, device=d.device)
    cid = torch.empty((max(R, 1), max(K, 1)), dtype=torch.int32, device=d.device)
    cpr = torch.empty((max(R, 1), max(K, 1)), dtype=torch.float32, device=d.device) if temperature > 0 else None
    den = torch.empty((max(R, 1), d._c.vocab), dtype=torch.float32, device=d.device) if dense and temperature > 0 \
        else None
    if not logits.is_contiguous() or logits.dtype != torch.float32 or logits.device.type != "cuda":
        raise ValueError("logits: contiguous fp32 device tensor [R, V]")
    hs = (c_void_p * n)(*[s.h for s in sessions])
    offs = (c_int32 * (n + 1))(*[int(x) for x in row_offsets])
    cur = (c_int32 * n)(*[int(x) for x in current])
    p = abi.SelectParams(float(temperature), int(round))
    check(d.lib, d.lib.dflash_select(hs, n, offs, logits.data_ptr(), cur, byref(p), tok.data_ptr(), cid.data_ptr(),
                                     cpr.data_ptr() if cpr is not None else None,
                                     den.data_ptr() if den is not None else None))
    return tok[:R], cid[:R], (cpr[:R] if cpr is not None else None), (den[:R] if den is not None else None)


def verify_noalloc(sessions: Sequence[Session], draft_offsets: Sequence[int], target_logits: torch.Tensor,
                   draft_ids: Optional[torch.Tensor], draft_probs: Optional[torch.Tensor], temperature: float,
                   round: int, accepted_out: torch.Tensor, next_out: torch.Tensor) -> None:
    """dflash_verify_noalloc: as ``verify`` into the caller's int32 device
    outputs, with the library's static scratch array instead of a workspace
    (nothing is allocated, here or in the library)."""
    d = sessions[0].d
    n = len(sessions)
    for t, dt in ((target_logits, torch.float32), (draft_ids, torch.int32), (draft_probs, torch.float32),
                  (accepted_out, torch.int32), (next_out, torch.int32)):
        if t is not None and (not t.is_contiguous() or t.device.type != "cuda" or t.dtype != dt):
            raise ValueError("verify operands: contiguous device tensors, fp32 logits / probabilities, int32 ids")
    if accepted_out.numel() < n or next_out.numel() < n:
        raise ValueError("outputs need one entry per session")
    hs = (c_void_p * n)(*[s.h for s in sessions])
    offs = (c_int32 * (n + 1))(*[int(x) for x in draft_offsets])
    p = abi.VerifyParams(float(temperature), int(round))
    check(d.lib, d.lib.dflash_verify_noalloc(hs, n, offs, target_logits.data_ptr(),
                                             draft_ids.data_ptr() if draft_ids is not None else None,
                                             draft_probs.data_ptr() if draft_probs is not None else None,
                                             byref(p), accepted_out.data_ptr(), next_out.data_ptr()))


def sample(sessions: Sequence[Session], row_offsets: Sequence[int], logits: torch.Tensor, temperature: float,
           rep_penalty: float = 1.0, history: int = 512, round: int = 0,
           probs: bool = False) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    d = sessions[0].d
    n = len(sessions)
    R = int(row_offsets[n])
    ids = torch.empty((max(R, 1),), dtype=torch.int32, device=d.device)
    pr = None
    if probs and temperature > 0:
        pr = torch.empty((max(R, 1), d._c.vocab), dtype=torch.float32, device=d.device)
    hs = (c_void_p * n)(*[s.h for s in sessions])
    offs = (c_int32 * (n + 1))(*[int(x) for x in row_offsets])
    p = abi.SampleParams(float(temperature), float(rep_penalty), int(history), int(round))
    check(d.lib, d.lib.dflash_sample(hs, n, offs, logits.data_ptr(), byref(p), ids.data_ptr(),
                                     pr.data_ptr() if pr is not None else None))
    return ids[:R], (pr[:R] if pr is not None else None)


class WidthPolicy:
    """Draft width controller (dflash_width_policy_*): per-position acceptance
    estimates and the width that maximises expected emitted tokens per unit of
    round time.  Host-only; ``lib`` defaults to the HIP library."""

    def __init__(self, max_width: int, draft_fixed: float, draft_per_row: float, verify_fixed: float = 0.0,
                 verify_per_row: float = 0.0, decay: float = 0.95, lib=None):
        self.lib = lib if lib is not None else abi.load("hip")
        self.max_width = int(max_width)
        h = c_void_p()
        check(self.lib, self.lib.dflash_width_policy_create(self.max_width, float(draft_fixed), float(draft_per_row),
                                                            float(verify_fixed), float(verify_per_row),
                                                            float(decay), byref(h)))
        self.h = h.value

    def observe(self, drafted: int, accepted: int) -> None:
        check(self.lib, self.lib.dflash_width_policy_observe(self.h, int(drafted), int(accepted)))

    def choose(self) -> int:
        n = self.lib.dflash_width_policy_choose(self.h)
        if n < 0:
            check(self.lib, n)
        return n

    def rates(self) -> list:
        buf = (ctypes.c_float * self.max_width)()
        check(self.lib, self.lib.dflash_width_policy_rates(self.h, buf))
        return list(buf)

    def close(self) -> None:
        if self.h:
            h, self.h = self.h, None
            self.lib.dflash_width_policy_destroy(h)

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001
            pass
