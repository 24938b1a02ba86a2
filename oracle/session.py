"""The drafting session's state machine (test infrastructure only).

Restates Ollama ``mlxrunner/dflash.go`` (type ``dflashDraftSession`` and its
methods ``committed``, ``flush``, ``takePending``, ``commitBlock`` and
``propose``):

* ``committed``: the run starts ``start = ctxOffset + pending - position``
  rows into what the session already holds; ``start < 0`` would leave a gap in
  the draft context and is refused; rows ``[start, T)`` join the pending
  buffer, and reaching the pending bound (256 rows there) flushes.
* ``flush``: rewind any outstanding block first (even with nothing pending),
  then write every pending row in one context-only forward and advance
  ``ctxOffset`` past them.
* ``commitBlock``: when a block is outstanding, cut the cache back to
  ``ctxOffset``; a no-op otherwise.
* ``propose``: ``n = min(maxTokens, blockSize-1)``; nothing when ``n <= 0`` or
  no context was ever committed; otherwise rewind, take the pending rows into
  the same forward, schedule the block at the new frontier and run the block
  forward.

The one deliberate change: a gap is reported as ``ContextGap`` with the state
untouched instead of a panic.  The Laguna drop-before-fc rule (mlxcel PR
"add the Laguna DFlash drafter", review commit "trim the hot path") skips
context rows that no later query can see: slots below
``frontier - (window - 1)``.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np

from .model import DraftModel, PositionCache


class ContextGap(Exception):
    pass


class OracleSession:
    def __init__(self, model: DraftModel, restored_offset: int = 0):
        self.model = model
        self.cfg = model.cfg
        self.ctx_offset = int(restored_offset)
        self.pending_feats: List[np.ndarray] = []
        self.pending_count = 0
        self.outstanding = False
        self.cache_len = int(restored_offset)
        self.cache = PositionCache(self.cfg)
        self.history: List[int] = []
        self.rows_written = 0

    # -- state ---------------------------------------------------------------
    def state(self):
        return (self.ctx_offset, self.pending_count, self.cache_len, int(self.outstanding))

    # -- committed / flush ---------------------------------------------------
    def committed(self, tokens, feats, position: int) -> None:
        tokens = np.asarray(tokens)
        T = int(tokens.shape[0])
        start = self.ctx_offset + self.pending_count - int(position)
        if start < 0:
            raise ContextGap(f"committed run at {position} leaves a context gap at "
                             f"{self.ctx_offset + self.pending_count}")
        if start < T:
            self.pending_feats.append(np.asarray(feats[start:T]))
            self.history.extend(int(t) for t in tokens[start:T])
            self.pending_count += T - start
            if self.pending_count >= self.cfg.flush_rows:
                self.flush()

    def commit_block(self) -> None:
        if not self.outstanding:
            return
        self.cache_len = self.ctx_offset
        self.outstanding = False

    def _take_pending(self) -> None:
        """Write the pending rows to the cache and advance ctxOffset past them."""
        P = self.pending_count
        if P == 0:
            return
        feats = np.concatenate(self.pending_feats, axis=0)
        positions = self.ctx_offset + np.arange(P)
        frontier = self.ctx_offset + P
        keep = np.ones(P, dtype=bool)
        if self.cfg.window:
            keep = positions >= frontier - (self.cfg.window - 1)
        if keep.any():
            kv = self.model.context_kv(feats[keep], positions[keep])
            for l, (K, V) in enumerate(kv):
                self.cache.write(l, positions[keep], K, V)
            self.rows_written += int(keep.sum())
        self.pending_feats = []
        self.pending_count = 0
        self.ctx_offset = frontier
        self.cache_len = frontier

    def flush(self) -> None:
        self.commit_block()
        self._take_pending()

    # -- propose -------------------------------------------------------------
    def propose(self, current: int, max_tokens: int) -> Optional[dict]:
        n = min(int(max_tokens), self.cfg.block_size - 1)
        if n <= 0 or self.ctx_offset + self.pending_count == 0:
            return None
        self.commit_block()
        self._take_pending()
        F = self.ctx_offset
        tokens = [int(current)] + [self.cfg.mask_id] * n
        self.cache_len = F + n + 1
        self.outstanding = True
        out = self.model.block_forward(tokens, F, self.cache)
        out["n"] = n
        out["F"] = F
        return out

    # -- readback ------------------------------------------------------------
    def cache_kv(self, layer: int, positions):
        positions = np.asarray(positions, dtype=np.int64)
        return self.cache.k[layer][positions], self.cache.v[layer][positions]
