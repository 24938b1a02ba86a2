"""Float64 forward of the DFlash drafter (test infrastructure only).

What the pages fix, and where:

* Ollama ``mlxrunner/dflash.go`` (type ``dflashDraftSession`` comment and
  ``propose``/``selectBlock``): a context entry at slot S derives only from
  the target features at S; the block is the anchor token plus n mask tokens
  in one forward; row i predicts the token at its own position, so rows
  1..n are unembedded and the anchor row is dropped.
* mlxcel PR "add the Laguna DFlash drafter" (PR body; review commits "trim the
  hot path"): the context path is ``aux_hidden_norms`` -> ``fc`` ->
  ``hidden_norm``; each layer passes the context through its own
  ``input_layernorm`` before a K/V-only projection; attention is fused-QKV
  with a per-head sigmoid gate and a per-query sliding window over
  [context | block]; context rows older than the window are dropped before
  ``fc``; no attention bias.

Readings where the pages are silent (each one is a config switch, listed with
reasons in the design notes): Qwen3-style decoder layer (pre-norm attention
with per-head q/k RMSNorm and rotate-half RoPE, SwiGLU MLP, residuals around
both); RMSNorm y = x / sqrt(mean(x^2)+eps) * g; RoPE position = slot; key s is
visible to query p iff p - s < W; separate embedding and unembedding tables
with a final RMSNorm before the unembedding; fused qkv rows ordered q | k | v;
gate = sigmoid of one ``g_proj`` scalar per q head, multiplied into that
head's attention output before ``o_proj``.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

import numpy as np

from .numerics import rms_norm, rope, round_bf16, sigmoid, silu, softmax


class DraftModel:
    """The drafter's weights plus its two forwards, in float64."""

    def __init__(self, cfg, weights: Dict[str, np.ndarray], emulate_bf16: bool = False):
        self.cfg = cfg
        self.w = weights
        self.emulate = bool(emulate_bf16 and cfg.dtype == "bf16")
        self._small: Dict[str, np.ndarray] = {}

    # -- helpers -------------------------------------------------------------
    def st(self, x: np.ndarray) -> np.ndarray:
        """A value the GPU stores in bf16: rounded in emulation mode."""
        return round_bf16(x) if self.emulate else np.asarray(x, dtype=np.float64)

    def g(self, name: str) -> np.ndarray:
        if name not in self._small:
            self._small[name] = np.asarray(self.w[name], dtype=np.float64)
        return self._small[name]

    def lin(self, x: np.ndarray, name: str, row0: int = 0, rows: Optional[int] = None) -> np.ndarray:
        """x @ W[row0:row0+rows].T with W upcast to float64 piecewise."""
        W = self.w[name]
        if rows is None:
            rows = W.shape[0] - row0
        out = np.empty((x.shape[0], rows), dtype=np.float64)
        step = max(1, (1 << 25) // W.shape[1])
        for r in range(0, rows, step):
            e = min(rows, r + step)
            out[:, r:e] = x @ np.asarray(W[row0 + r:row0 + e], dtype=np.float64).T
        return out

    def _proj(self, x: np.ndarray, l: int, part: str) -> np.ndarray:
        """q, k or v projection of layer l (a row slice of qkv_proj when fused)."""
        c = self.cfg
        qd, kd = c.q_heads * c.head_dim, c.kv_heads * c.head_dim
        p = f"layers.{l}."
        if c.fused_qkv:
            off = {"q": 0, "k": qd, "v": qd + kd}[part]
            return self.lin(x, p + "qkv_proj", off, qd if part == "q" else kd)
        return self.lin(x, p + part + "_proj")

    # -- context path --------------------------------------------------------
    def context_kv(self, feats: np.ndarray, positions) -> List[Tuple[np.ndarray, np.ndarray]]:
        """K/V cache entries of context rows.

        ``feats`` is [P, taps*Ht] (taps in target-layer order), ``positions``
        the P slots.  Returns, per layer, K and V of shape [P, Hkv, D].  Row r
        depends on ``feats[r]`` and ``positions[r]`` only.
        """
        c = self.cfg
        P = feats.shape[0]
        pos = np.asarray(positions, dtype=np.int64)
        f = np.asarray(feats, dtype=np.float64)
        if c.aux_norms:
            f = f.reshape(P, c.taps, c.target_hidden)
            f = rms_norm(f, self.g("aux_norms"), c.rms_eps).reshape(P, c.fc_in)
        h = self.lin(self.st(f), "fc")
        h = rms_norm(h, self.g("hidden_norm"), c.rms_eps)
        out = []
        for l in range(c.layers):
            x = h
            if c.ctx_input_norm:
                x = rms_norm(h, self.g(f"layers.{l}.input_layernorm"), c.rms_eps)
            x = self.st(x)
            k = self._proj(x, l, "k").reshape(P, c.kv_heads, c.head_dim)
            v = self._proj(x, l, "v").reshape(P, c.kv_heads, c.head_dim)
            if c.qk_norm:
                k = rms_norm(k, self.g(f"layers.{l}.k_norm"), c.rms_eps)
            k = rope(k, pos, c.rope_theta)
            out.append((self.st(k), self.st(v)))
        return out

    # -- block path ----------------------------------------------------------
    def visible(self, F: int, M: int, i: int, s: int) -> bool:
        """Is key position s visible to block row i (query position F+i)?"""
        c = self.cfg
        p = F + i
        if s < 0 or s >= F + M:
            return False
        if s >= F and c.causal and s > p:
            return False
        if c.window and p - s >= c.window:
            return False
        return True

    def block_forward(self, tokens, F: int, cache) -> Dict[str, np.ndarray]:
        """Forward of the block [anchor, mask x n] at positions F..F+n.

        ``cache`` has ``k[l]``/``v[l]`` arrays indexed by absolute position
        ([positions, Hkv, D]) and a ``write(l, positions, K, V)`` method; the
        block's own K/V are written there first (the block is scheduled into
        the draft cache), then every row attends over the visible positions.
        Returns the last hidden state [M, H] and logits of rows 1..n [n, V].
        """
        c = self.cfg
        tokens = np.asarray(tokens, dtype=np.int64)
        M = tokens.shape[0]
        D, Hq, Hkv = c.head_dim, c.q_heads, c.kv_heads
        G = Hq // Hkv
        pos = F + np.arange(M)
        h = np.asarray(self.w["embed"][tokens], dtype=np.float64)
        for l in range(c.layers):
            p = f"layers.{l}."
            x = self.st(rms_norm(h, self.g(p + "input_layernorm"), c.rms_eps))
            q = self._proj(x, l, "q").reshape(M, Hq, D)
            k = self._proj(x, l, "k").reshape(M, Hkv, D)
            v = self._proj(x, l, "v").reshape(M, Hkv, D)
            if c.qk_norm:
                q = rms_norm(q, self.g(p + "q_norm"), c.rms_eps)
                k = rms_norm(k, self.g(p + "k_norm"), c.rms_eps)
            q = self.st(rope(q, pos, c.rope_theta))
            k = self.st(rope(k, pos, c.rope_theta))
            cache.write(l, pos, k, self.st(v))
            K, V = cache.k[l], cache.v[l]
            a = np.zeros((M, Hq, D))
            scale = 1.0 / np.sqrt(D)
            for i in range(M):
                keys = [s for s in range(max(0, F + i - c.window + 1) if c.window else 0, F + M)
                        if self.visible(F, M, i, s)]
                for hq in range(Hq):
                    gk = hq // G
                    kk = K[keys, gk, :]
                    vv = V[keys, gk, :]
                    pr = softmax(kk @ q[i, hq] * scale)
                    a[i, hq] = pr @ vv
            if c.gate:
                gate = sigmoid(self.lin(x, p + "g_proj"))
                a = a * gate[:, :, None]
            a = self.st(a).reshape(M, Hq * D)
            h = h + self.lin(a, p + "o_proj")
            x2 = self.st(rms_norm(h, self.g(p + "post_attention_layernorm"), c.rms_eps))
            mlp = self.st(silu(self.lin(x2, p + "gate_proj")) * self.lin(x2, p + "up_proj"))
            h = h + self.lin(mlp, p + "down_proj")
        z = self.lin(self.st(rms_norm(h[1:], self.g("norm"), c.rms_eps)), "lm_head")
        return {"hidden": h, "logits": z}


class PositionCache:
    """Draft K/V cache addressed by absolute position (NaN where never written).

    The GPU keeps a ring for windowed configs; the logical content at every
    position still visible is the same, and reading an entry the window drop
    never computed propagates NaN, so such a read cannot go unnoticed.
    """

    def __init__(self, cfg, capacity: int = 64):
        self.cfg = cfg
        shape = (capacity, cfg.kv_heads, cfg.head_dim)
        self.k = [np.full(shape, np.nan) for _ in range(cfg.layers)]
        self.v = [np.full(shape, np.nan) for _ in range(cfg.layers)]

    def _grow(self, need: int):
        cap = self.k[0].shape[0]
        if need <= cap:
            return
        new = max(need, 2 * cap)
        for arrs in (self.k, self.v):
            for l, a in enumerate(arrs):
                b = np.full((new,) + a.shape[1:], np.nan)
                b[:cap] = a
                arrs[l] = b

    def write(self, l: int, positions, K: np.ndarray, V: np.ndarray):
        positions = np.asarray(positions, dtype=np.int64)
        if positions.size == 0:
            return
        self._grow(int(positions.max()) + 1)
        self.k[l][positions] = K
        self.v[l][positions] = V
