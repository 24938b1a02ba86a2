"""Seeded synthetic inputs for the DFlash block-diffusion drafter forward.

This module is data only: model shapes, seeded weights, seeded target-tap
features, seeded token streams and the synthetic round script.  It holds none
of the drafter's arithmetic.  Both the CPU oracle (``oracle/``) and the HIP
path (``block_diffusion_drafter_fwd_amd``) read their inputs from here and
from nowhere else they share.

The pages give no checkpoint, data or prompts (Ollama ``mlxrunner/dflash.go``
and mlxcel PR #1771 measure on real checkpoints and code prompts), so every
tensor is drawn from a counter-keyed NumPy PCG64 stream:

* weight ``name`` of shape S: N(0, 0.02), drawn in 2**24-element pieces, piece
  ``j`` from ``default_rng([seed, crc32(name), j])``; bf16 configurations
  round the value to bf16 (round-to-nearest-even) so that both sides see the
  same bf16 numbers.
* RMSNorm gains: 1.0 (``gains="unit"``) or U(0.5, 1.5) (``gains="random"``)
  so that every norm is exercised in parity tests.
* tap features of session ``s`` at absolute position ``S``: row ``S % 256`` of
  a [256, taps*Ht] N(0, 1) block drawn from ``default_rng([seed, 7, s,
  S // 256])`` (bf16-rounded for bf16 configurations).
* committed tokens at position ``S``: U{0..V-2} from the same kind of block
  stream (key ``[seed, 11, s, S // 256]``); the mask id V-1 never appears.
"""
from __future__ import annotations

import dataclasses
import math
import threading
import zlib
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = [
    "DraftConfig", "Workload", "CONFIGS", "WORKLOADS", "config", "weight_specs",
    "make_weights", "bf16_bits", "FeatureSource", "RoundScript", "SyntheticTarget", "session_lengths",
]

_PIECE = 1 << 24          # elements per independently keyed weight piece
_CHUNK = 256              # rows per feature / token block


@dataclasses.dataclass(frozen=True)
class DraftConfig:
    """Shape and switches of one synthetic drafter.

    Field names follow the pages' vocabulary: ``block_size`` and ``mask_id``
    are ``BlockParams()``; ``flush_rows`` is the pending bound that triggers a
    context-only flush; ``window`` is the Laguna sliding window (0 = dense);
    ``gate`` is the per-head sigmoid ``g_proj`` gate; ``aux_norms`` the per-tap
    ``aux_hidden_norms``; ``ctx_input_norm`` the per-layer ``input_layernorm``
    on context rows before their K/V projection; ``fused_qkv`` a single
    ``qkv_proj`` with rows ordered q | k | v.
    """

    name: str
    dtype: str                 # "fp32" | "bf16"
    hidden: int
    layers: int
    q_heads: int
    kv_heads: int
    head_dim: int
    taps: int
    target_hidden: int
    vocab: int
    block_size: int
    intermediate: int
    window: int = 0
    causal: bool = False
    qk_norm: bool = True
    gate: bool = False
    aux_norms: bool = False
    ctx_input_norm: bool = False
    fused_qkv: bool = False
    flush_rows: int = 256
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6
    sel_candidates: int = 0        # DFlash2 selector: candidates per drafted row (0: none)
    sel_dim: int = 0               # DFlash2 selector: width of its two token tables

    @property
    def mask_id(self) -> int:
        return self.vocab - 1

    @property
    def fc_in(self) -> int:
        return self.taps * self.target_hidden

    @property
    def draft_limit(self) -> int:
        return self.block_size - 1

    def replace(self, **kw) -> "DraftConfig":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class Workload:
    """A synthetic run: prompt lengths, rounds and sampling settings."""

    name: str
    config: str
    sessions: int = 1
    context: int = 0               # prompt slots per session (0: per-session draw)
    context_lo: int = 0            # log-uniform draw bounds when sessions > 1
    context_hi: int = 0
    commit_rows: int = 256         # rows per committed() call in the prompt phase
    rounds: int = 20
    max_tokens: int = 0            # 0: block_size - 1; -1: per-session U{1..B-1}
    temperature: float = 0.0
    rep_penalty: float = 1.0
    history: int = 512
    probs: bool = False
    flush_fraction: float = 0.0    # share of sessions calling flush before a batched propose


_TINY = DraftConfig(
    name="tiny", dtype="fp32", hidden=64, layers=2, q_heads=4, kv_heads=4, head_dim=16,
    taps=5, target_hidden=64, vocab=32, block_size=8, intermediate=192, causal=True,
    flush_rows=16)

CONFIGS: Dict[str, DraftConfig] = {
    "tiny": _TINY,
    # tiny scale with every Laguna switch on (window 6, gate, aux norms,
    # context input_layernorm, fused qkv) for forced-accept scripts
    "tiny_w": _TINY.replace(name="tiny_w", window=6, gate=True, aux_norms=True,
                            ctx_input_norm=True, fused_qkv=True, causal=False),
    "qwen": DraftConfig(
        name="qwen", dtype="bf16", hidden=2048, layers=5, q_heads=32, kv_heads=8,
        head_dim=128, taps=5, target_hidden=2048, vocab=151936, block_size=16,
        intermediate=6144),
    "laguna": DraftConfig(
        name="laguna", dtype="bf16", hidden=2048, layers=4, q_heads=16, kv_heads=4,
        head_dim=128, taps=5, target_hidden=2048, vocab=100352, block_size=8,
        intermediate=6144, window=512, gate=True, aux_norms=True,
        ctx_input_norm=True, fused_qkv=True),
    "long": DraftConfig(
        name="long", dtype="bf16", hidden=4096, layers=5, q_heads=32, kv_heads=8,
        head_dim=128, taps=5, target_hidden=4096, vocab=262144, block_size=8,
        intermediate=12288),
}

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", "tiny", context=48, commit_rows=16, rounds=20),
    "tiny_w": Workload("tiny_w", "tiny_w", context=48, commit_rows=16, rounds=20),
    "qwen": Workload("qwen", "qwen", context=4096, rounds=200),
    "laguna": Workload("laguna", "laguna", context=32768, rounds=200),
    "batched": Workload("batched", "qwen", sessions=64, context_lo=1024, context_hi=16384,
                        rounds=50, max_tokens=-1, temperature=0.7, rep_penalty=1.1,
                        history=512, flush_fraction=0.25),
    "long": Workload("long", "long", context=131072, rounds=200, max_tokens=7,
                     temperature=1.0, probs=True),
}


def config(name: str, **overrides) -> DraftConfig:
    cfg = CONFIGS[name]
    return cfg.replace(**overrides) if overrides else cfg


# --------------------------------------------------------------------------
# weights
# --------------------------------------------------------------------------

def weight_specs(cfg: DraftConfig) -> List[Tuple[str, Tuple[int, ...], str]]:
    """(name, shape, kind) for every drafter tensor; kind is 'normal' or 'gain'.

    Linear weights are [out_features, in_features].
    """
    H, D = cfg.hidden, cfg.head_dim
    qd, kd = cfg.q_heads * D, cfg.kv_heads * D
    specs: List[Tuple[str, Tuple[int, ...], str]] = [
        ("embed", (cfg.vocab, H), "normal"),
        ("lm_head", (cfg.vocab, H), "normal"),
        ("fc", (H, cfg.fc_in), "normal"),
        ("hidden_norm", (H,), "gain"),
        ("norm", (H,), "gain"),
    ]
    if cfg.aux_norms:
        specs.append(("aux_norms", (cfg.taps, cfg.target_hidden), "gain"))
    if cfg.sel_candidates:
        specs += [("sel_prev", (cfg.vocab, cfg.sel_dim), "normal"), ("sel_next", (cfg.vocab, cfg.sel_dim), "normal")]
    for l in range(cfg.layers):
        p = f"layers.{l}."
        specs += [(p + "input_layernorm", (H,), "gain"),
                  (p + "post_attention_layernorm", (H,), "gain")]
        if cfg.fused_qkv:
            specs.append((p + "qkv_proj", (qd + 2 * kd, H), "normal"))
        else:
            specs += [(p + "q_proj", (qd, H), "normal"), (p + "k_proj", (kd, H), "normal"),
                      (p + "v_proj", (kd, H), "normal")]
        if cfg.qk_norm:
            specs += [(p + "q_norm", (D,), "gain"), (p + "k_norm", (D,), "gain")]
        if cfg.gate:
            specs.append((p + "g_proj", (cfg.q_heads, H), "normal"))
        specs += [(p + "o_proj", (H, qd), "normal"),
                  (p + "gate_proj", (cfg.intermediate, H), "normal"),
                  (p + "up_proj", (cfg.intermediate, H), "normal"),
                  (p + "down_proj", (H, cfg.intermediate), "normal")]
    return specs


def _round_to_bf16_values(x: np.ndarray) -> np.ndarray:
    """float32 -> float32 holding the nearest bf16 value (ties to even)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of a float32 array whose values are bf16-exact."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("array holds values that are not bf16-representable")
    return (u >> np.uint32(16)).astype(np.uint16)


def _draw_normal(seed: int, name: str, shape, std: float, bf16: bool,
                 threads: int = 8) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    key = zlib.crc32(name.encode())
    pieces = list(range((n + _PIECE - 1) // _PIECE))

    def work(js):
        for j in js:
            lo, hi = j * _PIECE, min(n, (j + 1) * _PIECE)
            v = np.random.default_rng([seed, key, j]).standard_normal(hi - lo, dtype=np.float32)
            v *= np.float32(std)
            out[lo:hi] = _round_to_bf16_values(v) if bf16 else v

    if len(pieces) <= 1 or threads <= 1:
        work(pieces)
    else:
        groups = [pieces[i::threads] for i in range(threads)]
        ths = [threading.Thread(target=work, args=(g,)) for g in groups if g]
        for t in ths:
            t.start()
        for t in ths:
            t.join()
    return out.reshape(shape)


def make_weights(cfg: DraftConfig, seed: int = 0, gains: str = "unit",
                 std: float = 0.02) -> Dict[str, np.ndarray]:
    """All drafter tensors as float32 arrays (bf16-exact values for bf16 configs)."""
    bf16 = cfg.dtype == "bf16"
    w: Dict[str, np.ndarray] = {}
    for name, shape, kind in weight_specs(cfg):
        if kind == "normal":
            w[name] = _draw_normal(seed, name, shape, std, bf16)
        elif gains == "unit":
            w[name] = np.ones(shape, dtype=np.float32)
        else:
            g = np.random.default_rng([seed, zlib.crc32(name.encode()), 99]).uniform(
                0.5, 1.5, size=shape).astype(np.float32)
            w[name] = _round_to_bf16_values(g) if bf16 else g
    return w


# --------------------------------------------------------------------------
# features and tokens, addressed by absolute position
# --------------------------------------------------------------------------

class FeatureSource:
    """Target-tap feature rows and committed tokens of one session.

    Row ``S`` is fixed by (seed, session, S) alone, so any slice can be drawn
    in any order and both sides see identical values.
    """

    def __init__(self, cfg: DraftConfig, seed: int = 0, session: int = 0):
        self.cfg = cfg
        self.seed = seed
        self.session = session
        self._cache: Dict[Tuple[str, int], np.ndarray] = {}

    def _block(self, kind: str, c: int) -> np.ndarray:
        k = (kind, c)
        if k not in self._cache:
            if len(self._cache) > 8:
                self._cache.clear()
            if kind == "f":
                rng = np.random.default_rng([self.seed, 7, self.session, c])
                v = rng.standard_normal((_CHUNK, self.cfg.fc_in), dtype=np.float32)
                if self.cfg.dtype == "bf16":
                    v = _round_to_bf16_values(v).reshape(_CHUNK, self.cfg.fc_in)
            else:
                rng = np.random.default_rng([self.seed, 11, self.session, c])
                v = rng.integers(0, self.cfg.vocab - 1, size=_CHUNK, dtype=np.int32)
            self._cache[k] = v
        return self._cache[k]

    def _rows(self, kind: str, first: int, count: int) -> np.ndarray:
        parts = []
        s = first
        end = first + count
        while s < end:
            c, o = divmod(s, _CHUNK)
            take = min(end - s, _CHUNK - o)
            parts.append(self._block(kind, c)[o:o + take])
            s += take
        if not parts:
            shape = (0, self.cfg.fc_in) if kind == "f" else (0,)
            return np.zeros(shape, dtype=np.float32 if kind == "f" else np.int32)
        return np.ascontiguousarray(np.concatenate(parts, axis=0))

    def features(self, first: int, count: int) -> np.ndarray:
        return self._rows("f", first, count)

    def tokens(self, first: int, count: int) -> np.ndarray:
        return self._rows("t", first, count)


def session_lengths(wl: Workload, seed: int = 0) -> List[int]:
    """Prompt length of every session: fixed, or log-uniform in [lo, hi]."""
    if wl.sessions == 1 or wl.context:
        return [wl.context] * wl.sessions
    rng = np.random.default_rng([seed, 13])
    u = rng.uniform(math.log(wl.context_lo), math.log(wl.context_hi), size=wl.sessions)
    return [int(round(math.exp(x))) for x in u]


class RoundScript:
    """The synthetic round driver of one session.

    Per round: the caller proposes ``n`` rows; the script draws an accept
    length ``a`` in U{0..n}; the committed run is the anchor token plus ``a``
    seeded tokens (the script does not feed drafted ids back, so both sides
    stay on identical inputs whatever they draft); the next anchor is a seeded
    bonus token in U{0..V-2}.
    """

    def __init__(self, cfg: DraftConfig, wl: Workload, seed: int = 0, session: int = 0):
        self.cfg = cfg
        self.rng = np.random.default_rng([seed, 17, session])
        if wl.max_tokens == -1:
            self.max_tokens = int(self.rng.integers(1, cfg.block_size))
        elif wl.max_tokens == 0:
            self.max_tokens = cfg.block_size - 1
        else:
            self.max_tokens = wl.max_tokens
        self.flush_before = bool(self.rng.uniform() < wl.flush_fraction)

    def first_anchor(self) -> int:
        return int(self.rng.integers(0, self.cfg.vocab - 1))

    def accept(self, n: int) -> int:
        return int(self.rng.integers(0, n + 1))

    def bonus(self) -> int:
        return int(self.rng.integers(0, self.cfg.vocab - 1))


class SyntheticTarget:
    """Stand-in for the target model of a verification round (no checkpoint is
    here): the logits of the n + 1 positions that follow a drafted block.

    Row i (the token after block position i; row n is the bonus position) is
    N(0, sigma) noise drawn from ``default_rng([seed, 23, session, round])``
    plus ``boost`` on one preferred token: for a row below n, with
    probability ``agree`` (a seeded coin from the same stream) the token the
    draft proposed there, else a seeded token; for row n always a seeded
    token.  With boost well above the noise's maximum the preferred token is
    the row's argmax, so a greedy round accepts the drafts up to the first
    coin that came up "disagree" (expected accepted drafts
    sum_{j<=n} agree^j), and a sampling round accepts a draft about as often.
    It depends only on the seeds, the round and the drafted ids, so two
    drafters that draft the same ids see the same target.
    """

    def __init__(self, vocab: int, seed: int = 0, session: int = 0, sigma: float = 1.0,
                 boost: float = 10.0, agree: float = 0.7):
        self.vocab, self.seed, self.session = vocab, seed, session
        self.sigma, self.boost, self.agree = sigma, boost, agree

    def draws(self, rnd: int, n: int):
        """(noise [n+1, V], coins [n] (True: prefer the draft), random tokens [n+1])."""
        rng = np.random.default_rng([self.seed, 23, self.session, rnd])
        noise = rng.standard_normal((n + 1, self.vocab), dtype=np.float32) * np.float32(self.sigma)
        coins = rng.uniform(size=n) < self.agree
        toks = rng.integers(0, self.vocab - 1, size=n + 1)
        return noise, coins, toks

    def rows(self, rnd: int, drafted) -> np.ndarray:
        """Target logits [n + 1, V] (float32) for the drafted ids of a round."""
        drafted = np.asarray(drafted, dtype=np.int64).reshape(-1)
        n = drafted.size
        noise, coins, toks = self.draws(rnd, n)
        pref = np.where(coins, drafted, toks[:n]) if n else np.zeros(0, np.int64)
        noise[np.arange(n), pref] += np.float32(self.boost)
        noise[n, toks[n]] += np.float32(self.boost)
        return noise
