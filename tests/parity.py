"""Lock-step parity driver: the HIP library (through its C ABI) against the
float64 oracle, on identical seeded inputs from ``synth``.

Compared after every call: the session state (ctxOffset, pending, cache
length, outstanding block, rows projected) bit-exactly; logits, the block
hidden state, probabilities and cache K/V within the relative tolerance
(max |gpu - ref| / max |ref|: 2e-2 bf16, 1e-4 fp32); token ids exactly
wherever the oracle's top-1/top-2 score gap exceeds the tie margin (one bf16
ulp of the top score for bf16, 1e-4 of it for fp32; divided by the
temperature when sampling).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

import synth
from oracle.model import DraftModel
from oracle.sampler import sample_row, top2_gap
from oracle.session import ContextGap as OracleGap, OracleSession
from tests.helpers import rel_err


def tol(cfg) -> float:
    return 2e-2 if cfg.dtype == "bf16" else 1e-4


def probs_tol(z_gpu, z_ref, temperature: float) -> float:
    """Bound on max|p_gpu - p_ref| / max p_ref implied by the logit deviation.

    softmax(z/T) moves by at most a factor exp(2 max|dz| / T) when the logits
    move by dz, so probabilities are held to that (plus float32 rounding of
    the exponentials); the logit deviation itself is held to the logits
    tolerance separately.
    """
    dz = float(np.max(np.abs(np.asarray(z_gpu, dtype=np.float64) - np.asarray(z_ref, dtype=np.float64))))
    return math.expm1(2.0 * dz / temperature) + 1e-4


def margin(cfg, top: float, temperature: float = 0.0) -> float:
    top = abs(top)
    if cfg.dtype == "bf16":
        m = 2.0 ** (math.floor(math.log2(top)) - 7) if top > 0 else 0.0
    else:
        m = 1e-4 * top
    return m / temperature if temperature > 0 else m


def device_tensors(cfg, arrays: dict, device="cuda") -> dict:
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(device=device).to(dt) for k, v in arrays.items()}


def feats_dev(cfg, f: np.ndarray, device="cuda") -> torch.Tensor:
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    return torch.from_numpy(np.ascontiguousarray(f)).to(device=device).to(dt)


@dataclass
class Report:
    worst: dict = field(default_factory=dict)
    ids_compared: int = 0
    ids_skipped: int = 0
    rounds: int = 0
    greedy_compared: int = 0
    greedy_skipped: int = 0
    sampled_compared: int = 0
    sampled_skipped: int = 0
    sampled_expected_skips: float = 0.0   # sum over sampled rows of P(top-2 gap <= margin)
    greedy_expected_skips: float = 0.0    # the same for greedy rows (spacing model of the top logits)

    def note(self, key, value):
        self.worst[key] = max(self.worst.get(key, 0.0), value)

    def skip_bound_ok(self) -> bool:
        """Skipped rows within their expected tie counts (plus Poisson slack):
        sampled rows from the exact Gumbel-max tie probability, greedy rows
        from the spacing model of the top logits."""
        def ok(skipped, e):
            return skipped <= e + 3.0 * math.sqrt(e) + 2.0
        return ok(self.sampled_skipped, self.sampled_expected_skips) and \
            ok(self.greedy_skipped, self.greedy_expected_skips)

    def summary(self, name: str) -> dict:
        return {"case": name, "rounds": self.rounds, "greedy_compared": self.greedy_compared,
                "greedy_skipped": self.greedy_skipped, "sampled_compared": self.sampled_compared,
                "sampled_skipped": self.sampled_skipped,
                "sampled_expected_skips": round(self.sampled_expected_skips, 3),
                "greedy_expected_skips": round(self.greedy_expected_skips, 3),
                "worst": {k: float(f"{v:.3g}") for k, v in self.worst.items()}}


def tie_probability(probs, tau: float) -> float:
    """P(top-1 minus top-2 score <= tau) for Gumbel-max scores a_t + g_t with
    softmax(a) = probs: token k wins by more than tau with probability
    p_k e^-tau / (1 - p_k (1 - e^-tau)) (shift a_k down by tau and take the
    Gumbel-max probability of k), summed over k."""
    p = np.asarray(probs, dtype=np.float64)
    e = math.exp(-tau)
    return float(max(0.0, 1.0 - np.sum(p * e / (1.0 - p * (1.0 - e)))))


def greedy_tie_probability(z, tau: float, k: int = 8) -> float:
    """P(top-1 minus top-2 logit <= tau) for a row of many logits drawn from a
    smooth distribution: near the top the spacings D_j between the j-th and
    (j+1)-th largest values satisfy j D_j ~ Exp(b) (Renyi's representation
    for distributions in the Gumbel domain), so the top gap is Exp(b) with b
    estimated from the row's spacings 2..k+1 (the first is the one tested)."""
    z = np.asarray(z, dtype=np.float64)
    top = np.sort(np.partition(z, -(k + 2))[-(k + 2):])[::-1]
    d = top[:-1] - top[1:]
    b = float(np.mean((np.arange(1, d.size + 1) * d)[1:k + 1]))
    return 1.0 - math.exp(-tau / b) if b > 0 else 1.0


def log_summary(rep: Report, name: str) -> None:
    """Appends the case's id coverage to $DFLASH_PARITY_LOG (JSON lines)."""
    import json
    import os
    path = os.environ.get("DFLASH_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rep.summary(name)) + "\n")


class Pair:
    """One GPU session and its two oracle twins (exact and bf16-emulating)."""

    def __init__(self, drafter, cfg, weights_np, capacity, seed=0, sid=0, restored=0, twins=None):
        self.cfg = cfg
        self.g = drafter.session(capacity, seed=seed, stream_id=sid, restored_offset=restored)
        if twins is None:
            twins = (False, True) if cfg.dtype == "bf16" else (False,)
        self.o = [OracleSession(DraftModel(cfg, weights_np, emulate_bf16=e), restored) for e in twins]
        self.seed, self.sid = seed, sid

    def check_state(self, where=""):
        gs = self.g.state()
        for o in self.o:
            assert tuple(gs) == tuple(o.state()), f"{where}: gpu {gs} oracle {o.state()}"
        assert self.g.rows_written == self.o[0].rows_written, where

    def committed(self, tokens, feats, position):
        err = None
        for o in self.o:
            try:
                o.committed(tokens, feats, position)
            except OracleGap as e:
                err = e
        try:
            self.g.committed(tokens, feats_dev(self.cfg, feats), position)
            assert err is None, "oracle refused a run the library accepted"
        except Exception as e:  # noqa: BLE001
            if err is None:
                raise
            assert "gap" in str(e), e

    def flush(self):
        for o in self.o:
            o.flush()
        self.g.flush()

    def commit_block(self):
        for o in self.o:
            o.commit_block()
        self.g.commit_block()

    def propose(self, current, max_tokens, rep: Report, hidden=True):
        outs = [o.propose(current, max_tokens) for o in self.o]
        n, logits, hid = self.g.propose(current, max_tokens, hidden=hidden)
        if outs[0] is None:
            assert n == 0
            return None
        assert n == outs[0]["n"]
        z = logits.double().cpu().numpy()
        for k, out in enumerate(outs):
            e = rel_err(z, out["logits"])
            rep.note(f"logits[{k}]", e)
            assert e < tol(self.cfg), f"logits rel err {e} (oracle mode {k})"
            if hid is not None:
                e = rel_err(hid.double().cpu().numpy(), out["hidden"])
                rep.note(f"hidden[{k}]", e)
                assert e < tol(self.cfg), f"hidden rel err {e}"
        return n, logits, outs[-1]

    def check_cache(self, rep: Report, positions=None):
        ctx_offset, _, cache_len, _ = self.g.state()
        lo = 0
        if self.cfg.window:
            lo = max(0, ctx_offset - (self.cfg.window - 1))
        if positions is None:
            positions = np.arange(lo, cache_len)
        positions = np.asarray(positions)
        if positions.size == 0:
            return
        for l in range(self.cfg.layers):
            p0, p1 = int(positions.min()), int(positions.max()) + 1
            k, v = self.g.cache_read(l, p0, p1 - p0)
            k = k.double().cpu().numpy()[positions - p0]
            v = v.double().cpu().numpy()[positions - p0]
            for j, o in enumerate(self.o):
                K, V = o.cache_kv(l, positions)
                ek, ev = rel_err(k, K), rel_err(v, V)
                rep.note(f"cache[{j}]", max(ek, ev))
                assert ek < tol(self.cfg) and ev < tol(self.cfg), (l, ek, ev)


def id_margin(cfg, z_gpu, z_ref, temperature: float, rho: float = 1.0) -> float:
    """Gap above which the GPU must return the oracle's id: the tie margin (one
    bf16 ulp of the top logit, over T when sampling), or twice the row's
    measured logit deviation in score units when larger.  Both sides score
    token t as z'_t (greedy) or z'_t/T + g_t with the same g_t (sampling);
    z' moves by at most rho times the logit deviation (the penalty), and two
    score vectors within d of each other per token agree on the argmax
    whenever the oracle's top-1/top-2 gap exceeds 2d — greedy rows as much
    as sampled ones (the bf16 path's logits deviate by up to ~0.1, several
    ulps of the top logit)."""
    zr = np.asarray(z_ref, dtype=np.float64)
    m = margin(cfg, float(np.max(np.abs(zr))), temperature)
    d = float(np.max(np.abs(np.asarray(z_gpu, dtype=np.float64) - zr))) * max(1.0, rho)
    if temperature <= 0:
        return max(m, 2.0 * d)
    return max(m, 2.0 * d / temperature + 1e-4)


def check_ids(gpu_ids, ref_rows, rep: Report, probs=None):
    """ref_rows: (oracle id, oracle scores, margin) per row; probs: the
    oracle's sampling distribution of each row (None for greedy rows).  Rows
    whose top-2 gap exceeds the margin must agree; the others are ties both
    answers are right for, and the GPU's id must then score within twice the
    margin of the oracle's best."""
    for r, (gid, (oid, scores, tau)) in enumerate(zip(gpu_ids, ref_rows)):
        sampled = probs is not None and probs[r] is not None
        if sampled:
            rep.sampled_expected_skips += tie_probability(probs[r], tau)
        else:
            rep.greedy_expected_skips += greedy_tie_probability(scores, tau)
        if top2_gap(scores) > tau:
            rep.ids_compared += 1
            if sampled:
                rep.sampled_compared += 1
            else:
                rep.greedy_compared += 1
            if int(gid) != int(oid):
                sc = np.asarray(scores, dtype=np.float64)
                rank = int(np.sum(sc > sc[int(gid)]))
                raise AssertionError(f"id {gid} != oracle {oid} (gap {top2_gap(scores)}, margin {tau}; the "
                                     f"GPU's id is the oracle's rank {rank}, {sc[int(oid)] - sc[int(gid)]} below)")
        else:
            sc = np.asarray(scores, dtype=np.float64)
            assert sc[int(gid)] >= sc.max() - 2.0 * tau, \
                f"tie row: GPU id {gid} scores {sc.max() - sc[int(gid)]} below the best (margin {tau})"
            rep.ids_skipped += 1
            if sampled:
                rep.sampled_skipped += 1
            else:
                rep.greedy_skipped += 1


def run_session_script(drafter, cfg, wl: synth.Workload, weights_np, capacity, rounds=None, seed=0, sid=0,
                       sample=True, check_cache_every=0, twins=None, cache_sample=None) -> Report:
    """The synthetic round driver (prompt in commit_rows pieces, then rounds
    of propose -> sample -> accept -> rewind -> commit) on GPU and oracle.
    twins: the oracle modes to run (default: exact and, for bf16, emulating);
    cache_sample: when set, the prompt's and the final cache are checked at
    that many seeded slots instead of every slot (long contexts)."""
    from block_diffusion_drafter_fwd_amd import sample as gpu_sample
    rep = Report()
    fs = synth.FeatureSource(cfg, seed, sid)
    rs = synth.RoundScript(cfg, wl, seed, sid)
    pr = Pair(drafter, cfg, weights_np, capacity, seed, sid, twins=twins)
    ctx_len = wl.context

    def cache_positions():
        if not cache_sample:
            return None
        ctx, _, cache_len, _ = pr.g.state()
        lo = max(0, ctx - (cfg.window - 1)) if cfg.window else 0
        pick = np.random.default_rng([seed, sid, cache_len]).integers(lo, cache_len, size=cache_sample)
        return np.unique(np.concatenate([pick, [lo, cache_len - 1]]))

    for p in range(0, ctx_len, wl.commit_rows):
        T = min(wl.commit_rows, ctx_len - p)
        pr.committed(fs.tokens(p, T), fs.features(p, T), p)
        if not cache_sample or p + T >= ctx_len:
            pr.check_state(f"prompt commit at {p}")
    pr.check_cache(rep, cache_positions())
    current = rs.first_anchor()
    for r in range(wl.rounds if rounds is None else rounds):
        if rs.flush_before:
            pr.flush()
        res = pr.propose(current, rs.max_tokens, rep)
        pr.check_state(f"round {r} propose")
        if res is not None and sample:
            n, logits, out = res
            ids, probs = gpu_sample([pr.g], [0, n], logits, wl.temperature, wl.rep_penalty, wl.history, r,
                                    probs=wl.probs)
            ids = ids.cpu().numpy()
            o = pr.o[-1]
            ref, ref_probs = [], []
            for i in range(n):
                oid, oprob, score = sample_row(out["logits"][i], o.history[-wl.history:] if wl.history else [],
                                               wl.temperature, wl.rep_penalty, pr.seed, pr.sid, r, i)
                ref.append((oid, score, id_margin(cfg, logits[i].double().cpu().numpy(), out["logits"][i],
                                                  wl.temperature, wl.rep_penalty)))
                ref_probs.append(oprob)
                if probs is not None:
                    e = rel_err(probs[i].double().cpu().numpy(), oprob)
                    pt = probs_tol(logits[i].double().cpu().numpy(), out["logits"][i], wl.temperature)
                    rep.note("probs", e)
                    rep.note("probs/bound", e / pt)
                    assert e < pt, f"probs rel err {e} above the bound {pt} implied by the logits"
            check_ids(ids, ref, rep, ref_probs)
        n = res[0] if res is not None else 0
        a = rs.accept(n)
        pr.commit_block()
        F = pr.o[0].ctx_offset + pr.o[0].pending_count
        toks = np.concatenate([[current], fs.tokens(F + 1, a)]).astype(np.int32)
        pr.committed(toks, fs.features(F, a + 1), F)
        pr.check_state(f"round {r} commit")
        current = rs.bonus()
        rep.rounds += 1
        if check_cache_every and (r + 1) % check_cache_every == 0:
            pr.check_cache(rep, cache_positions())
    pr.flush()
    pr.check_state("final flush")
    pr.check_cache(rep, cache_positions())
    return rep
