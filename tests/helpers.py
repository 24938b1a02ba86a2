"""Shared test utilities: golden-script driver and comparison metrics.

Nothing here computes any part of the drafter; it only drives a session-like
object and measures differences.
"""
from __future__ import annotations

import json
import os
from typing import Callable

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def run_script(script: dict, make_session: Callable, features: Callable, gap_error):
    """Drive ``make_session()`` through a golden script, asserting every state.

    The session object must offer committed(tokens, feats, position),
    flush(), commit_block(), propose(current, max_tokens) -> n, state() ->
    (ctx_offset, pending, cache_len, outstanding) and rows_written.
    ``features(position, count)`` returns the feature rows of a run.
    """
    s = make_session(script["restored_offset"])
    for k, step in enumerate(script["steps"]):
        op = step["op"]
        where = f"step {k} ({op}: {step.get('why', '')})"
        if op == "committed":
            toks = np.asarray(step["tokens"], dtype=np.int32)
            feats = features(step["position"], len(toks))
            if step.get("error") == "gap":
                try:
                    s.committed(toks, feats, step["position"])
                except gap_error:
                    pass
                else:
                    raise AssertionError(f"{where}: expected a context-gap error")
            else:
                s.committed(toks, feats, step["position"])
        elif op == "flush":
            s.flush()
        elif op == "commit_block":
            s.commit_block()
        elif op == "propose":
            n = s.propose(step["current"], step["max_tokens"])
            assert n == step["n"], f"{where}: n {n} != {step['n']}"
        else:
            raise ValueError(op)
        assert tuple(s.state()) == tuple(step["state"]), f"{where}: state {s.state()} != {step['state']}"
        if "rows_written" in step:
            assert s.rows_written == step["rows_written"], \
                f"{where}: rows_written {s.rows_written} != {step['rows_written']}"
    return s


def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| over a whole tensor."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    den = np.max(np.abs(ref)) if ref.size else 1.0
    if den == 0:
        den = 1.0
    return float(np.max(np.abs(got - ref)) / den) if ref.size else 0.0
