"""The oracle's state machine against hand-derived golden scripts (CPU only).

The expected states in tests/golden/*.json follow from the integer rules of
Ollama mlxrunner/dflash.go (committed / flush / commitBlock / takePending /
propose) and the Laguna drop-before-fc rule; they were worked out by hand, not
produced by any implementation.
"""
import numpy as np
import pytest

import synth
from oracle.model import DraftModel
from oracle.session import ContextGap, OracleSession
from tests.helpers import load_golden, run_script


class _Adapter:
    def __init__(self, s):
        self.s = s

    def committed(self, t, f, p):
        self.s.committed(t, f, p)

    def flush(self):
        self.s.flush()

    def commit_block(self):
        self.s.commit_block()

    def propose(self, c, m):
        r = self.s.propose(c, m)
        return 0 if r is None else r["n"]

    def state(self):
        return self.s.state()

    @property
    def rows_written(self):
        return self.s.rows_written


@pytest.mark.parametrize("fixture", ["session_script.json", "window_drop_script.json"])
def test_golden_script(fixture):
    g = load_golden(fixture)
    c = g["config"]
    cfg = synth.config("tiny", block_size=c["block_size"], flush_rows=c["flush_rows"],
                       window=c["window"], causal=c["window"] == 0)
    w = synth.make_weights(cfg, seed=0)
    fs = synth.FeatureSource(cfg, 0)
    run_script(g, lambda off: _Adapter(OracleSession(DraftModel(cfg, w), off)),
               lambda pos, cnt: fs.features(pos, cnt), ContextGap)


def test_restored_offset_skips_held_prefix():
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg, seed=0)
    fs = synth.FeatureSource(cfg, 0)
    s = OracleSession(DraftModel(cfg, w), restored_offset=20)
    assert s.state() == (20, 0, 20, 0)
    s.committed(fs.tokens(0, 22), fs.features(0, 22), 0)            # rows 20, 21 are new
    assert s.state() == (20, 2, 20, 0)
    assert s.history == [int(t) for t in fs.tokens(20, 2)]
    with pytest.raises(ContextGap):
        s.committed(fs.tokens(30, 1), fs.features(30, 1), 30)
    assert s.state() == (20, 2, 20, 0)
