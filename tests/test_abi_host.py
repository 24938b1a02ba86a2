"""C ABI tests that need no GPU.

* libdflash.so loads and exports every function include/dflash.h declares
  (nothing is called: there is no device here).
* The session state machine, through the same C ABI built over the trace
  backend (libdflash_host.so), follows the golden scripts hand-derived from
  Ollama mlxrunner/dflash.go, rejects gaps and bad configs with the documented
  codes and unchanged state, and plans the expected context passes (chunking
  by flush_rows, Laguna drop-before-fc).
"""
import ctypes
import os
import re
from ctypes import byref, c_int32, c_int64, c_void_p

import numpy as np
import pytest

from block_diffusion_drafter_fwd_amd import abi
from tests.helpers import load_golden, run_script

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "dflash.h")).read()
    return sorted(set(re.findall(r"\b(dflash_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported_by_hip_library():
    if not os.path.exists(abi.LIB_HIP):
        pytest.skip("libdflash.so not built")
    lib = ctypes.CDLL(abi.LIB_HIP)
    names = _header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(abi.SYMBOLS), "binding and header disagree"


# --------------------------------------------------------------------------
# host (trace) build
# --------------------------------------------------------------------------

@pytest.fixture(scope="module")
def host():
    from block_diffusion_drafter_fwd_amd import build
    build.build_host()
    lib = abi.load("host")
    lib.dflash_trace_count.restype = ctypes.c_int
    lib.dflash_trace_line.argtypes = [ctypes.c_int, ctypes.c_char_p, ctypes.c_int]
    return lib


def _trace(lib):
    out = []
    buf = ctypes.create_string_buffer(4096)
    for i in range(lib.dflash_trace_count()):
        lib.dflash_trace_line(i, buf, 4096)
        out.append(buf.value.decode())
    lib.dflash_trace_clear()
    return out


class FakeModel:
    """dflash_config + dflash_weights whose pointers are host buffers: the
    trace backend checks shapes and never dereferences data."""

    def __init__(self, lib, **kw):
        base = dict(dtype=abi.FP32, hidden=64, layers=2, q_heads=4, kv_heads=4, head_dim=16, taps=5,
                    target_hidden=64, vocab=32, block_size=8, mask_id=31, window=0, intermediate=192,
                    causal=1, qk_norm=1, gate=0, aux_norms=0, ctx_input_norm=0, fused_qkv=0,
                    attention_bias=0, flush_rows=16)
        base.update(kw)
        self.c = abi.Config()
        for k, v in base.items():
            setattr(self.c, k, v)
        self.c.rope_theta = 10000.0
        self.c.rms_eps = 1e-6
        self.buf = np.zeros(64, dtype=np.uint8)
        self.lib = lib
        self.W = self.weights()

    def t(self, *shape):
        x = abi.Tensor()
        x.data = self.buf.ctypes.data
        x.ndim = len(shape)
        for i, s in enumerate(shape):
            x.shape[i] = s
        return x

    def weights(self, **override):
        c = self.c
        H, V, I, D = c.hidden, c.vocab, c.intermediate, c.head_dim
        qd, kd = c.q_heads * D, c.kv_heads * D
        W = abi.Weights()
        W.embed, W.lm_head, W.fc = self.t(V, H), self.t(V, H), self.t(H, c.taps * c.target_hidden)
        W.hidden_norm, W.norm = self.t(H), self.t(H)
        W.aux_norms = self.t(c.taps, c.target_hidden)
        self.layers = (abi.LayerWeights * c.layers)()
        for l in range(c.layers):
            L = self.layers[l]
            L.input_layernorm = L.post_attention_layernorm = self.t(H)
            L.q_proj, L.k_proj, L.v_proj = self.t(qd, H), self.t(kd, H), self.t(kd, H)
            L.qkv_proj = self.t(qd + 2 * kd, H)
            L.q_norm = L.k_norm = self.t(D)
            L.g_proj = self.t(c.q_heads, H)
            L.o_proj = self.t(H, qd)
            L.gate_proj = L.up_proj = self.t(I, H)
            L.down_proj = self.t(H, I)
            for k, v in override.items():
                setattr(L, k, v)
        W.layers = ctypes.cast(self.layers, ctypes.POINTER(abi.LayerWeights))
        return W

    def create(self):
        ctx = c_void_p()
        rc = self.lib.dflash_create(byref(self.c), byref(self.W), byref(ctx))
        return rc, ctx


class HostSession:
    def __init__(self, lib, ctx, capacity=4096, restored=0, max_sessions=1):
        self.lib = lib
        n = lib.dflash_session_bytes(ctx, capacity)
        self.arena = np.zeros(n, dtype=np.uint8)
        ws = lib.dflash_workspace_bytes(ctx, max_sessions)
        self.ws = np.zeros(ws, dtype=np.uint8)
        self.h = c_void_p()
        abi.check(lib, lib.dflash_session_open(ctx, self.arena.ctypes.data, n, capacity, self.ws.ctypes.data,
                                               ws, max_sessions, restored, 1, 2, None, byref(self.h)))
        self.feat = np.zeros(1 << 16, dtype=np.uint8)

    def committed(self, tokens, feats, position):
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        abi.check(self.lib, self.lib.dflash_committed(self.h, t.ctypes.data_as(ctypes.POINTER(c_int32)),
                                                      self.feat.ctypes.data, len(t), position))

    def flush(self):
        abi.check(self.lib, self.lib.dflash_flush(self.h))

    def commit_block(self):
        abi.check(self.lib, self.lib.dflash_commit_block(self.h))

    def propose(self, current, max_tokens):
        n = c_int32()
        logits = np.zeros(16, dtype=np.float32)
        abi.check(self.lib, self.lib.dflash_propose(self.h, current, max_tokens, logits.ctypes.data, None,
                                                    byref(n)))
        return n.value

    def state(self):
        a, b, c, d, e = c_int32(), c_int32(), c_int32(), c_int32(), c_int64()
        abi.check(self.lib, self.lib.dflash_session_state(self.h, byref(a), byref(b), byref(c), byref(d),
                                                          byref(e)))
        self._rw = e.value
        return a.value, b.value, c.value, d.value

    @property
    def rows_written(self):
        self.state()
        return self._rw


@pytest.mark.parametrize("fixture", ["session_script.json", "window_drop_script.json"])
def test_golden_scripts_through_c_abi(host, fixture):
    g = load_golden(fixture)
    c = g["config"]
    fm = FakeModel(host, block_size=c["block_size"], flush_rows=c["flush_rows"], window=c["window"],
                   causal=int(c["window"] == 0))
    rc, ctx = fm.create()
    assert rc == 0, host.dflash_last_error()
    _trace(host)
    run_script(g, lambda off: HostSession(host, ctx, capacity=64, restored=off),
               lambda pos, cnt: None, abi.ContextGap)
    host.dflash_destroy(ctx)


def test_chunked_flush_plan(host):
    fm = FakeModel(host, flush_rows=16)
    rc, ctx = fm.create()
    assert rc == 0
    s = HostSession(host, ctx)
    _trace(host)
    s.committed(np.arange(5), None, 0)
    s.committed(np.arange(5, 45), None, 5)          # 45 rows >= 16: flush everything
    tr = [l for l in _trace(host) if l.startswith("ctx")]
    assert tr == ["ctx sess=0 pos0=0 rows=16", "ctx sess=0 pos0=16 rows=16", "ctx sess=0 pos0=32 rows=13"]
    assert s.state() == (45, 0, 45, 0) and s.rows_written == 45


def test_flushed_chunks_of_fresh_rows_are_read_in_place(host):
    """A flushed chunk made only of the committed run's rows is projected
    from the caller's buffer (no copy); rows joining buffered ones, rows that
    stay pending and unaligned rows are copied into the pending buffer."""
    fm = FakeModel(host, flush_rows=16)
    rc, ctx = fm.create()
    assert rc == 0
    s = HostSession(host, ctx)

    def commit(T, pos, offset=0):
        t = np.arange(pos, pos + T, dtype=np.int32)
        abi.check(host, host.dflash_committed(s.h, t.ctypes.data_as(ctypes.POINTER(c_int32)),
                                              s.feat.ctypes.data + offset, T, pos))
        return [l for l in _trace(host) if l.startswith(("copy", "ctx"))]

    assert s.feat.ctypes.data % 16 == 0
    _trace(host)
    assert commit(40, 0) == ["ctx sess=0 pos0=0 rows=16", "ctx sess=0 pos0=16 rows=16", "ctx sess=0 pos0=32 rows=8"]
    assert commit(5, 40) == ["copy rows=5"]
    assert commit(20, 45) == ["copy rows=11", "ctx sess=0 pos0=40 rows=16", "ctx sess=0 pos0=56 rows=9"]
    assert commit(16, 65, offset=2) == ["copy rows=16", "ctx sess=0 pos0=65 rows=16"]
    assert s.state() == (81, 0, 81, 0) and s.rows_written == 81


def test_window_drop_plan_skips_old_chunks(host):
    fm = FakeModel(host, flush_rows=16, window=6, causal=0)
    rc, ctx = fm.create()
    assert rc == 0
    s = HostSession(host, ctx, capacity=64)
    _trace(host)
    s.committed(np.arange(100), None, 0)            # frontier 100: keep slots >= 95
    tr = [l for l in _trace(host) if l.startswith("ctx")]
    assert tr == ["ctx sess=0 pos0=95 rows=1", "ctx sess=0 pos0=96 rows=4"]
    assert s.state() == (100, 0, 100, 0) and s.rows_written == 5


def test_history_ring_and_sample_plan(host):
    fm = FakeModel(host)
    rc, ctx = fm.create()
    s = HostSession(host, ctx)
    _trace(host)
    s.committed(np.arange(600), None, 0)
    # a flushing commit keeps its history tokens on the host until the ring
    # is next read (the sample) or written (a one-step commit)
    assert [l for l in _trace(host) if l.startswith("hist")] == []
    n = s.propose(3, 7)
    logits = np.zeros(16, dtype=np.float32)
    ids = np.zeros(16, dtype=np.int32)
    offs = (c_int32 * 2)(0, n)
    hs = (c_void_p * 1)(s.h)
    p = abi.SampleParams(0.7, 1.1, 512, 4)
    abi.check(host, host.dflash_sample(hs, 1, offs, logits.ctypes.data, byref(p), ids.ctypes.data, None))
    tr = [l for l in _trace(host) if l.startswith(("hist", "sample"))]
    toks = [int(x) for l in tr[:-1] for x in l.split("tokens=")[1].split(",")]
    assert toks == list(range(88, 600))             # only the last 512 are kept, written before the sample
    assert tr[0].startswith("hist slot=0 ")
    assert tr[-1] == "sample rows=7 round=4 hist=600@0"      # ring of 512 written from slot 0
    abi.check(host, host.dflash_sample(hs, 1, offs, logits.ctypes.data, byref(p), ids.ctypes.data, None))
    assert [l for l in _trace(host) if l.startswith("hist")] == []   # written once


def test_deferred_history_is_written_before_a_one_step_commit(host):
    """A one-step commit writes its tokens to the device ring directly, so the
    history a flushing commit left on the host goes out first (a later write
    of the older tokens would overwrite the newer ones)."""
    fm = FakeModel(host, flush_rows=16)
    rc, ctx = fm.create()
    s = HostSession(host, ctx)
    _trace(host)
    s.committed(np.arange(20), None, 0)              # flushes: 20 tokens kept on the host
    s.committed(np.arange(20, 23), None, 20)         # one step: the 20 first, then these 3
    tr = [l for l in _trace(host) if l.startswith(("hist", "copy"))]
    assert tr == ["hist slot=0 tokens=" + ",".join(str(i) for i in range(20)), "hist slot=20 tokens=20,21,22",
                  "copy rows=3"]


@pytest.mark.parametrize("field,value", [("block_size", 1), ("block_size", 513), ("window", 1),
                                         ("window", (1 << 20) + 1), ("attention_bias", 1), ("kv_heads", 3),
                                         ("dtype", 5), ("layers", 17)])
def test_config_bounds(host, field, value):
    fm = FakeModel(host, **{field: value})
    rc, ctx = fm.create()
    assert rc == abi.E_CONFIG, (field, value, rc)


def test_bf16_shape_rules(host):
    fm = FakeModel(host, dtype=abi.BF16)                 # head_dim 16 not allowed on the bf16 path
    assert fm.create()[0] == abi.E_CONFIG


def test_weight_shape_checks(host):
    fm = FakeModel(host)
    fm.W = fm.weights(q_proj=fm.t(60, 64))               # wrong q_proj rows
    rc, _ = fm.create()
    assert rc == abi.E_SHAPE and b"q_proj" in host.dflash_last_error()
    fm = FakeModel(host, fused_qkv=1)
    fm.W = fm.weights(qkv_proj=fm.t(64 + 64 + 63, 64))
    assert fm.create()[0] == abi.E_SHAPE
    fm = FakeModel(host, gate=1)
    fm.W = fm.weights(g_proj=fm.t(4, 63))                # input width
    assert fm.create()[0] == abi.E_SHAPE
    fm = FakeModel(host)
    fm.W = fm.weights(k_norm=fm.t(15))                   # per-head norm length
    assert fm.create()[0] == abi.E_SHAPE


def test_gap_and_capacity_errors_leave_state(host):
    fm = FakeModel(host)
    rc, ctx = fm.create()
    s = HostSession(host, ctx, capacity=32)
    s.committed(np.arange(10), None, 0)
    with pytest.raises(abi.ContextGap):
        s.committed(np.arange(3), None, 11)
    assert s.state() == (0, 10, 0, 0)
    with pytest.raises(abi.DFlashError) as e:
        s.committed(np.arange(20), None, 10)             # 30 + block 8 > 32
    assert e.value.code == abi.E_CAPACITY
    assert s.state() == (0, 10, 0, 0)


def test_windowed_capacity_rule(host):
    fm = FakeModel(host, window=6, causal=0)
    rc, ctx = fm.create()
    n = host.dflash_session_bytes(ctx, 12)
    arena = np.zeros(n, dtype=np.uint8)
    ws = np.zeros(host.dflash_workspace_bytes(ctx, 1), dtype=np.uint8)
    h = c_void_p()
    rc = host.dflash_session_open(ctx, arena.ctypes.data, n, 12, ws.ctypes.data, ws.size, 1, 0, 0, 0, None,
                                  byref(h))
    assert rc == abi.E_CAPACITY                          # needs >= 6 + 8 - 1 = 13
    HostSession(host, ctx, capacity=13)


def test_batch_rules(host):
    fm = FakeModel(host)
    rc, ctx = fm.create()
    a = HostSession(host, ctx, max_sessions=4)
    b = HostSession(host, ctx, max_sessions=4)
    b.ws, b.h2 = a.ws, None
    # sessions with different workspaces cannot be batched
    logits = np.zeros(64, dtype=np.float32)
    offs = (c_int32 * 3)()
    hs = (c_void_p * 2)(a.h, b.h)
    cur = (c_int32 * 2)(1, 2)
    mt = (c_int32 * 2)(3, 3)
    a.committed(np.arange(4), None, 0)
    rc = host.dflash_propose_batch(hs, 2, cur, mt, logits.ctypes.data, offs)
    assert rc == abi.E_ARG
    # a batch over one workspace; a session with no context contributes no rows
    ws = np.zeros(host.dflash_workspace_bytes(ctx, 4), dtype=np.uint8)
    sess = []
    for k in range(3):
        n = host.dflash_session_bytes(ctx, 64)
        arena = np.zeros(n, dtype=np.uint8)
        h = c_void_p()
        abi.check(host, host.dflash_session_open(ctx, arena.ctypes.data, n, 64, ws.ctypes.data, ws.size, 4,
                                                 0, 0, k, None, byref(h)))
        sess.append((h, arena))
    feat = np.zeros(1 << 14, dtype=np.uint8)
    for k, (h, _) in enumerate(sess[:2]):
        t = np.arange(3 + k, dtype=np.int32)
        abi.check(host, host.dflash_committed(h, t.ctypes.data_as(ctypes.POINTER(c_int32)), feat.ctypes.data,
                                              len(t), 0))
    _trace(host)
    hs = (c_void_p * 3)(*[h for h, _ in sess])
    cur = (c_int32 * 3)(5, 6, 7)
    mt = (c_int32 * 3)(2, 9, 4)
    offs = (c_int32 * 4)()
    abi.check(host, host.dflash_propose_batch(hs, 3, cur, mt, logits.ctypes.data, offs))
    assert list(offs) == [0, 2, 9, 9]
    tr = _trace(host)
    assert tr == ["ctx sess=0 pos0=0 rows=3", "ctx sess=1 pos0=0 rows=4",
                  "block sess=0 F=3 M=3 cur=5", "block sess=1 F=4 M=8 cur=6"]


def _shared_sessions(host, ctx, count, max_sessions=4, capacity=64):
    """`count` sessions over one workspace (what a batched call requires)."""
    ws = np.zeros(host.dflash_workspace_bytes(ctx, max_sessions), dtype=np.uint8)
    out = []
    for k in range(count):
        s = HostSession.__new__(HostSession)
        s.lib = host
        n = host.dflash_session_bytes(ctx, capacity)
        s.arena = np.zeros(n, dtype=np.uint8)
        s.ws = ws
        s.h = c_void_p()
        abi.check(host, host.dflash_session_open(ctx, s.arena.ctypes.data, n, capacity, ws.ctypes.data, ws.size,
                                                 max_sessions, 0, 0, k, None, byref(s.h)))
        s.feat = np.zeros(1 << 16, dtype=np.uint8)
        out.append(s)
    return out


def _prepare_for_flush(sessions):
    """Session 0: 3 pending rows; 1: nothing; 2: an outstanding block, then 5
    pending rows committed after the rewind; 3: 12 pending rows."""
    a, b, c, d = sessions
    a.committed(np.arange(3), None, 0)
    c.committed(np.arange(4), None, 0)
    assert c.propose(5, 3) == 3
    c.commit_block()
    c.committed(np.arange(5), None, 4)
    d.committed(np.arange(12), None, 0)


@pytest.mark.parametrize("window", [0, 6])
def test_flush_batch_equals_single_flushes(host, window):
    """dflash_flush_batch gives every session the state, and plans the same
    context rows (window drop included), as dflash_flush per session."""
    fm = FakeModel(host, window=window)
    rc, ctx = fm.create()
    assert rc == 0
    one = _shared_sessions(host, ctx, 4)
    many = _shared_sessions(host, ctx, 4)
    _prepare_for_flush(one)
    _prepare_for_flush(many)
    _trace(host)
    for s in one:
        s.flush()
    t_one = _trace(host)
    hs = (c_void_p * 4)(*[s.h for s in many])
    abi.check(host, host.dflash_flush_batch(hs, 4))
    t_many = _trace(host)
    assert [s.state() for s in many] == [s.state() for s in one]
    assert [s.rows_written for s in many] == [s.rows_written for s in one]
    # a single-session flush names its session 0; sessions 0, 2 and 3 have rows
    single = [ln.split(" ", 2)[2] for ln in t_one if ln.startswith("ctx ")]
    batched = [ln.split(" ", 2) for ln in t_many if ln.startswith("ctx ")]
    assert [(b[1], b[2]) for b in batched] == list(zip(["sess=0", "sess=2", "sess=3"], single))
    st = [s.state() for s in many]
    assert st[0] == (3, 0, 3, 0) and st[1] == (0, 0, 0, 0) and st[2] == (9, 0, 9, 0) and st[3] == (12, 0, 12, 0)
    if window:
        # frontier 12, window 6: only slots 7..11 of session 3 are projected
        assert "ctx sess=3 pos0=7 rows=5" in t_many


def test_flush_batch_rejects_bad_batches(host):
    fm = FakeModel(host)
    rc, ctx = fm.create()
    a, b = _shared_sessions(host, ctx, 2)
    a.committed(np.arange(3), None, 0)
    before = a.state()
    hs = (c_void_p * 2)(a.h, a.h)
    assert host.dflash_flush_batch(hs, 2) == abi.E_ARG            # a session twice
    other = HostSession(host, ctx)
    hs = (c_void_p * 2)(a.h, other.h)
    assert host.dflash_flush_batch(hs, 2) == abi.E_ARG            # another workspace
    assert host.dflash_flush_batch(hs, 0) == abi.E_ARG
    assert a.state() == before                                    # state unchanged on every error


def _commit_batch(host, sessions, runs, positions):
    n = len(sessions)
    toks = [np.asarray(r, dtype=np.int32) for r in runs]
    offs = np.zeros(n + 1, dtype=np.int32)
    offs[1:] = np.cumsum([len(t) for t in toks])
    flat = np.ascontiguousarray(np.concatenate(toks) if offs[-1] else np.zeros(1, dtype=np.int32))
    hs = (c_void_p * n)(*[s.h for s in sessions])
    feats = (c_void_p * n)(*[s.feat.ctypes.data for s in sessions])
    pos = (c_int32 * n)(*positions)
    return host.dflash_committed_batch(hs, n, flat.ctypes.data_as(ctypes.POINTER(c_int32)),
                                       offs.ctypes.data_as(ctypes.POINTER(c_int32)), feats, pos)


def test_committed_batch_equals_single_commits(host):
    """dflash_committed_batch leaves every session as dflash_committed on each
    would, with the same history writes, row copies and context passes:
    a plain run, a run that repeats committed positions (skipped), a run that
    reaches the flush threshold (flushes), and a history ring that wraps."""
    fm = FakeModel(host)
    rc, ctx = fm.create()
    assert rc == 0
    one = _shared_sessions(host, ctx, 4, capacity=2048)
    many = _shared_sessions(host, ctx, 4, capacity=2048)
    for group in (one, many):
        group[1].committed(np.arange(6), None, 0)
        for p in range(0, 505, 5):              # session 3: 505 history tokens, 1 pending row short of a flush
            group[3].committed(np.arange(5) + p, None, p)
    _trace(host)
    runs = [np.arange(4) + 100, np.arange(8) + 200, np.arange(20) + 300, np.arange(9) + 400]
    positions = [0, 3, 0, 505]                  # session 1 repeats positions 3..5
    for s, r, p in zip(one, runs, positions):
        s.committed(r, None, p)
    t_one = _trace(host)
    abi.check(host, _commit_batch(host, many, runs, positions))
    t_many = _trace(host)
    assert [s.state() for s in many] == [s.state() for s in one]
    assert [s.rows_written for s in many] == [s.rows_written for s in one]
    # the same history writes, row copies and context rows (a single-session
    # call names its session 0, so session indices are dropped)
    def planned(trace):
        return sorted(re.sub(r" sess=\d+", "", ln) for ln in trace)
    assert planned(t_many) == planned(t_one)
    st = [s.state() for s in many]
    assert st[0] == (0, 4, 0, 0) and st[1][:2] == (0, 11)    # 6 pending + the 5 rows past them
    assert st[2][:2] == (20, 0)                 # reached flush_rows = 16: flushed


def test_committed_batch_rejects_any_bad_run(host):
    fm = FakeModel(host)
    rc, ctx = fm.create()
    ss = _shared_sessions(host, ctx, 3, capacity=64)
    ss[0].committed(np.arange(3), None, 0)
    before = [s.state() for s in ss]
    _trace(host)
    # session 2's run starts past its frontier: the whole batch is refused
    rc = _commit_batch(host, ss, [np.arange(2), np.arange(2), np.arange(2)], [3, 0, 5])
    assert rc == abi.E_CONTEXT_GAP
    assert [s.state() for s in ss] == before and _trace(host) == []
    rc = _commit_batch(host, [ss[0], ss[0]], [np.arange(2), np.arange(2)], [3, 5])
    assert rc == abi.E_ARG                      # a session twice
    rc = _commit_batch(host, ss[:1], [np.arange(70)], [3])
    assert rc == abi.E_CAPACITY                 # 73 + block > capacity 64
    assert [s.state() for s in ss] == before


# --------------------------------------------------------------------------
# device failures (DFLASH_E_HIP injected by the trace backend)
# --------------------------------------------------------------------------

def _ring_from_trace(lines, ring):
    """Replays the history writes of a trace onto a host model of the ring."""
    for l in lines:
        m = re.match(r"hist slot=(\d+) tokens=(.*)", l)
        if m:
            slot = int(m.group(1))
            toks = [int(x) for x in m.group(2).split(",") if x]
            ring[slot:slot + len(toks)] = toks
    return ring


def _sample(lib, s, history=512):
    ids = np.zeros(8, dtype=np.int32)
    logits = np.zeros(8, dtype=np.float32)
    offs = (c_int32 * 2)(0, 1)
    hs = (c_void_p * 1)(s.h)
    p = abi.SampleParams(0.0, 1.1, history, 0)
    abi.check(lib, lib.dflash_sample(hs, 1, offs, logits.ctypes.data, byref(p), ids.ctypes.data, None))


def _drive(s, step):
    """One call of the script: ('c', tokens, position), ('f',) or ('p', cur, n)."""
    if step[0] == "c":
        t = np.ascontiguousarray(np.asarray(step[1], dtype=np.int32))
        return s.lib.dflash_committed(s.h, t.ctypes.data_as(ctypes.POINTER(c_int32)), s.feat.ctypes.data,
                                      len(t), step[2])
    if step[0] == "f":
        return s.lib.dflash_flush(s.h)
    n = c_int32()
    logits = np.zeros(16, dtype=np.float32)
    return s.lib.dflash_propose(s.h, step[1], step[2], logits.ctypes.data, None, byref(n))


SCRIPT = [("c", list(range(100, 110)), 0), ("p", 3, 7), ("c", [3, 501, 502], 10),
          ("c", list(range(200, 220)), 13), ("p", 9, 5), ("c", [9], 33), ("f",),
          ("c", list(range(300, 800)), 34), ("p", 4, 7), ("c", [4, 7], 534)]


def _sampled_window(lines, ring):
    """(count, head) the sampler saw, from its trace line, and the ring slots
    it reads: the last min(count, 512) ending at head."""
    m = [re.search(r"hist=(\d+)@(\d+)", l) for l in lines if l.startswith("sample")]
    count, head = int(m[-1].group(1)), int(m[-1].group(2))
    hn = min(count, 512)
    return count, head, [int(ring[(head - hn + i) % 512]) for i in range(hn)]


def test_device_failure_leaves_host_state_unchanged(host):
    """Every device step of every call of a script (one-step commits, flushing
    commits, a 500-token run that wraps the history ring, proposes, a flush)
    is made to fail in turn.  The failing call returns DFLASH_E_HIP and the
    session's host state (offsets, pending rows, cache length, outstanding
    block, rows written) is what it was before the call; retrying the call
    then gives the states of a run that never failed, and the history window
    the sampler reads holds the same tokens (the failed call's partial ring
    writes are overwritten from the host copy)."""
    fm = FakeModel(host, flush_rows=16)
    rc, ctx = fm.create()
    assert rc == 0
    ref = HostSession(host, ctx, capacity=2048)
    _trace(host)
    ref_states, ref_windows = [], []
    ref_ring = np.full(512, -1)
    for step in SCRIPT:
        assert _drive(ref, step) == 0
        ref_states.append((ref.state(), ref.rows_written))
        _sample(host, ref)
        lines = _trace(host)
        _ring_from_trace(lines, ref_ring)
        ref_windows.append(_sampled_window(lines, ref_ring))
    injected = 0
    for k in range(len(SCRIPT)):
        for fail_at in range(1, 16):
            s = HostSession(host, ctx, capacity=2048)
            for step in SCRIPT[:k]:
                assert _drive(s, step) == 0
            _sample(host, s)
            lines = _trace(host)
            ring = _ring_from_trace(lines, np.full(512, -1))
            window = _sampled_window(lines, ring)
            before = (s.state(), s.rows_written)
            host.dflash_trace_fail_in(fail_at)
            rc = _drive(s, SCRIPT[k])
            host.dflash_trace_fail_in(0)
            _ring_from_trace(_trace(host), ring)        # what the failed call did write
            if rc == 0:                                  # the call has fewer device steps
                break
            injected += 1
            assert rc == abi.E_HIP, (k, fail_at, rc)
            assert (s.state(), s.rows_written) == before, (k, fail_at)
            _sample(host, s)                             # the sampler still sees the old history
            lines = _trace(host)
            _ring_from_trace(lines, ring)
            assert _sampled_window(lines, ring) == window, (k, fail_at)
            assert _drive(s, SCRIPT[k]) == 0
            assert (s.state(), s.rows_written) == ref_states[k], (k, fail_at)
            _sample(host, s)
            lines = _trace(host)
            _ring_from_trace(lines, ring)
            assert _sampled_window(lines, ring) == ref_windows[k], (k, fail_at)
    assert injected >= len(SCRIPT)
    host.dflash_destroy(ctx)


# --------------------------------------------------------------------------
# DFlash2 selector arguments
# --------------------------------------------------------------------------

@pytest.mark.parametrize("k,ds", [(17, 8), (-1, 8), (33, 8), (4, 0), (4, 257)])
def test_selector_config_bounds(host, k, ds):
    """K in 1..min(16, V), Ds in 1..256 (the 32-token vocabulary of the fake
    model bounds K too)."""
    fm = FakeModel(host, sel_candidates=k, sel_dim=ds)
    assert fm.create()[0] == abi.E_CONFIG, (k, ds)


def test_selector_tables_and_state(host):
    fm = FakeModel(host, sel_candidates=4, sel_dim=8)
    rc, _ = fm.create()                                   # tables missing
    assert rc == abi.E_SHAPE and b"sel_prev" in host.dflash_last_error()
    fm.W.sel_prev = fm.t(32, 8)
    fm.W.sel_next = fm.t(32, 7)
    assert fm.create()[0] == abi.E_SHAPE and b"sel_next" in host.dflash_last_error()
    fm.W.sel_next = fm.t(32, 8)
    rc, ctx = fm.create()
    assert rc == 0, host.dflash_last_error()
    s = HostSession(host, ctx)
    out = np.zeros(64, dtype=np.int32)
    offs = (c_int32 * 2)(0, 3)
    cur = (c_int32 * 1)(5)
    hs = (c_void_p * 1)(s.h)
    p = abi.SelectParams(0.5, 2)
    _trace(host)
    rc = host.dflash_select(hs, 1, offs, out.ctypes.data, cur, byref(p), out.ctypes.data, out.ctypes.data,
                            out.ctypes.data, out.ctypes.data)
    assert rc == 0 and _trace(host) == ["select rows=3 round=2 dense=1 anchors=5"]
    bad = (c_int32 * 1)(32)                                # anchor outside the vocabulary
    assert host.dflash_select(hs, 1, offs, out.ctypes.data, bad, byref(p), out.ctypes.data, out.ctypes.data,
                              None, None) == abi.E_ARG
    many = (c_int32 * 2)(0, 8)                             # more rows than blockSize - 1
    assert host.dflash_select(hs, 1, many, out.ctypes.data, cur, byref(p), out.ctypes.data, out.ctypes.data,
                              None, None) == abi.E_ARG
    host.dflash_destroy(ctx)
    plain = FakeModel(host)                                # no selector configured
    rc, ctx2 = plain.create()
    s2 = HostSession(host, ctx2)
    hs2 = (c_void_p * 1)(s2.h)
    assert host.dflash_select(hs2, 1, offs, out.ctypes.data, cur, byref(p), out.ctypes.data, out.ctypes.data,
                              None, None) == abi.E_STATE
    host.dflash_destroy(ctx2)


def test_profile_stages(host):
    """Every stage the header documents opens and closes (no launches on the
    trace backend: zero time, zero launches); an unknown stage is E_ARG."""
    fm = FakeModel(host)
    rc, ctx = fm.create()
    assert rc == 0
    ms, n = ctypes.c_double(), ctypes.c_int32()
    for stage in ("unembed", "attention", "attention_partial", "flush_fc", "flush_kv", "layer_gemms", "sampler",
                  "verify", "select"):
        assert host.dflash_profile_begin(ctx, stage.encode()) == 0, stage
        assert host.dflash_profile_end(ctx, ctypes.byref(ms), ctypes.byref(n)) == 0, stage
        assert n.value == 0
    assert host.dflash_profile_begin(ctx, b"no_such_stage") == abi.E_ARG
    host.dflash_destroy(ctx)
