"""GPU parity: the HIP library through its C ABI against the float64 oracle.

Sizes keep the model dimensions of each configuration family (so every
kernel runs its real tiling: 256-row flushes through the tiled MFMA GEMM,
16-row blocks through the skinny one, the 64-query-row attention tile) while
cutting layers, vocabulary (ragged: not a multiple of any tile) and context
(ragged flush tails), so that the oracle finishes in seconds.  Probabilities
are held to the bound their own logit deviation implies (see
tests/parity.py: probs_tol); the logits are held to 2e-2 (bf16) / 1e-4 (fp32).
"""
import sys

import numpy as np
import pytest
import torch

import synth
from tests.parity import (Pair, Report, check_ids, device_tensors, feats_dev, id_margin, log_summary, margin,
                          probs_tol, rel_err, run_session_script, tol)

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_fwd_amd import abi
    abi.load("hip")
    return True


def _drafter(cfg, w, max_sessions=1):
    from block_diffusion_drafter_fwd_amd import Drafter
    return Drafter(cfg, device_tensors(cfg, w), max_sessions=max_sessions)


W = synth.Workload
CASES = {
    # name: (config, workload, capacity)
    "tiny": (synth.config("tiny"), synth.WORKLOADS["tiny"], 48 + 8 * 20 + 16),
    "tiny_w": (synth.config("tiny_w"), synth.WORKLOADS["tiny_w"], 6 + 8 - 1),
    "tiny_sampling": (synth.config("tiny", causal=False),
                      W("ts", "tiny", context=37, commit_rows=5, rounds=12, temperature=0.7, rep_penalty=1.1,
                        history=24, probs=True, max_tokens=-1, flush_fraction=1.0), 400),
    "qwen_small": (synth.config("qwen", layers=2, vocab=5003),
                   W("qs", "qwen", context=300, commit_rows=256, rounds=5), 512),
    "laguna_small": (synth.config("laguna", layers=2, vocab=4099),
                     W("ls", "laguna", context=1100, commit_rows=300, rounds=5), 512 + 8 - 1),
    "long_small": (synth.config("long", layers=1, vocab=3001),
                   W("lo", "long", context=270, commit_rows=256, rounds=4, max_tokens=7, temperature=1.0,
                     probs=True), 400),
    # full sizes, in the launch configuration the bench times (5 layers, the
    # 151936-token unembedding on the persistent kernel; window 512 ring with
    # 4 layers and a 100352-token vocabulary), short contexts so the oracle
    # keeps up
    "qwen_full": (synth.config("qwen"), W("qf", "qwen", context=300, commit_rows=256, rounds=3), 512),
    "laguna_full": (synth.config("laguna"), W("lf", "laguna", context=1100, commit_rows=300, rounds=3),
                    512 + 8 - 1),
    # the long configuration's widths (hidden 4096, fc 20480 -> 4096, 8 fc
    # slices on the 256-row tiles) with a vocabulary large enough for the
    # persistent unembedding at K = 4096 (eight 64-wide k steps per wave);
    # 40009 is not a multiple of any tile
    "long_wide": (synth.config("long", layers=1, vocab=40009),
                  W("lw", "long", context=270, commit_rows=256, rounds=3, max_tokens=7, temperature=1.0,
                    probs=True), 400),
    # the long configuration at full size (5 layers, hidden 4096, the
    # 262144-token unembedding and sampler with probabilities), short context
    "long_full": (synth.config("long"), W("lf5", "long", context=270, commit_rows=256, rounds=2, max_tokens=7,
                                            temperature=1.0, probs=True), 400),
    "batched_shape_sampling": (synth.config("qwen", layers=1, vocab=3001),
                               W("bs", "qwen", context=130, commit_rows=40, rounds=5, max_tokens=-1,
                                 temperature=0.7, rep_penalty=1.1, history=512, probs=True), 300),
    # the bench's context lengths: the Qwen-style drafter at full size over
    # its whole 4096-slot prompt (the attention split takes one workgroup
    # per CU: 31 items of 192 keys per kv head), and the long configuration's
    # attention geometry (32 q / 8 kv heads x 128) over a 32768-slot prompt
    # (one resident round of 57 items of 576 keys per kv head, the branch the
    # 131072-slot bench takes with 2112-key items), its widths cut so the
    # oracle keeps up
    "qwen_ctx4096": (synth.config("qwen"), W("q4k", "qwen", context=4096, commit_rows=256, rounds=3),
                     4096 + 4 * 16 + 64),
    "long_ctx32k": (synth.config("long", hidden=1024, target_hidden=256, intermediate=3072, layers=1,
                                 vocab=3001),
                    W("l32k", "long", context=32768, commit_rows=256, rounds=3, max_tokens=7, temperature=1.0,
                      probs=True), 32768 + 4 * 8 + 64),
    # a 32768-key sliding window over a ring that has wrapped (34000 context
    # rows in 32775 slots): the attention split takes chunks of 256 keys or
    # more whose items interleave their tiles, each key's slot its position
    # modulo the capacity
    "laguna_ring32k": (synth.config("laguna", hidden=1024, target_hidden=256, intermediate=3072, layers=1,
                                    vocab=3001, window=32768),
                       W("lr32", "laguna", context=34000, commit_rows=256, rounds=3), 32768 + 8 - 1),
}
# cases whose prompt is long: the oracle runs its bf16-emulating twin only and
# the caches are checked at sampled slots
LONG_CASES = {"long_ctx32k": 48, "laguna_ring32k": 48}


@pytest.mark.parametrize("name", list(CASES))
def test_round_script_parity(cuda, name):
    cfg, wl, cap = CASES[name]
    say(f"[parity] {name}: weights")
    w = synth.make_weights(cfg, seed=1, gains="random")
    d = _drafter(cfg, w)
    say(f"[parity] {name}: running {wl.rounds} rounds, context {wl.context}")
    long = name in LONG_CASES
    rep = run_session_script(d, cfg, wl, w, cap, seed=1, sid=3, twins=(True,) if long else None,
                             cache_sample=LONG_CASES.get(name))
    say(f"[parity] {name}: {rep.summary(name)}")
    log_summary(rep, name)
    assert rep.ids_compared > 0
    # a row whose top-2 gap lies inside the margin is a tie both answers are
    # right for (skipped, counted); sampled rows may skip about as many as
    # their exact tie probabilities add up to, greedy rows a tenth
    assert rep.skip_bound_ok(), rep.summary(name)


def test_restored_offset_and_gap(cuda):
    """open() at a restored offset skips the held prefix; a run past the
    frontier is refused with the state unchanged (dflash.go committed)."""
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg, seed=2)
    d = _drafter(cfg, w)
    fs = synth.FeatureSource(cfg, 2)
    s = d.session(128)
    s.committed(fs.tokens(0, 20), feats_dev(cfg, fs.features(0, 20)), 0)
    st = s.state()
    from block_diffusion_drafter_fwd_amd import ContextGap
    with pytest.raises(ContextGap):
        s.committed([1, 2], torch.zeros((2, cfg.fc_in), device="cuda"), 25)
    assert s.state() == st


def test_committed_rows_from_unaligned_features(cuda):
    """Feature rows whose device address is not 16-byte aligned take the
    separate history write + copy path; both paths leave the same cache and
    the same block logits (bit for bit)."""
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg, seed=3)
    d = _drafter(cfg, w)
    fs = synth.FeatureSource(cfg, 4)
    T = 11                                  # below the flush threshold: rows stay pending until propose
    feats = feats_dev(cfg, fs.features(0, T))
    flat = torch.empty(feats.numel() + 1, dtype=feats.dtype, device="cuda")
    flat[1:].copy_(feats.reshape(-1))
    unaligned = flat[1:].view(feats.shape)  # contiguous, 4-byte aligned
    assert unaligned.data_ptr() % 16 != 0
    outs = []
    for f in (feats, unaligned):
        s = d.session(128)
        s.committed(fs.tokens(0, T), f, 0)
        n, lg, _ = s.propose(int(fs.tokens(T, 1)[0]), cfg.block_size - 1)
        k, v = s.cache_read(0, 0, T)
        torch.cuda.synchronize()
        outs.append((lg[:n].cpu(), k.cpu(), v.cpu()))
        s.close()
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


def test_truncated_block_matches_full_block_under_causal_mask(cuda):
    """Drafting n < B-1 rows gives the full block's first n rows when the block
    mask is causal (rows never see later rows): the truncation is exact there,
    as the pages say; the bidirectional shift is measured by bench.py."""
    cfg = synth.config("tiny")
    assert cfg.causal
    w = synth.make_weights(cfg, seed=5)
    d = _drafter(cfg, w)
    fs = synth.FeatureSource(cfg, 6)
    s = d.session(128)
    s.committed(fs.tokens(0, 40), feats_dev(cfg, fs.features(0, 40)), 0)
    cur = int(fs.tokens(40, 1)[0])
    n_full, full, _ = s.propose(cur, cfg.block_size - 1)
    full = full.cpu().clone()
    s.commit_block()
    assert n_full == cfg.block_size - 1
    for n in range(1, cfg.block_size - 1):
        k, part, _ = s.propose(cur, n)
        s.commit_block()
        assert k == n
        e = rel_err(part.double().cpu().numpy(), full[:n].double().numpy())
        assert e < 1e-5, (n, e)
    s.close()


BATCHED = {
    # vocab 4099: the block-path and unembedding GEMMs take the 4-wave tiled kernel
    "small_vocab": (4099, [260, 300, 17, 0, 45], [15, 3, 7, 5, 1]),
    # vocab 20011 over 46 rows: the unembedding has enough column tiles for
    # the 8-wave 256 x 128 kernel (ragged last tile)
    "large_vocab": (20011, [130, 0, 70, 33], [15, 15, 15, 15]),
    # 270 logit rows over vocab 66001 (516 column tiles): the unembedding takes
    # the 512 x 128 tile form of the 8-wave kernel (all rows in one tile)
    "rows_over_256": (66001, [37, 0, 52, 18, 90, 25, 61, 44, 33, 70, 29, 48, 56, 21, 64, 39, 27, 81, 45],
                      [15] * 19, 2),
    # 63 sessions whose keys exceed one resident round of attention
    # workgroups: the split runs in several rounds, items dispatched largest
    # first, the chunk chosen by the host's schedule model (the 1300-key
    # sessions split into several items at the smaller candidates); 945 logit
    # rows take the tiled unembedding with four row tiles
    "multi_round": (3001, [30] * 57 + [1300] * 6, [15] * 63, 2, 1400),
}


@pytest.mark.parametrize("case", list(BATCHED))
def test_batched_propose_matches_oracle(cuda, case):
    """dflash_propose_batch over sessions of ragged context (one with none)
    equals each session's own oracle propose; one batched sample call draws
    every row with per-session penalties."""
    from block_diffusion_drafter_fwd_amd import committed_batch, propose_batch, sample
    from oracle.sampler import sample_row
    vocab, lens, mts = BATCHED[case][:3]
    rounds = BATCHED[case][3] if len(BATCHED[case]) > 3 else 3
    capacity = BATCHED[case][4] if len(BATCHED[case]) > 4 else 512
    cfg = synth.config("qwen", layers=2, vocab=vocab)
    w = synth.make_weights(cfg, seed=4, gains="random")
    d = _drafter(cfg, w, max_sessions=len(lens))
    pairs = [Pair(d, cfg, w, capacity, seed=4, sid=k) for k in range(len(lens))]
    srcs = [synth.FeatureSource(cfg, 4, k) for k in range(len(lens))]
    for k, (pr, L) in enumerate(zip(pairs, lens)):
        for p in range(0, L, 100):
            T = min(100, L - p)
            pr.committed(srcs[k].tokens(p, T), srcs[k].features(p, T), p)
    rep = Report()
    rng = np.random.default_rng(0)
    for r in range(rounds):
        say(f"[parity] batched round {r}")
        cur = [int(x) for x in rng.integers(0, cfg.vocab - 1, len(lens))]
        outs = [[o.propose(c, m) for o in pr.o] for pr, c, m in zip(pairs, cur, mts)]
        offs, logits = propose_batch([pr.g for pr in pairs], cur, mts)
        for k, pr in enumerate(pairs):
            pr.check_state(f"batched round {r} session {k}")
            rows = logits[offs[k]:offs[k + 1]].double().cpu().numpy()
            if outs[k][0] is None:
                assert offs[k + 1] == offs[k]
                continue
            for j, out in enumerate(outs[k]):
                e = rel_err(rows, out["logits"])
                rep.note(f"logits[{j}]", e)
                assert e < tol(cfg), (k, j, e)
        ids, probs = sample([pr.g for pr in pairs], offs, logits, 0.7, 1.1, 512, r, probs=True)
        ids = ids.cpu().numpy()
        ref, ref_probs = [], []
        for k, pr in enumerate(pairs):
            if outs[k][0] is None:
                continue
            o = pr.o[-1]
            for i in range(outs[k][-1]["n"]):
                z = outs[k][-1]["logits"][i]
                oid, op, sc = sample_row(z, o.history[-512:], 0.7, 1.1, 4, k, r, i)
                ref.append((oid, sc, id_margin(cfg, logits[offs[k] + i].double().cpu().numpy(), z, 0.7, 1.1)))
                ref_probs.append(op)
                e = rel_err(probs[offs[k] + i].double().cpu().numpy(), op)
                pt = probs_tol(logits[offs[k] + i].double().cpu().numpy(), z, 0.7)
                rep.note("probs", e)
                rep.note("probs/bound", e / pt)
                assert e < pt, (k, i, e, pt)
        check_ids(ids, ref, rep, ref_probs)
        # every session's accepted run in one dflash_committed_batch call; the
        # oracle commits session by session
        bs, runs, fts, poss = [], [], [], []
        for k, pr in enumerate(pairs):
            pr.commit_block()
            F = pr.o[0].ctx_offset + pr.o[0].pending_count
            if F:
                toks = np.array([cur[k], 7], dtype=np.int32)
                for o in pr.o:
                    o.committed(toks, srcs[k].features(F, 2), F)
                bs.append(pr.g)
                runs.append(toks)
                fts.append(feats_dev(cfg, srcs[k].features(F, 2)))
                poss.append(F)
        if bs:
            committed_batch(bs, runs, fts, poss)
    say(f"[parity] batched {case}: {rep.summary(case)}")
    log_summary(rep, f"batched_{case}")
    for pr in pairs:
        pr.flush()
        pr.check_state("final")
        pr.check_cache(rep)
    assert rep.ids_compared > 0
    assert rep.skip_bound_ok(), rep.summary(case)


def test_batched_workload_at_full_size_sampled_sessions(cuda):
    """The batched workload at full size, in the launch configuration the
    bench times: 64 sessions with log-uniform prompts of 1050..15434 slots
    (363424 in all) flushed in 256-row chunks, the 5-layer model and the
    151936-token vocabulary, one batched propose with U{1..15} drafted rows
    per session (the tiled block GEMMs and the paired SwiGLU epilogue, the
    multi-round attention split over the host's largest-first order, the
    256 x 256 unembedding tiles) and one batched sample with penalties and
    probabilities.  A session's rows depend only on its own context, so the
    oracle computes three of them on their own: the shortest, the median and
    the longest.  Feature rows repeat with period 4096 (slot S carries the
    seeded row S mod 4096, as in the bench)."""
    from block_diffusion_drafter_fwd_amd import propose_batch, sample
    from oracle.model import DraftModel
    from oracle.sampler import sample_row
    from oracle.session import OracleSession
    wl = synth.WORKLOADS["batched"]
    cfg = synth.config(wl.config)
    B, S, period = cfg.block_size, wl.sessions, 4096
    assert period % wl.commit_rows == 0
    lens = synth.session_lengths(wl, 0)
    say("[parity] batched full size: weights")
    w = synth.make_weights(cfg, seed=2, gains="random")
    d = _drafter(cfg, w, max_sessions=S)
    fs = synth.FeatureSource(cfg, 0, 0)
    toks, feats = fs.tokens(0, period), fs.features(0, period)
    feats_d = feats_dev(cfg, feats)

    def chunks(L):
        for p in range(0, L, wl.commit_rows):
            o = p % period
            yield p, o, min(wl.commit_rows, L - p)

    say(f"[parity] batched full size: {sum(lens)} prompt rows on the GPU")
    sess = [d.session(L + 4 * B, seed=0, stream_id=k) for k, L in enumerate(lens)]
    for k, s in enumerate(sess):
        for p, o, T in chunks(lens[k]):
            s.committed(toks[o:o + T], feats_d[o:o + T], p)
        s.flush()
    rng = np.random.default_rng(7)
    cur = [int(x) for x in rng.integers(0, cfg.vocab, S)]
    mts = [int(x) for x in rng.integers(1, B, S)]
    offs, logits = propose_batch(sess, cur, mts)
    ids, probs = sample(sess, offs, logits, wl.temperature, wl.rep_penalty, wl.history, 0, probs=True)
    assert offs[S] == sum(mts)
    ids = ids.cpu().numpy()
    order = np.argsort(lens, kind="stable")
    models = [DraftModel(cfg, w, emulate_bf16=e) for e in (False, True)]
    rep = Report()
    ref, ref_probs = [], []
    for k in (int(order[0]), int(order[S // 2]), int(order[-1])):
        say(f"[parity] batched full size: oracle session {k} ({lens[k]} slots, {mts[k]} rows)")
        os_ = [OracleSession(m) for m in models]
        for o in os_:
            for p, q, T in chunks(lens[k]):
                o.committed(toks[q:q + T], feats[q:q + T], p)
            o.flush()
        outs = [o.propose(cur[k], mts[k]) for o in os_]
        assert offs[k + 1] - offs[k] == outs[0]["n"] == mts[k]
        z_gpu = logits[offs[k]:offs[k + 1]].double().cpu().numpy()
        for j, out in enumerate(outs):
            e = rel_err(z_gpu, out["logits"])
            rep.note(f"logits[{j}]", e)
            assert e < tol(cfg), (k, j, e)
        hist = os_[-1].history[-wl.history:]
        for i in range(mts[k]):
            z = outs[-1]["logits"][i]
            oid, op, sc = sample_row(z, hist, wl.temperature, wl.rep_penalty, 0, k, 0, i)
            ref.append((oid, sc, id_margin(cfg, z_gpu[i], z, wl.temperature, wl.rep_penalty)))
            ref_probs.append(op)
            e = rel_err(probs[offs[k] + i].double().cpu().numpy(), op)
            pt = probs_tol(z_gpu[i], z, wl.temperature)
            rep.note("probs/bound", e / pt)
            assert e < pt, (k, i, e, pt)
        sel = slice(offs[k], offs[k + 1])
        check_ids(ids[sel], ref[-mts[k]:], rep, ref_probs[-mts[k]:])
    say(f"[parity] batched full size: {rep.summary('batched_full')}")
    log_summary(rep, "batched_full")
    assert rep.ids_compared > 0
    assert rep.skip_bound_ok(), rep.summary("batched_full")


def test_long_context_cache_rows_at_full_length(cuda):
    """The long configuration's whole 131072-slot prompt through 256-row
    flushes, checked at sampled slots: a context row's K/V depend only on the
    features at its own slot and its position (DFlash context rows are local
    to their slot), so the oracle computes just the sampled rows.  Feature
    rows repeat with period 4096 (row S carries the seeded features of row
    S mod 4096, as in the bench); positions, slots and RoPE angles run over
    the full length."""
    from oracle.model import DraftModel
    cfg = synth.config("long")
    w = synth.make_weights(cfg, seed=0, gains="random")
    d = _drafter(cfg, w)
    total, period = 131072, 4096
    s = d.session(total + cfg.block_size)
    src = synth.FeatureSource(cfg, seed=0, session=0)
    feats = src.features(0, period)
    toks = src.tokens(0, period)
    fd = feats_dev(cfg, feats)
    say(f"long full-length flush: {total} slots in {cfg.flush_rows}-row flushes")
    for p0 in range(0, total, period):
        s.committed(toks, fd, p0)
    s.flush()
    torch.cuda.synchronize()
    assert s.state()[0] == total and s.state()[1] == 0
    slots = np.array([0, 1, 255, 256, 4095, 4096, 65535, 65536, 100003, total - 257, total - 2, total - 1])
    for emulate in (False, True):
        model = DraftModel(cfg, w, emulate_bf16=emulate)
        ref = model.context_kv(feats[slots % period], slots)
        for l in range(cfg.layers):
            for j, S in enumerate(slots):
                k, v = s.cache_read(l, int(S), 1)
                k = k.double().cpu().numpy()[0]
                v = v.double().cpu().numpy()[0]
                ek, ev = rel_err(k, ref[l][0][j]), rel_err(v, ref[l][1][j])
                assert ek < tol(cfg) and ev < tol(cfg), (emulate, l, int(S), ek, ev)
    s.close()
    d.close()


@pytest.mark.parametrize("name", ["qwen", "laguna"])
def test_one_call_many_chunks_matches_oracle(cuda, name):
    """One committed call of 1100 rows after 37 pending ones: the library
    flushes it in 256-row chunks, every second chunk read from the caller's
    rows on the session's second stream with the workspace's second set of
    context buffers (the first chunk, which takes the pending rows through
    the pending buffer, stays on the session's stream).  Cache rows at slots
    in every chunk (the window's on laguna: only its last 511 rows are
    projected, in two chunks) and a propose right after the call (ordered
    behind both streams) match the oracle; a second large call then
    continues the context."""
    from oracle.model import DraftModel
    from oracle.session import OracleSession
    cfg = synth.config(name, layers=2, vocab=4099 if name == "laguna" else 5003)
    w = synth.make_weights(cfg, seed=3, gains="random")
    d = _drafter(cfg, w)
    cap = 2400 + 64 if not cfg.window else cfg.window + cfg.block_size - 1
    s = d.session(cap)
    src = synth.FeatureSource(cfg, seed=3, session=0)
    o = OracleSession(DraftModel(cfg, w, emulate_bf16=True))
    T0, T1, T2 = 37, 1100, 1000
    feats = src.features(0, T0 + T1 + T2)
    toks = src.tokens(0, T0 + T1 + T2)
    fd = feats_dev(cfg, feats)
    s.committed(toks[:T0], fd[:T0], 0)
    o.committed(toks[:T0], feats[:T0], 0)
    s.committed(toks[T0:T0 + T1], fd[T0:T0 + T1], T0)
    o.committed(toks[T0:T0 + T1], feats[T0:T0 + T1], T0)
    torch.cuda.synchronize()
    F = T0 + T1
    assert s.state()[0] == F and s.state()[1] == 0
    lo = F - (cfg.window - 1) if cfg.window else 0
    slots = np.array([x for x in (0, 36, 37, 255, 256, 292, 293, 511, 548, 549, 804, 805, 1060, 1061, F - 2, F - 1)
                      if x >= lo])
    model = DraftModel(cfg, w, emulate_bf16=True)
    ref = model.context_kv(feats[slots], slots)
    for l in range(cfg.layers):
        for j, S in enumerate(slots):
            k, v = s.cache_read(l, int(S), 1)
            ek = rel_err(k.double().cpu().numpy()[0], ref[l][0][j])
            ev = rel_err(v.double().cpu().numpy()[0], ref[l][1][j])
            assert ek < tol(cfg) and ev < tol(cfg), (l, int(S), ek, ev)
    anchor = int(toks[F])
    n, logits, _ = s.propose(anchor, cfg.block_size - 1)
    out = o.propose(anchor, cfg.block_size - 1)
    err = rel_err(logits.double().cpu().numpy(), out["logits"])
    say(f"[one call, many chunks] {name}: {len(slots)} slots x {cfg.layers} layers, logits rel err {err:.2e}")
    assert n == out["logits"].shape[0] and err < tol(cfg), err
    s.commit_block()
    o.commit_block()
    s.committed(toks[F:F + T2], fd[F:F + T2], F)
    o.committed(toks[F:F + T2], feats[F:F + T2], F)
    anchor = int(toks[F + T2 - 1])
    n, logits, _ = s.propose(anchor, cfg.block_size - 1)
    out = o.propose(anchor, cfg.block_size - 1)
    err = rel_err(logits.double().cpu().numpy(), out["logits"])
    assert err < tol(cfg), err
    s.close()
    d.close()


@pytest.mark.parametrize("name", ["qwen", "laguna"])
def test_flush_batch_matches_oracle(cuda, name):
    """dflash_flush_batch over sessions sharing a workspace (one with no
    rows, one with an outstanding block, ragged pending counts; the window
    ring and its drop-before-fc on laguna) leaves every session in the state,
    and with the cache rows, of the oracle's flush of each session."""
    from block_diffusion_drafter_fwd_amd import flush_batch
    cfg = synth.config(name, layers=2, vocab=3001)
    w = synth.make_weights(cfg, seed=5, gains="random")
    d = _drafter(cfg, w, max_sessions=4)
    cap = 2048 if not cfg.window else cfg.window + cfg.block_size - 1
    pairs = [Pair(d, cfg, w, cap, seed=5, sid=k) for k in range(4)]
    srcs = [synth.FeatureSource(cfg, 5, k) for k in range(4)]
    rep = Report()
    for r, counts in enumerate([(3, 0, 9, 255), (1, 17, 0, 200)]):
        say(f"[parity] flush_batch {name} pass {r}")
        if r == 0:   # session 2 drafts a block first, so the batched flush has to rewind it
            pairs[2].committed(srcs[2].tokens(0, 4), srcs[2].features(0, 4), 0)
            pairs[2].propose(11, 5, rep, hidden=False)
        for k, (pr, T) in enumerate(zip(pairs, counts)):
            F = pr.o[0].ctx_offset + pr.o[0].pending_count
            if T:
                pr.committed(srcs[k].tokens(F, T), srcs[k].features(F, T), F)
        for pr in pairs:
            for o in pr.o:
                o.flush()
        flush_batch([pr.g for pr in pairs])
        for k, pr in enumerate(pairs):
            pr.check_state(f"flush_batch pass {r} session {k}")
            pr.check_cache(rep)
    say(f"[parity] flush_batch {name} worst {rep.worst}")


@pytest.mark.parametrize("V", [3001, 8192])
def test_sample_rows_with_masked_logits(cuda, V):
    """Rows whose logits are mostly -inf (a caller's banned tokens: the first
    2048 ids of every row, so whole groups of eight that a thread meets first,
    and half of the rest), with the penalty on: the probabilities are those of
    the oracle (zero on the masked ids, summing to one: no NaN from a thread
    that has seen only -inf), and the ids are never masked and equal the
    oracle's draws where the top-2 gap exceeds the tie margin.  V = 3001 takes
    the bounds-checked pass, V = 8192 the one for whole groups of eight."""
    from block_diffusion_drafter_fwd_amd import sample
    from oracle.sampler import sample_row
    cfg = synth.config("qwen", layers=1, vocab=V)
    w = synth.make_weights(cfg, seed=8, gains="random")
    d = _drafter(cfg, w, max_sessions=1)
    s = d.session(1024, seed=8, stream_id=0)
    fs = synth.FeatureSource(cfg, 8, 0)
    toks = 2040 + (np.arange(40) * 13) % 90          # history straddling the masked prefix, penalised
    s.committed(toks, feats_dev(cfg, fs.features(0, 40)), 0)
    rng = np.random.default_rng(V)
    z = rng.normal(scale=2.0, size=(12, V)).astype(np.float32)
    z[:, :2048] = -np.inf
    z[:, 2048:][rng.random((12, V - 2048)) < 0.5] = -np.inf
    logits = torch.from_numpy(z).cuda()
    rep = Report()
    for rnd, (T, probs) in enumerate(((0.0, False), (0.7, True))):
        ids, pr = sample([s], [0, 12], logits, T, 1.3, 512, rnd, probs=probs)
        ids = ids.cpu().numpy()
        assert np.all(np.isfinite(z[np.arange(12), ids])), ids
        zd = z.astype(np.float64)
        zf = np.where(np.isfinite(zd), zd, 0.0)         # (the margins look at the finite logits)
        ref, orows = [], []
        for i in range(12):
            oid, op, sc = sample_row(zd[i], list(toks), T, 1.3, 8, 0, rnd, i)
            ref.append((oid, sc, id_margin(cfg, zf[i], zf[i], T, 1.3)))
            orows.append(op)
        check_ids(ids, ref, rep, orows if probs else None)
        if probs:
            pg = pr.double().cpu().numpy()
            assert np.all(np.isfinite(pg))
            assert np.all(pg[~np.isfinite(z)] == 0.0)
            np.testing.assert_allclose(pg.sum(axis=1), 1.0, atol=1e-5)
            np.testing.assert_allclose(pg, np.stack(orows), rtol=1e-4, atol=1e-8)
    say(f"[parity] masked sampling V={V}: ids compared {rep.ids_compared}")
    assert rep.ids_compared >= 18


def test_one_session_sample_equals_table_path_and_sees_deferred_history(cuda):
    """A one-session sample call (its descriptor in the kernel arguments, no
    tables) draws exactly what the same session draws inside a two-session
    call (tables), and both see the prompt's history tokens, which a flushing
    commit leaves on the host until the sample writes them to the ring: the
    ids equal the oracle's draws with that history wherever the top-2 gap
    exceeds the tie margin."""
    from block_diffusion_drafter_fwd_amd import sample
    from oracle.sampler import sample_row
    cfg = synth.config("qwen", layers=1, vocab=3001)
    w = synth.make_weights(cfg, seed=6, gains="random")
    d = _drafter(cfg, w, max_sessions=2)
    ss = [d.session(1024, seed=6, stream_id=k) for k in range(2)]
    fs = synth.FeatureSource(cfg, 6, 0)
    toks = (np.arange(300) * 7) % 50                 # history: ids 0..49, penalised
    for s in ss:
        s.committed(toks, feats_dev(cfg, fs.features(0, 300)), 0)   # 300 >= 256 rows: flushes
    gen = torch.Generator(device="cuda").manual_seed(6)
    logits = torch.randn((30, cfg.vocab), generator=gen, device="cuda") * 2
    logits[:, :50] += 3.0                            # the penalised ids would win without the penalty
    rep = Report()
    for rnd, (T, probs) in enumerate(((0.0, False), (0.7, True))):
        ids1, p1 = sample([ss[0]], [0, 15], logits[:15], T, 1.3, 512, rnd, probs=probs)
        ids2, p2 = sample(ss, [0, 15, 30], logits, T, 1.3, 512, rnd, probs=probs)
        assert torch.equal(ids1.cpu(), ids2[:15].cpu())
        if probs:
            assert torch.equal(p1.cpu(), p2[:15].cpu())
        z = logits.double().cpu().numpy()
        ref = []
        for i in range(15):
            oid, _, sc = sample_row(z[i], list(toks), T, 1.3, 6, 0, rnd, i)
            ref.append((oid, sc, id_margin(cfg, z[i], z[i], T, 1.3)))
        check_ids(ids1.cpu().numpy(), ref, rep)
    assert rep.ids_compared >= 25
