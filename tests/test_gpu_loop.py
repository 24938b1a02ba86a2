"""GPU parity of the closed speculative round, chained on the GPU: propose ->
dflash_sample (ids and, when sampling, the proposal probabilities) ->
dflash_verify against a seeded synthetic target -> dflash_commit_block +
dflash_committed of the anchor and the accepted drafts, the correction or
bonus token becoming the next anchor (Ollama ``mlxrunner/dflash.go``,
``propose``: verification uses the actual proposal distribution; mlxcel PR
"add the Laguna DFlash drafter", review commit: the greedy round loop
verifies by a raw per-position argmax).

The oracle runs the same loop with its own draws and ``oracle.verify``.  The
synthetic target (``synth.SyntheticTarget``) is built from the oracle's
drafted ids, so both sides verify against identical logits wherever they
drafted the same ids.  Every round compares the drafted ids (ties excepted,
as in every sampler check), the accepted count and the next token exactly,
and the session state after the commit bit for bit.  A round whose outcome
sits on a tie (a drafted id inside the tie margin, an acceptance test
u*q(x) vs p(x) or a correction draw within the proposal probabilities'
measured deviation) has two right answers: the GPU session then commits the
oracle's outcome so both stay on one path; such rounds are counted, each
must be a round with a tie, and at least half the rounds must run on the
GPU's own outcomes.
"""
import numpy as np
import pytest
import torch

import synth
from oracle.sampler import sample_row
from oracle.verify import softmax, verify_block
from tests.parity import Pair, Report, check_ids, device_tensors, feats_dev, id_margin, log_summary, rel_err

pytestmark = pytest.mark.gpu

ROUNDS = 20
CASES = {
    # name: (config, temperature, repetition penalty)
    "qwen_greedy": (synth.config("qwen", layers=2, vocab=5003), 0.0, 1.0),
    "qwen_sampling": (synth.config("qwen", layers=2, vocab=5003), 0.7, 1.1),
    "long_sampling": (synth.config("long", layers=1, vocab=3001), 1.0, 1.0),
}


@pytest.fixture(scope="module")
def cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_fwd_amd import abi
    abi.load("hip")
    return True


def _close(info, a, n, tgt, o_q, x_dev, row_dev, temperature):
    """Is the oracle's verification decision within the deviation of the
    GPU's inputs, i.e. a tie both outcomes are right for?  x_dev[i]: the
    GPU's proposal probability of draft i minus the oracle's (absolute);
    row_dev[i]: the largest such difference over row i."""
    if temperature == 0.0:
        return False                      # identical fp32 target rows: the argmax is exact
    for (uq, p), dq in zip(info["tests"], x_dev):
        if abs(uq - p) <= dq + 1e-5 * max(uq, p, 1e-30):
            return True
    sc = np.asarray(info["scores"], dtype=np.float64)
    fin = np.flatnonzero(np.isfinite(sc))
    if fin.size < 2:
        return False
    t1, t2 = fin[np.argsort(sc[fin])[-2:]][::-1]
    gap = sc[t1] - sc[t2]
    if a == n:                            # bonus draw from target row / T: fp32 rounding only
        return gap < 1e-4
    # correction draw: log(max(0, p - q)) moves by at most row_dev / residual
    pa = softmax(tgt[a], temperature)
    r = np.maximum(0.0, pa - np.asarray(o_q[a], dtype=np.float64))
    slack = sum(row_dev[a] / r[t] if r[t] > 0 else np.inf for t in (t1, t2))
    return gap < 1e-4 + slack


@pytest.mark.parametrize("name", list(CASES))
def test_closed_round_matches_oracle(cuda, name):
    from block_diffusion_drafter_fwd_amd import Drafter, sample, verify
    cfg, T, rho = CASES[name]
    seed, sid = 11, 2
    B = cfg.block_size
    w = synth.make_weights(cfg, seed=seed, gains="random")
    d = Drafter(cfg, device_tensors(cfg, w))
    fs = synth.FeatureSource(cfg, seed, sid)
    target = synth.SyntheticTarget(cfg.vocab, seed=seed, session=sid)
    ctx = 300
    pr = Pair(d, cfg, w, ctx + (ROUNDS + 2) * B + 64, seed=seed, sid=sid)
    for p in range(0, ctx, 100):
        pr.committed(fs.tokens(p, 100), fs.features(p, 100), p)
    current = int(fs.tokens(ctx, 1)[0])
    rep = Report()
    forced, ties, accepted, emitted = 0, 0, [], 0
    for r in range(ROUNDS):
        n, logits, out = pr.propose(current, B - 1, rep, hidden=False)
        pr.check_state(f"round {r} propose")
        ids_d, probs_d = sample([pr.g], [0, n], logits, T, rho, 512, r, probs=T > 0)
        o = pr.o[-1]
        hist = o.history[-512:]
        o_ids, o_q, ref, ref_p = [], [], [], []
        for i in range(n):
            oid, oprob, score = sample_row(out["logits"][i], hist, T, rho, seed, sid, r, i)
            o_ids.append(oid)
            o_q.append(oprob)
            ref.append((oid, score, id_margin(cfg, logits[i].double().cpu().numpy(), out["logits"][i], T, rho)))
            ref_p.append(oprob)
        ids_g = ids_d.cpu().numpy()
        skipped_before = rep.ids_skipped
        check_ids(ids_g, ref, rep, ref_p if T > 0 else None)
        tie_row = rep.ids_skipped > skipped_before
        x_dev, row_dev = [], []
        if T > 0:
            pg = probs_d.double().cpu().numpy()
            for i in range(n):
                x = int(o_ids[i])
                x_dev.append(abs(pg[i, x] - o_q[i][x]))
                row_dev.append(float(np.max(np.abs(pg[i] - o_q[i]))))
                assert rel_err(pg[i], o_q[i]) < 5e-2, (r, i)
        # the target of this round, from the oracle's drafted ids, on both sides
        tgt = target.rows(r, o_ids)
        acc_d, nxt_d = verify([pr.g], [0, n], torch.from_numpy(tgt).cuda(), ids_d, probs_d, T, r)
        a_g, x_g = int(acc_d.cpu()[0]), int(nxt_d.cpu()[0])
        a_o, x_o, info = verify_block(tgt, o_ids, np.stack(o_q) if T > 0 and n else None, T, seed, sid, r)
        same_ids = np.array_equal(ids_g[:n], np.asarray(o_ids, dtype=ids_g.dtype))
        close = _close(info, a_o, n, tgt, o_q, x_dev, row_dev, T)
        ties += int(tie_row or close)
        if same_ids and not close:
            assert (a_g, x_g) == (a_o, x_o), (name, r, (a_g, x_g), (a_o, x_o))
            g_run = np.concatenate([[current], ids_g[:a_g]]).astype(np.int32)
        else:
            # check_ids has already passed: differing ids are tie rows, so a
            # forced round is always a round with a tie
            assert tie_row or close, (name, r)
            forced += 1                  # the GPU session follows the oracle's outcome
            g_run = np.concatenate([[current], o_ids[:a_o]]).astype(np.int32)
        o_run = np.concatenate([[current], o_ids[:a_o]]).astype(np.int32)
        # rewind the block and commit the anchor plus the accepted drafts
        pr.commit_block()
        F = pr.o[0].ctx_offset + pr.o[0].pending_count
        for oo in pr.o:
            oo.committed(o_run, fs.features(F, a_o + 1), F)
        pr.g.committed(g_run, feats_dev(cfg, fs.features(F, len(g_run))), F)
        pr.check_state(f"round {r} commit")
        assert list(g_run) == list(o_run)
        accepted.append(a_o)
        emitted += a_o + 1
        current = x_o
        rep.rounds += 1
    pr.flush()
    pr.check_state("final flush")
    pr.check_cache(rep)
    summ = rep.summary(f"closed_round_{name}")
    summ.update(forced_rounds=forced, tie_rounds=ties, accepted_per_round=float(np.mean(accepted)),
                emitted=emitted)
    print(f"[loop] {summ}", flush=True)
    log_summary(rep, f"closed_round_{name}")
    assert ROUNDS - forced >= ROUNDS // 2, summ                   # most rounds chained on the GPU alone
    assert sum(accepted) > 0 and max(accepted) >= 2, summ        # the loop commits multi-token runs
    assert rep.skip_bound_ok(), summ
