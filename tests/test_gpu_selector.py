"""GPU parity of the DFlash2 candidate selector (dflash_select) against the
oracle (``oracle.selector``).

1. Seeded logits, the same float32 array on both sides, ragged sessions
   (none, one, three and seven rows), a ragged vocabulary (9001) and the long
   configuration's 262144, K = 8 and 16 candidates, bf16 and fp32 tables,
   T = 0, 0.7 and 1: the candidate ids equal the oracle's exactly (the
   logits are identical, so the top-K is exact, ties to the lower id), the
   candidate probabilities and the dense rows within float32 rounding, and
   the tokens position by position up to the first position whose two best
   scores lie within 1e-4 (a tie both answers are right for; counted).  The
   positions are chosen in order, each from the one before, so one wrong
   predecessor would change the rest.
2. The selector on the drafter's own logits (propose -> select), against
   the oracle's propose and selector: candidates where the K-th/K+1-th logit
   gap exceeds twice the rows' logit deviation, tokens until the first
   position inside the margin.
"""
import numpy as np
import pytest
import torch

import synth
from oracle.selector import candidates, select_block

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_fwd_amd import abi
    abi.load("hip")
    return True


def _bf16(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _drafter(cfg, seed, table_scale):
    from block_diffusion_drafter_fwd_amd import Drafter
    from tests.parity import device_tensors
    w = synth.make_weights(cfg, seed=seed)
    rng = np.random.default_rng(seed)
    for n in ("sel_prev", "sel_next"):
        t = rng.normal(scale=table_scale, size=w[n].shape).astype(np.float32)
        w[n] = _bf16(t) if cfg.dtype == "bf16" else t
    return Drafter(cfg, device_tensors(cfg, w), max_sessions=4), w


ROWS = [1, 0, 3, 7]


def _compare(rep, tok_g, cid_g, cpr_g, tok_o, cid_o, cpr_o, scores_o, temperature):
    """Candidates exact; probabilities to float32 rounding; tokens until the
    first tie.  Returns the number of positions compared."""
    n = len(tok_o)
    np.testing.assert_array_equal(cid_g, cid_o)
    if temperature > 0:
        np.testing.assert_allclose(cpr_g, cpr_o, rtol=2e-5, atol=1e-7)
    compared = 0
    for i in range(n):
        sc = np.sort(np.asarray(scores_o[i], dtype=np.float64))
        sc = sc[np.isfinite(sc)]                # (a row masked to -inf has no finite score to tie)
        if sc.size > 1 and sc[-1] - sc[-2] < 1e-4:
            rep["ties"] += 1
            break                           # the next positions depend on this choice
        assert int(tok_g[i]) == int(tok_o[i]), (i, tok_g, tok_o)
        compared += 1
    return compared


@pytest.mark.parametrize("dtype,V,K", [("fp32", 9001, 8), ("bf16", 9001, 16), ("bf16", 262144, 8)])
@pytest.mark.parametrize("temperature", [0.0, 0.7, 1.0])
def test_select_matches_oracle_on_identical_logits(cuda, dtype, V, K, temperature):
    from block_diffusion_drafter_fwd_amd import select
    base = synth.config("tiny") if dtype == "fp32" else synth.config("qwen", layers=1, hidden=256, intermediate=768,
                                                                          target_hidden=64, block_size=8)
    cfg = base.replace(vocab=V, sel_candidates=K, sel_dim=64 if dtype == "bf16" else 24)
    d, w = _drafter(cfg, seed=V % 97 + K, table_scale=0.6)
    sessions = [d.session(64, seed=30 + k, stream_id=k) for k in range(len(ROWS))]
    rng = np.random.default_rng(K + int(temperature * 10))
    offs = np.concatenate([[0], np.cumsum(ROWS)]).astype(np.int32)
    rep = {"ties": 0, "compared": 0}
    for rnd in range(3):
        logits = rng.normal(scale=1.5, size=(int(offs[-1]), V)).astype(np.float32)
        logits[0, :40] = logits[0, 40]                              # exact ties at the top of one row
        anchors = [int(x) for x in rng.integers(0, V, len(ROWS))]
        tok, cid, cpr, den = select(sessions, offs, torch.from_numpy(logits).cuda(), anchors, temperature, rnd,
                                    dense=True)
        tok, cid = tok.cpu().numpy(), cid.cpu().numpy()
        cpr = cpr.cpu().numpy() if cpr is not None else None
        den = den.cpu().numpy() if den is not None else None
        for k, n in enumerate(ROWS):
            if n == 0:
                continue
            sl = slice(offs[k], offs[k + 1])
            t_o, c_o, p_o, s_o = select_block(logits[sl], anchors[k], w["sel_prev"], w["sel_next"], K, temperature,
                                              30 + k, k, rnd)
            rep["compared"] += _compare(rep, tok[sl], cid[sl], cpr[sl] if cpr is not None else None, t_o, c_o, p_o,
                                        s_o, temperature)
            if den is not None:
                for i in range(n):
                    row = den[offs[k] + i]
                    assert np.count_nonzero(row) <= K
                    np.testing.assert_allclose(row[c_o[i]], p_o[i], rtol=2e-5, atol=1e-7)
                    assert abs(row.sum() - 1.0) < 1e-5
    print(f"[select] {dtype} V={V} K={K} T={temperature}: {rep}", flush=True)
    assert rep["compared"] >= 20 and rep["ties"] <= 2, rep


def test_select_on_drafted_rows_matches_oracle(cuda):
    """propose -> select on the drafter's own logits (bf16, the long
    configuration's head geometry, K = 4, T = 1): candidates and tokens
    against the oracle's propose + selector where the margins separate them
    (the draw's uniforms are keyed by candidate rank, so a row counts only
    when every rank of its top K is separated by more than twice the logits'
    deviation)."""
    from block_diffusion_drafter_fwd_amd import select
    from oracle.model import DraftModel
    from oracle.session import OracleSession
    from tests.parity import feats_dev
    cfg = synth.config("long", layers=1, hidden=1024, target_hidden=256, intermediate=3072, vocab=5003,
                       sel_candidates=4, sel_dim=64)
    d, w = _drafter(cfg, seed=12, table_scale=0.6)
    fs = synth.FeatureSource(cfg, 12, 0)
    s = d.session(512, seed=12, stream_id=0)
    o = OracleSession(DraftModel(cfg, w, emulate_bf16=True))
    s.committed(fs.tokens(0, 300), feats_dev(cfg, fs.features(0, 300)), 0)
    o.committed(fs.tokens(0, 300), fs.features(0, 300), 0)
    compared = ties = cand_rows = 0
    for rnd in range(8):
        anchor = int(fs.tokens(300 + rnd, 1)[0])
        n, logits, _ = s.propose(anchor, 7)
        out = o.propose(anchor, 7)
        tok, cid, cpr, _ = select([s], [0, n], logits, [anchor], 1.0, rnd)
        zg = logits.double().cpu().numpy()
        zo = out["logits"]
        dev = float(np.max(np.abs(zg - zo)))
        t_o, c_o, p_o, s_o = select_block(zo, anchor, w["sel_prev"], w["sel_next"], 4, 1.0, 12, 0, rnd)
        cid = cid.cpu().numpy()
        tok = tok.cpu().numpy()
        pr = cpr.cpu().numpy()
        for i in range(n):                                   # every row: a valid candidate distribution
            assert tok[i] in cid[i] and len(set(cid[i])) == 4
            assert abs(pr[i].sum() - 1.0) < 1e-5 and np.all(pr[i] > 0)
        separated = []
        for i in range(n):
            srt = np.sort(zo[i])[::-1]
            gaps = srt[:4] - srt[1:5]
            separated.append(bool(np.min(gaps) > 2 * dev))   # every rank of the top 4 is separated
            if separated[-1]:
                np.testing.assert_array_equal(cid[i], c_o[i])
                cand_rows += 1
        for i in range(n):
            # a position is comparable when its candidate set and its best
            # score are both outside the logits' deviation; past the first
            # that is not, the choices depend on a tie
            sc = np.sort(s_o[i])
            if not separated[i] or sc[-1] - sc[-2] < 1e-4 + 2 * dev:
                ties += 1
                break
            assert int(tok[i]) == int(t_o[i]), (rnd, i, tok, t_o)
            compared += 1
        s.commit_block()
        o.commit_block()
    print(f"[select e2e] tokens compared {compared}, ties {ties}, candidate rows {cand_rows}", flush=True)
    assert compared >= 1 and cand_rows >= 4


@pytest.mark.parametrize("temperature", [0.0, 0.7])
def test_select_rows_with_fewer_finite_logits_than_candidates(cuda, temperature):
    """Rows masked to -inf except for fewer than K tokens (a caller's banned
    tokens; one row with a single finite logit, one row whose finite logits
    all sit in the last, partial 4096-token chunk) and, greedy only, a row
    with no finite logit at all.  The K best are still K real tokens: the
    finite ones by value, then the lowest ids among the -inf ones, as the
    oracle's value-then-id order gives them; a -inf candidate gets
    probability 0 and is never drawn."""
    from block_diffusion_drafter_fwd_amd import select
    V, K = 9001, 8
    cfg = synth.config("qwen", layers=1, hidden=256, intermediate=768, target_hidden=64, block_size=8).replace(
        vocab=V, sel_candidates=K, sel_dim=64)
    d, w = _drafter(cfg, seed=5, table_scale=0.6)
    # finite tokens per row (all < K); greedy adds a row with none
    finite = [5, 1, 7, 3, 6] + ([] if temperature > 0 else [0])
    rows = [3, 2] + ([] if temperature > 0 else [1])
    sessions = [d.session(64, seed=40 + k, stream_id=k) for k in range(len(rows))]
    rng = np.random.default_rng(17)
    offs = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    logits = np.full((int(offs[-1]), V), -np.inf, dtype=np.float32)
    for r, m in enumerate(finite):
        lo = 8192 if r == 3 else 0                        # row 3: only the last chunk's tokens
        ids = rng.choice(np.arange(lo, V), size=m, replace=False)
        logits[r, ids] = rng.normal(scale=1.5, size=m).astype(np.float32)
    anchors = [int(x) for x in rng.integers(0, V, len(rows))]
    tok, cid, cpr, den = select(sessions, offs, torch.from_numpy(logits).cuda(), anchors, temperature, 2, dense=True)
    tok, cid = tok.cpu().numpy(), cid.cpu().numpy()
    assert np.all((cid >= 0) & (cid < V))
    for k, n in enumerate(rows):
        sl = slice(offs[k], offs[k + 1])
        t_o, c_o, p_o, s_o = select_block(logits[sl], anchors[k], w["sel_prev"], w["sel_next"], K, temperature,
                                          40 + k, k, 2)
        pr = cpr.cpu().numpy()[sl] if temperature > 0 else None
        rep = {"ties": 0}
        assert _compare(rep, tok[sl], cid[sl], pr, t_o, c_o, p_o, s_o, temperature) == n, rep
        for i in range(n):
            r = offs[k] + i
            assert np.isfinite(logits[r, tok[r]]) or finite[r] == 0
            if temperature > 0:
                assert np.all(pr[i][~np.isfinite(logits[r, cid[r]])] == 0.0)
                row = den.cpu().numpy()[r]
                assert np.count_nonzero(row) == finite[r] and abs(row.sum() - 1.0) < 1e-5


@pytest.mark.parametrize("temperature", [0.0, 0.7])
def test_one_session_select_equals_the_same_session_in_a_batch(cuda, temperature):
    """A one-session call (its descriptor and anchor in the kernel arguments,
    no table upload) gives bit for bit what the same session gets inside a
    four-session call: tokens, candidate ids, probabilities and dense rows."""
    from block_diffusion_drafter_fwd_amd import select
    V, K = 9001, 8
    cfg = synth.config("qwen", layers=1, hidden=256, intermediate=768, target_hidden=64, block_size=8).replace(
        vocab=V, sel_candidates=K, sel_dim=64)
    d, w = _drafter(cfg, seed=6, table_scale=0.6)
    sessions = [d.session(64, seed=50 + k, stream_id=k) for k in range(len(ROWS))]
    rng = np.random.default_rng(31)
    offs = np.concatenate([[0], np.cumsum(ROWS)]).astype(np.int32)
    logits = torch.from_numpy(rng.normal(scale=1.5, size=(int(offs[-1]), V)).astype(np.float32)).cuda()
    anchors = [int(x) for x in rng.integers(0, V, len(ROWS))]
    tok, cid, cpr, den = select(sessions, offs, logits, anchors, temperature, 4, dense=True)
    for k, n in enumerate(ROWS):
        if n == 0:
            continue
        sl = slice(int(offs[k]), int(offs[k + 1]))
        t1, c1, p1, d1 = select([sessions[k]], [0, n], logits[sl].contiguous(), [anchors[k]], temperature, 4,
                                dense=True)
        assert torch.equal(t1, tok[sl]) and torch.equal(c1, cid[sl])
        if temperature > 0:
            assert torch.equal(p1, cpr[sl]) and torch.equal(d1, den[sl])
