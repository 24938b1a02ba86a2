"""GPU parity of speculative verification (dflash_verify) against the oracle.

Random target logits over a ragged vocabulary (9001 ids: three 4096-id
chunks, the last one short) for five sessions of different draft lengths
(one with none), greedy and sampling; the drafts are argmax runs broken at
chosen places (greedy), or draws from a draft distribution q, with q equal
to the target's p in some rows and concentrated on a token the target gives
almost no mass in others (sampling).  Decisions whose two sides lie within
float32 rounding of each other are counted and skipped."""
import numpy as np
import pytest
import torch

import synth
from oracle.verify import softmax, verify_block

pytestmark = pytest.mark.gpu

V = 9001
DRAFTS = [7, 0, 3, 7, 5]


@pytest.fixture(scope="module")
def setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_fwd_amd import Drafter, abi
    from tests.parity import device_tensors
    abi.load("hip")
    cfg = synth.config("tiny", vocab=V)
    w = synth.make_weights(cfg, seed=9)
    d = Drafter(cfg, device_tensors(cfg, w), max_sessions=len(DRAFTS))
    sessions = [d.session(64, seed=100 + k, stream_id=k) for k in range(len(DRAFTS))]
    return cfg, d, sessions


def _offsets():
    return np.concatenate([[0], np.cumsum(DRAFTS)]).astype(np.int32)


@pytest.mark.parametrize("rnd", [0, 1, 2])
def test_greedy_verify_matches_oracle(setup, rnd):
    from block_diffusion_drafter_fwd_amd import verify
    cfg, d, sessions = setup
    rng = np.random.default_rng(rnd)
    offs = _offsets()
    target = rng.normal(scale=2.0, size=(int(offs[-1]) + len(DRAFTS), V)).astype(np.float32)
    ids = np.zeros(max(1, int(offs[-1])), np.int32)
    for k, n in enumerate(DRAFTS):
        r0 = offs[k] + k
        brk = int(rng.integers(0, n + 1))                   # drafts agree with the target up to here
        for i in range(n):
            am = int(np.argmax(target[r0 + i]))
            ids[offs[k] + i] = am if i < brk else (am + 1 + int(rng.integers(0, V - 1))) % V
    acc, nxt = verify(sessions, offs, torch.from_numpy(target).cuda(), torch.from_numpy(ids).cuda(), None,
                      0.0, rnd)
    acc, nxt = acc.cpu().numpy(), nxt.cpu().numpy()
    for k, n in enumerate(DRAFTS):
        r0 = offs[k] + k
        a, x, _ = verify_block(target[r0:r0 + n + 1], ids[offs[k]:offs[k] + n], None, 0.0, 100 + k, k, rnd)
        assert (acc[k], nxt[k]) == (a, x), (k, acc[k], nxt[k], a, x)


@pytest.mark.parametrize("rnd,temperature", [(0, 1.0), (1, 0.7), (2, 1.0), (3, 0.7)])
def test_sampling_verify_matches_oracle(setup, rnd, temperature):
    from block_diffusion_drafter_fwd_amd import verify
    cfg, d, sessions = setup
    rng = np.random.default_rng(10 + rnd)
    offs = _offsets()
    R = int(offs[-1])
    target = rng.normal(scale=2.0, size=(R + len(DRAFTS), V)).astype(np.float32)
    q = np.zeros((max(1, R), V), np.float32)
    ids = np.zeros(max(1, R), np.int32)
    for k, n in enumerate(DRAFTS):
        r0 = offs[k] + k
        for i in range(n):
            kind = int(rng.integers(0, 3))
            if kind == 0:                                   # the draft proposes from the target itself
                qi = softmax(target[r0 + i], temperature)
            elif kind == 1:                                 # an unrelated draft distribution
                qi = softmax(rng.normal(scale=2.0, size=V), 1.0)
            else:                                           # a confident draft on a token the target shuns
                qi = np.full(V, 1e-6)
                qi[int(np.argmin(target[r0 + i]))] = 1.0
                qi /= qi.sum()
            q[offs[k] + i] = qi.astype(np.float32)
            qi64 = q[offs[k] + i].astype(np.float64)
            ids[offs[k] + i] = int(rng.choice(V, p=qi64 / qi64.sum()))
    acc, nxt = verify(sessions, offs, torch.from_numpy(target).cuda(), torch.from_numpy(ids).cuda(),
                      torch.from_numpy(q).cuda(), temperature, rnd)
    acc, nxt = acc.cpu().numpy(), nxt.cpu().numpy()
    compared = skipped = 0
    for k, n in enumerate(DRAFTS):
        r0 = offs[k] + k
        a, x, info = verify_block(target[r0:r0 + n + 1], ids[offs[k]:offs[k] + n], q[offs[k]:offs[k] + n],
                                  temperature, 100 + k, k, rnd)
        close_test = any(abs(uq - p) <= 1e-5 * max(uq, p, 1e-30) for uq, p in info["tests"])
        sc = np.sort(info["scores"][np.isfinite(info["scores"])])
        close_draw = sc.size > 1 and sc[-1] - sc[-2] < 1e-4
        if close_test or close_draw:
            skipped += 1
            continue
        compared += 1
        assert (acc[k], nxt[k]) == (a, x), (k, acc[k], nxt[k], a, x)
    assert compared >= 3 and skipped <= 1, (compared, skipped)


@pytest.mark.parametrize("temperature", [0.0, 0.8])
def test_out_of_vocabulary_draft_ids_are_rejected_like_the_oracle(setup, temperature):
    """Draft ids outside [0, V) (-1, V, V + 1000) at the first, a middle and
    the last drafted row of different sessions: the draft is rejected there
    without reading the target or draft rows at that id, and the correction
    is drawn as after any rejection (the oracle's reading)."""
    from block_diffusion_drafter_fwd_amd import verify
    cfg, d, sessions = setup
    rng = np.random.default_rng(21)
    offs = _offsets()
    R = int(offs[-1])
    target = rng.normal(scale=2.0, size=(R + len(DRAFTS), V)).astype(np.float32)
    q = np.zeros((max(1, R), V), np.float32)
    ids = np.zeros(max(1, R), np.int32)
    bad = {0: (0, -1), 2: (1, V), 3: (6, V + 1000), 4: (4, -7)}        # session: (row, id)
    for k, n in enumerate(DRAFTS):
        r0 = offs[k] + k
        for i in range(n):
            if temperature > 0:
                # before the bad row the draft proposes from the target itself
                # (accepted); from it on from an unrelated distribution, so the
                # residual the correction is drawn from is well away from zero
                before = k in bad and i < bad[k][0]
                qi = softmax(target[r0 + i], temperature) if before else softmax(rng.normal(scale=2.0, size=V), 1.0)
                q[offs[k] + i] = qi.astype(np.float32)
                qi = q[offs[k] + i].astype(np.float64)
                ids[offs[k] + i] = int(rng.choice(V, p=qi / qi.sum()))
            else:
                ids[offs[k] + i] = int(np.argmax(target[r0 + i]))
    for k, (i, x) in bad.items():
        ids[offs[k] + i] = x
    probs = torch.from_numpy(q).cuda() if temperature > 0 else None
    acc, nxt = verify(sessions, offs, torch.from_numpy(target).cuda(), torch.from_numpy(ids).cuda(), probs,
                      temperature, 5)
    acc, nxt = acc.cpu().numpy(), nxt.cpu().numpy()
    compared = 0
    for k, n in enumerate(DRAFTS):
        r0 = offs[k] + k
        a, x, info = verify_block(target[r0:r0 + n + 1], ids[offs[k]:offs[k] + n],
                                  q[offs[k]:offs[k] + n] if temperature > 0 else None, temperature, 100 + k, k, 5)
        if k in bad:
            assert acc[k] <= bad[k][0]
        close_test = any(abs(uq - p) <= 1e-5 * max(uq, p, 1e-30) for uq, p in info["tests"] if np.isfinite(uq))
        sc = np.sort(info["scores"][np.isfinite(info["scores"])])
        if close_test or (temperature > 0 and sc.size > 1 and sc[-1] - sc[-2] < 1e-4):
            continue
        compared += 1
        assert (acc[k], nxt[k]) == (a, x), (k, acc[k], nxt[k], a, x)
        assert 0 <= nxt[k] < V
    assert compared >= 4, compared


@pytest.mark.parametrize("temperature", [0.0, 0.9])
def test_masked_target_rows_verify_like_the_oracle(setup, temperature):
    """Target rows masked to -inf on most ids (the first 2048, so whole runs a
    thread meets first, and half of the rest), drafts proposed from the
    masked target itself up to a point and from an unrelated distribution
    over the unmasked ids after it: (accepted, next) equal the oracle's, the
    normaliser stays finite (no NaN from a thread that has seen only -inf),
    and next is never a masked id."""
    from block_diffusion_drafter_fwd_amd import verify
    cfg, d, sessions = setup
    rng = np.random.default_rng(33)
    offs = _offsets()
    R = int(offs[-1])
    target = rng.normal(scale=2.0, size=(R + len(DRAFTS), V)).astype(np.float32)
    target[:, :2048] = -np.inf
    target[:, 2048:][rng.random((R + len(DRAFTS), V - 2048)) < 0.5] = -np.inf
    q = np.zeros((max(1, R), V), np.float32)
    ids = np.zeros(max(1, R), np.int32)
    for k, n in enumerate(DRAFTS):
        r0 = offs[k] + k
        brk = int(rng.integers(0, n + 1))
        for i in range(n):
            ok = np.isfinite(target[r0 + i])
            if temperature > 0:
                if i < brk:
                    qi = softmax(target[r0 + i], temperature)
                else:
                    qi = np.where(ok, softmax(np.where(ok, rng.normal(scale=2.0, size=V), -np.inf), 1.0), 0.0)
                q[offs[k] + i] = qi.astype(np.float32)
                qi = q[offs[k] + i].astype(np.float64)
                ids[offs[k] + i] = int(rng.choice(V, p=qi / qi.sum()))
            else:
                am = int(np.argmax(target[r0 + i]))
                ids[offs[k] + i] = am if i < brk else int(rng.choice(np.flatnonzero(ok & (np.arange(V) != am))))
    probs = torch.from_numpy(q).cuda() if temperature > 0 else None
    acc, nxt = verify(sessions, offs, torch.from_numpy(target).cuda(), torch.from_numpy(ids).cuda(), probs,
                      temperature, 7)
    acc, nxt = acc.cpu().numpy(), nxt.cpu().numpy()
    compared = 0
    for k, n in enumerate(DRAFTS):
        r0 = offs[k] + k
        assert np.isfinite(target[r0 + acc[k], nxt[k]]), (k, acc[k], nxt[k])
        a, x, info = verify_block(target[r0:r0 + n + 1], ids[offs[k]:offs[k] + n],
                                  q[offs[k]:offs[k] + n] if temperature > 0 else None, temperature, 100 + k, k, 7)
        close_test = any(abs(uq - p) <= 1e-5 * max(uq, p, 1e-30) for uq, p in info["tests"] if np.isfinite(uq))
        sc = np.sort(info["scores"][np.isfinite(info["scores"])])
        if close_test or (sc.size > 1 and sc[-1] - sc[-2] < 1e-4):
            continue
        compared += 1
        assert (acc[k], nxt[k]) == (a, x), (k, acc[k], nxt[k], a, x)
    assert compared >= 4, compared


def test_verify_rejects_sampling_without_draft_probabilities(setup):
    from block_diffusion_drafter_fwd_amd import DFlashError, verify
    cfg, d, sessions = setup
    offs = _offsets()
    target = torch.zeros((int(offs[-1]) + len(DRAFTS), V), device="cuda")
    ids = torch.zeros((int(offs[-1]),), dtype=torch.int32, device="cuda")
    with pytest.raises(DFlashError):
        verify(sessions, offs, target, ids, None, 0.5, 0)


def _block(rng, n, temperature):
    """Target rows (n + 1), draft ids and draft probabilities of one block:
    greedy drafts follow the target's argmax up to a random break; sampled
    drafts are drawn from a mix of the target's own p and unrelated q."""
    target = rng.normal(scale=2.0, size=(n + 1, V)).astype(np.float32)
    ids = np.zeros(max(1, n), np.int32)
    q = np.zeros((max(1, n), V), np.float32)
    brk = int(rng.integers(0, n + 1))
    for i in range(n):
        if temperature == 0.0:
            am = int(np.argmax(target[i]))
            ids[i] = am if i < brk else (am + 1 + int(rng.integers(0, V - 1))) % V
        else:
            qi = softmax(target[i], temperature) if rng.integers(0, 2) else softmax(rng.normal(scale=2.0, size=V), 1.0)
            q[i] = qi.astype(np.float32)
            qi64 = q[i].astype(np.float64)
            ids[i] = int(rng.choice(V, p=qi64 / qi64.sum()))
    return target, ids, q


@pytest.mark.parametrize("n", [0, 3, 7])
@pytest.mark.parametrize("temperature", [0.0, 0.7, 1.0])
def test_one_session_verify_equals_batched_and_oracle(setup, n, temperature):
    """A one-session call (its descriptor and draft count travel in the
    kernel arguments; no tables are uploaded) gives the same (accepted, next)
    as the same session inside a five-session call, and as the oracle; n = 0
    (only the bonus row) and n = blockSize - 1 included."""
    from block_diffusion_drafter_fwd_amd import verify
    cfg, d, sessions = setup
    rng = np.random.default_rng(100 + n + int(10 * temperature))
    rnd = 5 + n
    target, ids, q = _block(rng, n, temperature)
    T = torch.from_numpy(target).cuda()
    I = torch.from_numpy(ids).cuda()
    Q = torch.from_numpy(q).cuda() if temperature > 0 else None
    acc1, nxt1 = verify(sessions[:1], [0, n], T, I, Q, temperature, rnd)
    # the same block as session 0 of a five-session call (the others draft 2 each)
    others = [_block(rng, 2, temperature) for _ in range(4)]
    tg = np.concatenate([target] + [o[0] for o in others])
    ii = np.concatenate([ids[:n]] + [o[1][:2] for o in others]).astype(np.int32)
    qq = np.concatenate([q[:n]] + [o[2][:2] for o in others]).astype(np.float32)
    offs = np.array([0, n, n + 2, n + 4, n + 6, n + 8], np.int32)
    accb, nxtb = verify(sessions, offs, torch.from_numpy(tg).cuda(), torch.from_numpy(ii).cuda(),
                        torch.from_numpy(qq).cuda() if temperature > 0 else None, temperature, rnd)
    one = (int(acc1.cpu()[0]), int(nxt1.cpu()[0]))
    assert one == (int(accb.cpu()[0]), int(nxtb.cpu()[0]))
    a, x, info = verify_block(target, ids[:n], q[:n] if temperature > 0 else None, temperature, 100, 0, rnd)
    close = temperature > 0 and (any(abs(uq - p) <= 1e-5 * max(uq, p, 1e-30) for uq, p in info["tests"]) or
                                 (lambda sc: sc.size > 1 and sc[-1] - sc[-2] < 1e-4)(
                                     np.sort(info["scores"][np.isfinite(info["scores"])])))
    if not close:
        assert one == (a, x), (one, a, x)


@pytest.mark.parametrize("temperature", [0.0, 0.7, 1.0])
def test_long_drafts_verify_matches_oracle(temperature):
    """Drafts longer than the acceptance pass's 16 waves (48-token blocks:
    40 and 23 drafted rows, so waves take a second and third row): greedy
    drafts that follow the target's argmax to row 37 (of 40) and through all
    23 rows; sampled drafts from the target's own p with a confident draft on
    a token the target shuns at row 33 (40 rows) and none in the other."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_fwd_amd import Drafter, abi, verify
    from tests.parity import device_tensors
    abi.load("hip")
    cfg = synth.config("tiny", vocab=V, block_size=48)
    d = Drafter(cfg, device_tensors(cfg, synth.make_weights(cfg, seed=9)), max_sessions=2)
    sessions = [d.session(128, seed=300 + k, stream_id=k) for k in range(2)]
    drafts = [40, 23]
    offs = np.array([0, 40, 63], np.int32)
    rng = np.random.default_rng(77 + int(10 * temperature))
    target = rng.normal(scale=2.0, size=(63 + 2, V)).astype(np.float32)
    ids = np.zeros(63, np.int32)
    q = np.zeros((63, V), np.float32)
    for k, (n, brk) in enumerate(zip(drafts, [37, 23])):
        r0 = offs[k] + k
        for i in range(n):
            if temperature == 0.0:
                am = int(np.argmax(target[r0 + i]))
                ids[offs[k] + i] = am if i < brk else (am + 1) % V
            else:
                if k == 0 and i == 33:
                    qi = np.full(V, 1e-6)
                    qi[int(np.argmin(target[r0 + i]))] = 1.0
                    qi /= qi.sum()
                else:
                    qi = softmax(target[r0 + i], temperature)
                q[offs[k] + i] = qi.astype(np.float32)
                qi64 = q[offs[k] + i].astype(np.float64)
                ids[offs[k] + i] = int(rng.choice(V, p=qi64 / qi64.sum()))
    acc, nxt = verify(sessions, offs, torch.from_numpy(target).cuda(), torch.from_numpy(ids).cuda(),
                      torch.from_numpy(q).cuda() if temperature > 0 else None, temperature, 4)
    acc, nxt = acc.cpu().numpy(), nxt.cpu().numpy()
    compared = 0
    for k, n in enumerate(drafts):
        r0 = offs[k] + k
        a, x, info = verify_block(target[r0:r0 + n + 1], ids[offs[k]:offs[k] + n],
                                  q[offs[k]:offs[k] + n] if temperature > 0 else None, temperature, 300 + k, k, 4)
        if temperature > 0:
            sc = np.sort(info["scores"][np.isfinite(info["scores"])])
            if any(abs(uq - p) <= 1e-5 * max(uq, p, 1e-30) for uq, p in info["tests"]) or \
                    (sc.size > 1 and sc[-1] - sc[-2] < 1e-4):
                continue
        compared += 1
        assert (acc[k], nxt[k]) == (a, x), (k, acc[k], nxt[k], a, x)
        if temperature == 0.0:
            assert a == (37 if k == 0 else 23)
    assert compared >= 1
