"""The allocation-free verification entry point (dflash_verify_noalloc)
against dflash_verify, through the C ABI, on the GPU.

Two calls in a row on the same sessions and outputs, the second with a
smaller input (fewer sessions, shorter drafts), greedy and sampling, at a
ragged vocabulary of 9001 ids and at the long configuration's 262144: the
accepted counts and next tokens equal dflash_verify's bit for bit (both run
the same kernels on the same inputs; only where their tables and statistics
live differs).  A call beyond the static array's size is refused with
DFLASH_E_CAPACITY and leaves the outputs untouched.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _inputs(rng, drafts, V, temperature):
    offs = np.concatenate([[0], np.cumsum(drafts)]).astype(np.int32)
    R = int(offs[-1])
    target = torch.from_numpy(rng.normal(scale=2.0, size=(R + len(drafts), V)).astype(np.float32)).cuda()
    ids = torch.from_numpy(rng.integers(0, V, size=max(1, R)).astype(np.int32)).cuda()
    # drafts that follow the target's argmax for a while, so some are accepted
    am = torch.argmax(target, dim=1).to(torch.int32).cpu().numpy()
    ids_h = ids.cpu().numpy()
    for k, n in enumerate(drafts):
        for i in range(min(n, int(rng.integers(0, n + 1)))):
            ids_h[offs[k] + i] = am[offs[k] + k + i]
    ids = torch.from_numpy(ids_h).cuda()
    probs = None
    if temperature > 0:
        q = torch.from_numpy(rng.normal(scale=2.0, size=(max(1, R), V)).astype(np.float32)).cuda()
        probs = torch.softmax(q, dim=1).contiguous()
    return offs, target, ids, probs


@pytest.mark.parametrize("V", [9001, 262144])
@pytest.mark.parametrize("temperature", [0.0, 0.7])
def test_noalloc_verify_equals_verify(V, temperature):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_fwd_amd import Drafter, verify, verify_noalloc
    from tests.parity import device_tensors
    cfg = synth.config("tiny", vocab=V)
    w = synth.make_weights(cfg, seed=3)
    d = Drafter(cfg, device_tensors(cfg, w), max_sessions=5)
    sessions = [d.session(64, seed=50 + k, stream_id=k) for k in range(5)]
    acc = torch.full((5,), -1, dtype=torch.int32, device="cuda")
    nxt = torch.full((5,), -1, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(V + int(10 * temperature))
    for rnd, (ss, drafts) in enumerate(((sessions, [7, 0, 3, 7, 5]), (sessions[:2], [2, 1]))):
        offs, target, ids, probs = _inputs(rng, drafts, V, temperature)
        a_ref, x_ref = verify(ss, offs, target, ids, probs, temperature, rnd)
        verify_noalloc(ss, offs, target, ids, probs, temperature, rnd, acc, nxt)
        torch.cuda.synchronize()
        k = len(ss)
        assert torch.equal(acc[:k].cpu(), a_ref.cpu()), (rnd, acc[:k].cpu(), a_ref.cpu())
        assert torch.equal(nxt[:k].cpu(), x_ref.cpu()), (rnd, nxt[:k].cpu(), x_ref.cpu())
        assert int(a_ref.sum()) > 0 or temperature > 0
    # one session alone (the descriptor in the kernel arguments, no tables)
    offs, target, ids, probs = _inputs(rng, [7], V, temperature)
    a_ref, x_ref = verify(sessions[:1], offs, target, ids, probs, temperature, 9)
    verify_noalloc(sessions[:1], offs, target, ids, probs, temperature, 9, acc, nxt)
    assert (int(acc[0]), int(nxt[0])) == (int(a_ref[0]), int(x_ref[0]))


def test_noalloc_verify_refuses_more_than_its_array():
    """40 sessions of 63 drafts at a 262144-token vocabulary need 2560 target
    rows x 2 KiB of statistics: more than the 4 MiB array.  Refused on the
    host (no kernel runs), outputs untouched."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_diffusion_drafter_fwd_amd import DFlashError, Drafter, abi, verify_noalloc
    from tests.parity import device_tensors
    V, S = 262144, 40
    cfg = synth.config("tiny", vocab=V, block_size=64)
    w = synth.make_weights(cfg, seed=3)
    d = Drafter(cfg, device_tensors(cfg, w), max_sessions=S)
    ss = [d.session(256, seed=k, stream_id=k) for k in range(S)]
    offs = np.concatenate([[0], np.cumsum([63] * S)]).astype(np.int32)
    target = torch.empty((int(offs[-1]) + S, V), device="cuda")
    ids = torch.zeros((int(offs[-1]),), dtype=torch.int32, device="cuda")
    acc = torch.full((S,), -1, dtype=torch.int32, device="cuda")
    nxt = torch.full((S,), -1, dtype=torch.int32, device="cuda")
    with pytest.raises(DFlashError) as e:
        verify_noalloc(ss, offs, target, ids, None, 0.0, 0, acc, nxt)
    assert e.value.code == abi.E_CAPACITY
    torch.cuda.synchronize()
    assert int(acc.min()) == -1 and int(acc.max()) == -1
