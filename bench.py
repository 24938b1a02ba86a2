"""Throughput of the DFlash drafter forward on one MI355X.

Workload (default, ``--config long``): the long-context, flush-heavy bf16
drafter (hidden 4096, 5 layers, 32 q / 8 kv heads x 128, fc 20480 -> 4096,
vocab 262144, blockSize 8), seeded N(0, 0.02) weights with unit norm gains,
N(0, 1) tap features, a 131072-slot prompt written by 256-row flushes, then
drafting rounds at the fixed depth 7 with temperature-1 sampling that returns
the full per-row probability vectors.  It is the largest configuration that
fits one GPU.

A step is one round of the whole hot path: rewind the outstanding block,
commit the accepted run (anchor + a drafted rows, a ~ U{0..n}; its feature
rows ride in the next propose's context pass), propose (pending rows ->
context K/V; anchor + n mask rows through every layer; rows 1..n
unembedded) and sample the rows.  value = drafted blocks/s (for the batched
workload one block per session per batched call).  The prompt phase is timed
separately and reported as flushed context rows/s (at least 32768 rows); the
prompt is handed over 4096 rows per committed call and flushed in 256-row
chunks (the windowed laguna prompt in flush-sized calls).
All inputs (weights, feature rows, tokens, accept lengths) are resident on
the device or host before the timed region, and Python's cyclic garbage
collector is paused inside every timed region.

Other workloads (``--config``): qwen (hidden 2048, vocab 151936, 4096-slot
context, n = 15, greedy), laguna (windowed, fused QKV, gate; 32768-slot
prompt of which 511 stay), batched (64 sessions with log-uniform 1k..16k
contexts, U{1..15} rows each, T = 0.7, repetition penalty 1.1).  Feature rows
of the long, laguna and batched prompts repeat with a period of 4096 slots
(values do not change the work).  The default run also times the batched
workload after the long one and reports it under ``kernels.batched``
(``--no-secondary`` skips it).

The JSON line carries the roofline of the dominant kernel (the one with the
most time per round), timed with HIP events on its stream inside the timed
region, per-stage rooflines from the same hooks (``kernels``; ``select`` is
the DFlash2 selector on the block's drafted rows, with 8 candidates and
64-wide tables), and the CPU oracle's rate on a bounded sample of the same
workload.  On the long workload
``kernels.share_of_8`` times the attention, unembedding and sampler at one
GPU's share of an eight-GPU split (131072 / 8 context slots, 262144 / 8
vocabulary ids), the shapes each GPU would run if the session were sharded.
"""
from __future__ import annotations

import argparse
import ctypes
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")
POOL_ROWS = 4096
PROMPT_CALL_ROWS = 4096   # prompt rows per committed call (POOL_ROWS: a call never straddles the pool)
# the kernel timed live inside the timed region: the one with the most time
# per round (the attention partials of five layers on the long workload, the
# unembedding elsewhere)
DOMINANT = {"long": "attention_partial", "qwen": "unembed", "laguna": "unembed", "tiny": "unembed"}
KERNEL_NAMES = {"unembed": "k_gemm_skinny_p (lm_head)", "attention_partial": "k_attn_partial",
                "attention": "k_attn_partial + k_attn_combine"}


def gc_pause() -> None:
    """Start of a timed region: collect now, then keep Python's cyclic
    garbage collector off until the region ends (as timeit does).  A full
    collection walks every object torch created and takes tens of
    milliseconds; left on, it lands inside a timed region at random."""
    gc.collect()
    gc.disable()


def pmc_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None when there is none or
    the kernel's source changed since the counters were taken."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    pmc = json.load(open(path))
    src = os.path.join(ROOT, pmc.get("source", ""))
    if not os.path.isfile(src):
        return None
    if hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] != pmc.get("kernel_source_sha256_16"):
        return None
    return pmc.get("hbm_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed rounds (default: the workload's)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="long", choices=["qwen", "laguna", "long", "batched", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=None, help="context rows of the oracle sample")
    ap.add_argument("--cpu-rounds", type=int, default=None, help="propose + sample rounds of the oracle sample")
    ap.add_argument("--no-stages", action="store_true",
                    help="time only the dominant kernel (skip the attention, sampler, verify, select and flush stages)")
    ap.add_argument("--no-spec-loop", action="store_true", help="skip the closed speculative round")
    ap.add_argument("--no-secondary", action="store_true",
                    help="default run: skip the batched workload timed after the long one")
    ap.add_argument("--no-width-sweep", action="store_true",
                    help="skip the propose-time-vs-n sweep and the truncated-block comparison")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy first (PMC byte-counter calibration)")
    return ap.parse_args()


class Stage:
    """Events-based timing of one engine stage (dflash_profile_begin/end)."""

    def __init__(self, lib, ctx):
        self.lib, self.ctx = lib, ctx

    def begin(self, name):
        from block_diffusion_drafter_fwd_amd.abi import check
        check(self.lib, self.lib.dflash_profile_begin(self.ctx, name.encode()))

    def end(self):
        from block_diffusion_drafter_fwd_amd.abi import check
        ms, launches = ctypes.c_double(), ctypes.c_int32()
        check(self.lib, self.lib.dflash_profile_end(self.ctx, ctypes.byref(ms), ctypes.byref(launches)))
        return ms.value, launches.value


SEL_K, SEL_DS = 8, 64      # the selector stage's candidates per row and table width


def select_stage(cfg, w_dev, lg, n, temperature, anchor, torch):
    """The DFlash2 selector (dflash_select) on the block's drafted rows as
    the last round left them: a drafter of this configuration with SEL_K
    candidates per row and SEL_DS-wide selector tables (the workload's
    weights plus two seeded tables), with the dense rows verification takes
    when sampling.  Bytes: the rows' logits read once (and the dense rows
    written when sampling)."""
    from block_diffusion_drafter_fwd_amd import Drafter, select
    c2 = cfg.replace(sel_candidates=SEL_K, sel_dim=SEL_DS)
    dev = lg.device
    gen = torch.Generator(device=dev).manual_seed(5)
    w2 = dict(w_dev)
    for k in ("sel_prev", "sel_next"):
        w2[k] = (torch.randn((cfg.vocab, SEL_DS), generator=gen, device=dev) * 0.02).to(w_dev["embed"].dtype)
    d2 = Drafter(c2, w2)
    st2 = Stage(d2.lib, d2.ctx)
    s2 = d2.session(cfg.window + cfg.block_size - 1 if cfg.window else cfg.block_size + 64)
    lgc = lg.contiguous()
    dense = temperature > 0
    for r in range(3):
        select([s2], [0, n], lgc, [anchor], temperature, r, dense=dense)
    st2.begin("select")
    for r in range(20):
        select([s2], [0, n], lgc, [anchor], temperature, r, dense=dense)
    ms, launches = st2.end()
    s2.close()
    d2.close()
    avg = ms / 1e3 / max(1, launches)
    sb = n * cfg.vocab * 4 * (2 if dense else 1)
    return hbm_line(sb, avg, alg_bytes_per_launch=sb, avg_launch_us=round(avg * 1e6, 2), launches=launches,
                    candidates=SEL_K, table_dim=SEL_DS, dense=dense)


def hbm_line(alg_bytes, avg_s, **extra):
    achieved = alg_bytes / avg_s / 1e9
    d = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(achieved / HBM_PEAK_GBS, 4)}
    d.update(extra)
    return d


def mfma_line(flops, avg_s, **extra):
    achieved = flops / avg_s / 1e12
    d = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
         "frac": round(achieved / MFMA_BF16_PEAK_TFS, 4)}
    d.update(extra)
    return d


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the drafter runs on one GPU only; sharding across GPUs is described, "
                                   "not implemented", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        a.fill_(1.0)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    out = run_workload(args, args.config, torch, synth, dev)
    if args.config == "long" and not args.no_secondary:
        # the batched workload (64 sessions, config 2's shape) as a secondary
        # entry; the long run's device memory is released first
        gc.collect()
        torch.cuda.empty_cache()
        sec = run_workload(args, "batched", torch, synth, dev, secondary=True)
        out["kernels"]["batched"] = {k: sec[k] for k in ("value", "unit", "ms_per_step", "steps",
                                                          "flushed_ctx_rows_per_s", "config", "kernels")}
    print(json.dumps(out), flush=True)


def run_workload(args, name, torch, synth, dev, secondary=False):
    wl = synth.WORKLOADS[name]
    cfg = synth.config(wl.config)
    steps = args.steps if (args.steps is not None and not secondary) else min(wl.rounds, 200)
    warmup = args.warmup if not secondary else 10
    bf16 = cfg.dtype == "bf16"
    dt = torch.bfloat16 if bf16 else torch.float32
    want_cpu = not args.no_cpu_baseline and not secondary
    t0 = time.time()
    w_np = synth.make_weights(cfg, seed=0, gains="unit")
    w_dev = {}
    for k in list(w_np):
        w_dev[k] = torch.from_numpy(w_np[k]).to(dev).to(dt)
        if not want_cpu:
            del w_np[k]
    torch.cuda.synchronize()
    gen_s = time.time() - t0

    if wl.sessions > 1:
        out = bench_batched(args, cfg, wl, w_dev, steps, warmup, torch, synth)
    else:
        out = bench_single(args, cfg, wl, w_dev, steps, warmup, torch, synth)
    del w_dev
    if want_cpu:
        rows, rounds = CPU_SAMPLE.get(name, (2048, 4))
        out["cpu_baseline"] = cpu_baseline(cfg, wl, w_np, args.cpu_rows or rows, args.cpu_rounds or rounds)
    else:
        out.setdefault("cpu_baseline", None)
    del w_np
    out["setup_s"] = round(gen_s, 1)
    return out


# bounded oracle samples (context rows flushed, propose + sample rounds),
# each about 10-30 s of CPU work
CPU_SAMPLE = {"long": (2048, 3), "qwen": (4096, 4), "laguna": (2048, 6), "batched": (2048, 4), "tiny": (48, 20)}


class FeaturePool:
    """Feature rows and tokens on the device: every row of the run when it is
    small (qwen), else a POOL_ROWS-row block that positions index modulo
    POOL_ROWS (chunks never straddle its end)."""

    def __init__(self, cfg, total_rows, dev, dt, torch, synth, full):
        fs = synth.FeatureSource(cfg, 0, 0)
        self.full = full
        rows = total_rows if full else POOL_ROWS + 64
        self.feats = torch.from_numpy(fs.features(0, rows)).to(dev).to(dt)
        self.toks = fs.tokens(0, rows)

    def at(self, p, T):
        o = p if self.full else p % POOL_ROWS
        return self.toks[o:o + T], self.feats[o:o + T]


def bench_single(args, cfg, wl, w_dev, steps, warmup, torch, synth):
    import numpy as np

    from block_diffusion_drafter_fwd_amd import Drafter, sample

    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    d = Drafter(cfg, w_dev)
    st = Stage(d.lib, d.ctx)
    B = cfg.block_size
    n_rounds = warmup + steps
    extra = 64 + 80                              # rounds after the timed ones (stage passes, closed loop)
    capacity = wl.context + (n_rounds + extra) * B + 64
    if cfg.window:
        capacity = cfg.window + B - 1
    rs = synth.RoundScript(cfg, wl, 0, 0)
    total_rows = wl.context + (n_rounds + extra) * B
    pool = FeaturePool(cfg, total_rows, dev, dt, torch, synth, full=wl.name == "qwen")
    n = min(rs.max_tokens, B - 1)
    plan = [(rs.accept(n), rs.bonus()) for _ in range(n_rounds + extra)]
    current0 = rs.first_anchor()
    logits = torch.empty((B - 1, cfg.vocab), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    # ---- prompt phase: flushed context rows/s (a fresh session per pass)
    # the prompt is handed over PROMPT_CALL_ROWS rows per committed call (the
    # library flushes it in wl.commit_rows-row chunks, two chunks at a time
    # on two streams); a windowed config projects only the rows its window
    # keeps, so its prompt goes in flush-sized calls as every row is projected
    call_rows = wl.commit_rows if cfg.window else max(wl.commit_rows, PROMPT_CALL_ROWS)

    def prompt(session, rows_per_call=None):
        step_rows = rows_per_call or call_rows
        for p in range(0, wl.context, step_rows):
            T = min(step_rows, wl.context - p)
            tk, ft = pool.at(p, T)
            session.committed(tk, ft, p)
        session.flush()

    warm = d.session(capacity)
    prompt(warm)
    warm.close()
    # at least 32768 prompt rows are timed (qwen: eight 4096-row prompts into
    # fresh sessions opened beforehand), so that one pass of a short prompt
    # (~1 ms) does not make the figure; the last session runs the rounds
    passes = max(1, -(-32768 // wl.context))
    fresh = [d.session(capacity) for _ in range(passes)]
    torch.cuda.synchronize()
    gc_pause()
    t = time.perf_counter()
    for f in fresh:
        prompt(f)
    torch.cuda.synchronize()
    flush_s = time.perf_counter() - t
    gc.enable()
    flush_rows_per_s = passes * wl.context / flush_s
    s = fresh[-1]
    for f in fresh[:-1]:
        f.close()
    del fresh

    # ---- round phase
    state = {"current": current0, "r": 0}
    F_seen = []

    def step():
        r = state["r"]
        n_, lg, _ = s.propose(state["current"], rs.max_tokens, logits=logits)
        sample([s], [0, n_], lg, wl.temperature, wl.rep_penalty, wl.history, r, probs=wl.probs)
        a, bonus = plan[r]
        s.commit_block()
        F = s.state()[0]
        F_seen.append(F)
        tk, ft = pool.at(F, a + 1)
        run = np.concatenate([[state["current"]], tk[1:a + 1]]).astype(np.int32)
        s.committed(run, ft, F)
        state["current"] = bonus
        state["r"] = r + 1

    for _ in range(warmup):
        step()
    F_seen.clear()
    dom = DOMINANT[wl.name] if cfg.dtype == "bf16" else "unembed"
    st.begin(dom)
    torch.cuda.synchronize()
    gc_pause()
    t = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t
    gc.enable()
    dom_ms, dom_launches = st.end()
    blocks_per_s = steps / elapsed

    elem = 2 if cfg.dtype == "bf16" else 4
    # attention: one launch (pair) per layer; its KV bytes over the visible keys
    F_mean = float(np.mean(F_seen)) if F_seen else float(wl.context)
    vis = min(F_mean, cfg.window - 1) + n + 1 if cfg.window else F_mean + n + 1
    kv_bytes = int(2 * cfg.kv_heads * vis * cfg.head_dim * elem)
    unembed_bytes = cfg.vocab * cfg.hidden * elem + n * cfg.hidden * elem + n * cfg.vocab * 4
    alg = {"unembed": unembed_bytes, "attention": kv_bytes, "attention_partial": kv_bytes}

    def line(stage, ms_, launches_, rounds_):
        avg = ms_ / 1e3 / max(1, launches_)
        return hbm_line(alg[stage], avg, traffic=pmc_traffic(stage, wl.name), kernel=KERNEL_NAMES[stage],
                        alg_bytes_per_launch=alg[stage], avg_launch_us=round(avg * 1e6, 2), launches=launches_,
                        us_per_round=round(ms_ * 1e3 / rounds_, 1))

    roofline = line(dom, dom_ms, dom_launches, steps)
    kernels = {dom: roofline}
    stage_rounds = 16
    if not args.no_stages:
        for name in ("unembed", "attention_partial", "attention", "sampler", "layer_gemms"):
            if name in kernels or (name == "attention_partial" and cfg.dtype != "bf16"):
                continue
            st.begin(name)
            for _ in range(stage_rounds):
                step()
            ms_s, l_s = st.end()
            avg = ms_s / 1e3 / max(1, l_s)
            if name == "layer_gemms":
                # every layer's projection weights once per round (+ the block
                # rows' activations, negligible), over the summed launch time
                lb = layer_weight_bytes(cfg) + (n + 1) * cfg.hidden * elem * 4 * cfg.layers
                kernels[name] = hbm_line(lb, ms_s / 1e3 / stage_rounds, alg_bytes_per_round=lb,
                                         launches_per_round=round(l_s / stage_rounds, 1),
                                         us_per_round=round(ms_s * 1e3 / stage_rounds, 1))
            elif name == "sampler":
                sb = n * cfg.vocab * 4 * (2 if wl.probs and wl.temperature > 0 else 1)
                kernels[name] = hbm_line(sb, avg, alg_bytes_per_launch=sb, avg_launch_us=round(avg * 1e6, 2),
                                         launches=l_s)
            else:
                kernels[name] = line(name, ms_s, l_s, stage_rounds)
        per_round = {k: v.get("us_per_round", 0) for k, v in kernels.items() if k in ("unembed", "attention_partial")}
        if per_round:
            roofline["dominant_by_time_per_round"] = max(per_round, key=per_round.get)
        # verification of one block against synthetic target logits (n drafts,
        # n + 1 target rows; with the draft probabilities when sampling)
        from block_diffusion_drafter_fwd_amd import verify
        gen = torch.Generator(device=dev).manual_seed(0)
        tgt = torch.randn((n + 1, cfg.vocab), generator=gen, device=dev)
        dids = torch.randint(0, cfg.vocab, (n,), generator=gen, device=dev, dtype=torch.int32)
        T = wl.temperature
        dpr = torch.softmax(torch.randn((n, cfg.vocab), generator=gen, device=dev), dim=1) if T > 0 else None
        for r in range(3):
            verify([s], [0, n], tgt, dids, dpr, T, r)
        st.begin("verify")
        for r in range(20):
            verify([s], [0, n], tgt, dids, dpr, T, r)
        ms_v, l_v = st.end()
        if l_v:
            avg = ms_v / 1e3 / l_v
            vb = (n + 1) * cfg.vocab * 4 + (n * cfg.vocab * 4 if T > 0 else 0)
            kernels["verify"] = hbm_line(vb, avg, alg_bytes_per_launch=vb, avg_launch_us=round(avg * 1e6, 2),
                                         launches=l_v)
        if cfg.dtype == "bf16":
            kernels["select"] = select_stage(cfg, w_dev, logits[:n], n, wl.temperature, state["current"], torch)
        # the context-path GEMMs over one more prompt each (fresh sessions)
        rows = wl.commit_rows
        flops = {"flush_fc": 2.0 * rows * cfg.fc_in * cfg.hidden,
                 "flush_kv": 2.0 * rows * cfg.hidden * cfg.layers * 2 * cfg.kv_heads * cfg.head_dim}
        for name in ("flush_fc", "flush_kv"):
            s2 = d.session(capacity)
            torch.cuda.synchronize()
            st.begin(name)
            prompt(s2, wl.commit_rows)       # one chunk per call: each GEMM alone on the GPU
            torch.cuda.synchronize()
            ms_k, l_k = st.end()
            s2.close()
            if l_k:
                avg = ms_k / 1e3 / l_k
                kernels[name] = mfma_line(flops[name], avg, rows=rows, avg_launch_us=round(avg * 1e6, 2),
                                          launches=l_k, target_frac=0.5)

    if not args.no_stages and wl.name == "long":
        kernels["share_of_8"] = share_of_gpus(cfg, wl, w_dev, pool, n, torch, np, synth)
    sweep = None if args.no_width_sweep else width_sweep(s, cfg, state["current"], logits, torch, np)
    spec = None if args.no_spec_loop else spec_loop(s, cfg, wl, pool, n, state["current"], logits, torch, np)
    policy = None
    if sweep:
        v_ms = kernels["verify"]["avg_launch_us"] / 1e3 if "verify" in kernels else 0.0
        policy = width_policy_compare(sweep["fixed_ms"], sweep["per_row_ms"], v_ms, n, np)
        if spec and not args.no_spec_loop:
            pol = width_policy_object(n, sweep["fixed_ms"], sweep["per_row_ms"], v_ms, 0.0)
            spec["adaptive"] = spec_loop(s, cfg, wl, pool, n, spec_state_current(s), logits, torch, np,
                                         policy=pol)

    return {
        "metric": "drafted blocks/s + flushed ctx rows/s at 1 GPU; % HBM / MFMA peak",
        "value": round(blocks_per_s, 2),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(elapsed / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "fp32",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) tap features; no checkpoint)",
        "config": {"workload": f"{wl.name}: {wl.context}-slot context in {wl.commit_rows}-row flushes, "
                               f"then rounds at n={n}" + (f", window {cfg.window}" if cfg.window else ""),
                   "hidden": cfg.hidden, "layers": cfg.layers,
                   "heads": f"{cfg.q_heads}/{cfg.kv_heads}x{cfg.head_dim}", "vocab": cfg.vocab,
                   "block_size": B, "context": wl.context, "temperature": wl.temperature},
        "flushed_ctx_rows_per_s": round(flush_rows_per_s, 1),
        "flush_rows_timed": passes * wl.context,
        "roofline": roofline,
        "kernels": kernels,
        **({"width_sweep": sweep} if sweep else {}),
        **({"spec_round": spec} if spec else {}),
        **({"width_policy": policy} if policy else {}),
    }


def spec_state_current(s):
    """An anchor for a fresh closed loop (any token works: the loop's rounds
    commit whatever the anchor is)."""
    return 5


def width_policy_object(max_width, draft_fixed, draft_per_row, verify_fixed, verify_per_row):
    from block_diffusion_drafter_fwd_amd.drafter import WidthPolicy
    return WidthPolicy(max_width, draft_fixed, draft_per_row, verify_fixed, verify_per_row, decay=0.95)


def width_policy_compare(draft_fixed, draft_per_row, verify_ms, max_width, np, rounds=4000):
    """Fixed depth (the full width, DFlash2's seven on this configuration)
    against the adaptive width controller (dflash_width_policy_*), in expected
    emitted tokens per millisecond of round time, on a seeded acceptance
    model: draft position j is accepted with probability alpha while every
    earlier one was.  The round costs the measured draft time (fixed + per
    row, from the width sweep) plus a verification cost: the measured
    verification kernels only (the target's forward is not here), or the
    pages' GB10 fit of a Laguna target's verify round (72 ms + 3.55 ms per
    verified row), where verify time, not drafting, decides the width."""
    out = []
    for label, v_fixed, v_row in (("verification kernels only", verify_ms, 0.0),
                                  ("GB10 target verify fit: 72 ms + 3.55 ms/row", 72.0, 3.55)):
        for alpha in (0.5, 0.7, 0.9):
            rng = np.random.default_rng([int(alpha * 100), int(v_fixed)])
            res = {}
            for pol_name in ("fixed", "adaptive"):
                pol = width_policy_object(max_width, draft_fixed, draft_per_row, v_fixed, v_row)
                tokens = cost = widths = 0.0
                for _ in range(rounds):
                    w = max_width if pol_name == "fixed" else pol.choose()
                    a = 0
                    while a < w and rng.random() < alpha:
                        a += 1
                    pol.observe(w, a)
                    tokens += a + 1
                    cost += draft_fixed + draft_per_row * w + v_fixed + v_row * (w + 1)
                    widths += w
                pol.close()
                res[pol_name] = {"tokens_per_ms": round(tokens / cost, 5), "mean_width": round(widths / rounds, 2)}
            out.append({"cost_model": label, "alpha": alpha, **res,
                        "adaptive_over_fixed": round(res["adaptive"]["tokens_per_ms"] / res["fixed"]["tokens_per_ms"], 4)})
    return out


def spec_loop(s, cfg, wl, pool, n, current, logits, torch, np, rounds=64, warm=8, agree=0.7, boost=10.0,
              policy=None):
    """The closed speculative round on the GPU: propose -> sample (ids and,
    when sampling, the proposal probabilities) -> verify against a seeded
    synthetic target -> rewind and commit the anchor plus the accepted
    drafts, the correction or bonus token becoming the next anchor.  The
    target (no target model is here) is N(0, 1) noise per position with
    +boost on one preferred token: the draft's own token with probability
    `agree`, else a seeded token (the bonus row: always a seeded token); its
    noise rows are drawn on the device before timing, the preference is
    added in the round.  The one host synchronisation per round reads the
    accepted count, the next token and the drafted ids, which the commit
    needs on the host.  Reported: emitted tokens (accepted + 1) per second
    of drafting, verification and commits, the target's own forward not
    included.  With `policy` (a width controller) each round drafts the
    width it chooses and reports the round's outcome to it."""
    from block_diffusion_drafter_fwd_amd import sample, verify
    dev = logits.device
    V, T = cfg.vocab, wl.temperature
    total = warm + rounds
    gen = torch.Generator(device=dev).manual_seed(1234)
    base = torch.randn((total, n + 1, V), generator=gen, device=dev)
    rng = np.random.default_rng(1234)
    coins = torch.from_numpy(rng.uniform(size=(total, n)) < agree).to(dev)
    toks = torch.from_numpy(rng.integers(0, V - 1, size=(total, n + 1))).to(dev)
    rows = torch.arange(n, device=dev)
    s.commit_block()
    state = {"cur": current, "acc": []}

    def rnd(r):
        width = policy.choose() if policy is not None else n
        k, lg, _ = s.propose(state["cur"], width, logits=logits)
        ids, probs = sample([s], [0, k], lg, T, wl.rep_penalty, wl.history, 10_000 + r, probs=T > 0)
        tgt = base[r]
        pref = torch.where(coins[r, :k], ids.long(), toks[r, :k])
        tgt[rows[:k], pref] += boost
        tgt[k, toks[r, k]] += boost
        acc, nxt = verify([s], [0, k], tgt[:k + 1], ids, probs, T, 10_000 + r)
        out = torch.cat([acc, nxt, ids]).cpu().numpy()          # the round's one synchronisation
        a, x = int(out[0]), int(out[1])
        s.commit_block()
        F = s.state()[0]
        _, ft = pool.at(F, a + 1)
        s.committed(np.concatenate([[state["cur"]], out[2:2 + a]]).astype(np.int32), ft, F)
        state["cur"] = x
        if policy is not None:
            policy.observe(k, a)
            state.setdefault("widths", []).append(k)
        return a

    for r in range(warm):
        rnd(r)
    torch.cuda.synchronize()
    gc_pause()
    t = time.perf_counter()
    for r in range(warm, total):
        state["acc"].append(rnd(r))
    torch.cuda.synchronize()
    el = time.perf_counter() - t
    gc.enable()
    acc = state["acc"]
    extra = {"mean_width": round(float(np.mean(state["widths"][warm:])), 2)} if policy is not None else {}
    return {"rounds": rounds, "width": n if policy is None else "adaptive", **extra, "temperature": T,
            "target_agree": agree,
            "accepted_per_round": round(float(np.mean(acc)), 3),
            "emitted_tokens_per_s": round((sum(acc) + rounds) / el, 1),
            "ms_per_round": round(el / rounds * 1e3, 4),
            "note": "drafter + verification + commit per round; the target's forward is synthetic and not timed"}


def layer_weight_bytes(cfg):
    """Bytes of every layer's projection weights (q|k|v(|g), o_proj, gate|up, down)."""
    elem = 2 if cfg.dtype == "bf16" else 4
    qd, kd, H, I = cfg.q_heads * cfg.head_dim, cfg.kv_heads * cfg.head_dim, cfg.hidden, cfg.intermediate
    per = (qd + 2 * kd + (cfg.q_heads if cfg.gate else 0)) * H + H * qd + 2 * I * H + H * I
    return per * cfg.layers * elem


def share_of_gpus(cfg, wl, w_dev, pool, n, torch, np, synth, gpus=8, rounds=16):
    """The long session's kernels at one GPU's share of a split over `gpus`
    GPUs (context sharded by slot, vocabulary by id): the attention over
    context / gpus slots, the unembedding and the sampler over vocab / gpus
    ids, each timed over `rounds` rounds at the workload's width.  A drafter
    with the first vocab / gpus rows of the embedding and lm_head stands for
    one GPU's vocabulary shard; the layer weights are shared."""
    from block_diffusion_drafter_fwd_amd import Drafter, sample

    dev = torch.device("cuda:0")
    V = cfg.vocab // gpus
    ctx = wl.context // gpus
    c = cfg.replace(vocab=V)
    w = dict(w_dev)
    w["embed"] = w_dev["embed"][:V]
    w["lm_head"] = w_dev["lm_head"][:V]
    d = Drafter(c, w)
    st = Stage(d.lib, d.ctx)
    B = cfg.block_size
    stages = ("attention_partial", "attention", "unembed", "sampler")
    s = d.session(ctx + (len(stages) + 1) * rounds * B + 64)
    for p in range(0, ctx, wl.commit_rows):
        tk, ft = pool.at(p, wl.commit_rows)
        s.committed((tk % V).astype(np.int32), ft, p)
    s.flush()
    logits = torch.empty((B - 1, V), dtype=torch.float32, device=dev)
    rs = synth.RoundScript(cfg, wl, 0, 0)
    state = {"current": rs.first_anchor() % V, "r": 0, "F": []}

    def step():
        r = state["r"]
        n_, lg, _ = s.propose(state["current"], n, logits=logits)
        sample([s], [0, n_], lg, wl.temperature, wl.rep_penalty, wl.history, r, probs=wl.probs)
        a = rs.accept(n)
        s.commit_block()
        F = s.state()[0]
        state["F"].append(F)
        tk, ft = pool.at(F, a + 1)
        run = np.concatenate([[state["current"]], tk[1:a + 1] % V]).astype(np.int32)
        s.committed(run, ft, F)
        state["current"] = rs.bonus() % V
        state["r"] = r + 1

    for _ in range(rounds // 2):
        step()
    out = {"gpus": gpus, "context_slots": ctx, "vocab": V}
    for name in stages:
        state["F"].clear()
        st.begin(name)
        for _ in range(rounds):
            step()
        ms, launches = st.end()
        avg = ms / 1e3 / max(1, launches)
        vis = float(np.mean(state["F"])) + n + 1
        if name.startswith("attention"):
            b = int(2 * cfg.kv_heads * vis * cfg.head_dim * 2)
        elif name == "unembed":
            b = V * cfg.hidden * 2 + n * cfg.hidden * 2 + n * V * 4
        else:
            b = n * V * 4 * (2 if wl.probs and wl.temperature > 0 else 1)
        out[name] = hbm_line(b, avg, alg_bytes_per_launch=b, avg_launch_us=round(avg * 1e6, 2), launches=launches,
                             us_per_round=round(ms * 1e3 / rounds, 1))
    s.close()
    d.close()
    return out


def width_sweep(s, cfg, current, logits, torch, np, reps=20):
    """Propose time against the drafted width n = 1..B-1 on the session's
    current context (each propose rewound, so the context is the same for
    every n), fit as fixed + per-row by least squares; and what drafting only
    n rows instead of the full block does to rows 1..n: nothing under a causal
    block mask, a shifted proposal distribution under a bidirectional one
    (the pages note that only the causal case is exact)."""
    B = cfg.block_size
    ns = list(range(1, B))
    ms = []
    for n in ns:
        for _ in range(3):
            s.propose(current, n, logits=logits)
            s.commit_block()
        torch.cuda.synchronize()
        gc_pause()
        t = time.perf_counter()
        for _ in range(reps):
            s.propose(current, n, logits=logits)
            s.commit_block()
        torch.cuda.synchronize()
        ms.append((time.perf_counter() - t) / reps * 1e3)
        gc.enable()
    per_row, fixed = np.polyfit(np.array(ns, dtype=np.float64), np.array(ms), 1)
    _, full, _ = s.propose(current, B - 1, logits=logits)
    full = full.double().cpu().numpy()
    s.commit_block()
    trunc = {"n": [], "max_abs_logit_diff": [], "mean_kl_full_vs_truncated": []}
    for n in sorted({1, 3, (B - 1) // 2, B - 2} - {0}):
        k, part, _ = s.propose(current, n, logits=logits)
        part = part.double().cpu().numpy()
        s.commit_block()

        def logp(z):
            z = z - z.max(axis=1, keepdims=True)
            return z - np.log(np.exp(z).sum(axis=1, keepdims=True))
        lf, lt = logp(full[:k]), logp(part[:k])
        kl = float(np.mean(np.sum(np.exp(lf) * (lf - lt), axis=1)))
        trunc["n"].append(k)
        trunc["max_abs_logit_diff"].append(float(np.max(np.abs(full[:k] - part[:k]))))
        trunc["mean_kl_full_vs_truncated"].append(kl)
    return {"n": ns, "propose_ms": [round(x, 4) for x in ms], "fixed_ms": round(float(fixed), 4),
            "per_row_ms": round(float(per_row), 5), "block_mask": "causal" if cfg.causal else "bidirectional",
            "truncation": trunc}


def bench_batched(args, cfg, wl, w_dev, steps, warmup, torch, synth):
    """64 sessions, one batched propose + one batched sample per round."""
    import numpy as np

    from block_diffusion_drafter_fwd_amd import Drafter, committed_batch, flush_batch, propose_batch, sample

    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    S = wl.sessions
    B = cfg.block_size
    lens = synth.session_lengths(wl, 0)
    n_rounds = warmup + steps
    d = Drafter(cfg, w_dev, max_sessions=S)
    st = Stage(d.lib, d.ctx)
    pool = FeaturePool(cfg, POOL_ROWS, dev, dt, torch, synth, full=False)
    scripts = [synth.RoundScript(cfg, wl, 0, k) for k in range(S)]
    caps = [L + (n_rounds + 16) * B + 64 for L in lens]
    logits = torch.empty((S * (B - 1), cfg.vocab), dtype=torch.float32, device=dev)

    def prompt(sessions):
        call_rows = max(wl.commit_rows, PROMPT_CALL_ROWS)
        for k, sess in enumerate(sessions):
            for p in range(0, lens[k], call_rows):
                T = min(call_rows, lens[k] - p)
                tk, ft = pool.at(p, T)
                sess.committed(tk, ft, p)
            sess.flush()

    sess = [d.session(caps[k], seed=0, stream_id=k) for k in range(S)]
    torch.cuda.synchronize()
    gc_pause()
    t = time.perf_counter()
    prompt(sess)
    torch.cuda.synchronize()
    flush_s = time.perf_counter() - t
    gc.enable()
    flush_rows_per_s = sum(lens) / flush_s

    cur = [sc.first_anchor() for sc in scripts]
    mts = [sc.max_tokens for sc in scripts]
    state = {"r": 0, "rows": []}

    def step():
        r = state["r"]
        flushing = [sess[k] for k, sc in enumerate(scripts) if sc.flush_before]
        if flushing:   # the sessions that flush before this round's propose, in one context pass
            flush_batch(flushing)
        offs, lg = propose_batch(sess, cur, mts, logits=logits)
        sample(sess, offs, lg, wl.temperature, wl.rep_penalty, wl.history, r, probs=wl.probs)
        state["rows"].append(offs[S])
        # every session rewinds and commits its accepted run (one batched call)
        runs, fts, poss = [], [], []
        for k, sc in enumerate(scripts):
            nk = offs[k + 1] - offs[k]
            a = sc.accept(nk)
            bonus = sc.bonus()
            sess[k].commit_block()
            F = sess[k].state()[0]
            tk, ft = pool.at(F, a + 1)
            runs.append(np.concatenate([[cur[k]], tk[1:a + 1]]).astype(np.int32))
            fts.append(ft)
            poss.append(F)
            cur[k] = bonus
        committed_batch(sess, runs, fts, poss)
        state["r"] = r + 1

    for _ in range(warmup):
        step()
    state["rows"].clear()
    st.begin("attention_partial")
    torch.cuda.synchronize()
    gc_pause()
    t = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t
    gc.enable()
    ms_a, l_a = st.end()
    blocks_per_s = steps * S / elapsed
    R = float(np.mean(state["rows"]))
    elem = 2
    ctx_now = [sess[k].state()[0] for k in range(S)]
    kv_bytes_layer = sum(2 * cfg.kv_heads * (c + B) * cfg.head_dim * elem for c in ctx_now)
    avg_a = ms_a / 1e3 / max(1, l_a)
    attn = hbm_line(kv_bytes_layer, avg_a, traffic=pmc_traffic("attention_partial", wl.name),
                    kernel="k_attn_partial (all sessions, one layer)", alg_bytes_per_launch=int(kv_bytes_layer),
                    avg_launch_us=round(avg_a * 1e6, 2), launches=l_a, us_per_round=round(ms_a * 1e3 / steps, 1))
    kernels = {"attention_partial": attn}
    for name in ("attention", "unembed", "sampler", "layer_gemms"):
        st.begin(name)
        for _ in range(4):
            step()
        ms_s, l_s = st.end()
        avg = ms_s / 1e3 / max(1, l_s)
        if name == "layer_gemms":
            # ~487 block rows: the projections are dense contractions
            fl = 2.0 * R * layer_weight_bytes(cfg) / elem
            kernels[name] = mfma_line(fl, ms_s / 1e3 / 4, rows=round(R, 1), launches_per_round=round(l_s / 4, 1),
                                      us_per_round=round(ms_s * 1e3 / 4, 1), target_frac=0.5)
        elif name == "unembed":
            kernels[name] = mfma_line(2.0 * R * cfg.hidden * cfg.vocab, avg, rows=round(R, 1),
                                      avg_launch_us=round(avg * 1e6, 2), launches=l_s, target_frac=0.5)
        elif name == "attention":
            kernels[name] = hbm_line(kv_bytes_layer, avg, kernel="k_attn_partial + k_attn_combine",
                                     alg_bytes_per_launch=int(kv_bytes_layer), avg_launch_us=round(avg * 1e6, 2),
                                     launches=l_s)
        else:
            sb = R * cfg.vocab * 4
            kernels[name] = hbm_line(sb, avg, alg_bytes_per_launch=int(sb), avg_launch_us=round(avg * 1e6, 2),
                                     launches=l_s)
    for x in sess:
        x.close()
    return {
        "metric": "drafted blocks/s + flushed ctx rows/s at 1 GPU; % HBM / MFMA peak",
        "value": round(blocks_per_s, 2),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(elapsed / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) tap features repeating every 4096 slots)",
        "config": {"workload": f"batched: {S} sessions, contexts log-uniform {wl.context_lo}..{wl.context_hi} "
                               f"(sum {sum(lens)}), U{{1..{B - 1}}} rows each, T={wl.temperature}, "
                               f"penalty {wl.rep_penalty}",
                   "hidden": cfg.hidden, "layers": cfg.layers, "vocab": cfg.vocab, "block_size": B,
                   "sessions": S, "rows_per_round": round(R, 1)},
        "flushed_ctx_rows_per_s": round(flush_rows_per_s, 1),
        "roofline": attn,
        "kernels": kernels,
    }


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, wl, w_np, rows, rounds):
    """The float64 oracle on a bounded sample of the same workload: `rows`
    context rows flushed in 256-row chunks, then `rounds` rounds of propose +
    sample over that context at the workload's width, temperature and
    penalty.  Reported per unit (blocks/s; flushed rows/s).  Its flush rate
    does not depend on the context length (rows are independent); its round
    rate over a context shorter than the workload's is an upper bound."""
    import numpy as np

    import synth
    from oracle.model import DraftModel
    from oracle.sampler import sample_row
    from oracle.session import OracleSession
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        cores = len(os.sched_getaffinity(0))
    fs = synth.FeatureSource(cfg, 0, 0)
    o = OracleSession(DraftModel(cfg, w_np))
    n = cfg.block_size - 1 if wl.max_tokens <= 0 else min(wl.max_tokens, cfg.block_size - 1)
    t = time.perf_counter()
    for p in range(0, rows, wl.commit_rows):
        T = min(wl.commit_rows, rows - p)
        o.committed(fs.tokens(p, T), fs.features(p, T), p)
    o.flush()
    t_flush = time.perf_counter() - t
    t = time.perf_counter()
    cur = 5
    for r in range(rounds):
        out = o.propose(cur, n)
        for i in range(out["n"]):
            sample_row(out["logits"][i], o.history[-wl.history:], wl.temperature, wl.rep_penalty, 0, 0, r, i)
        o.commit_block()
        F = o.ctx_offset
        o.committed(np.array([cur, 1, 2], dtype=np.int32), fs.features(F, 3), F)
        cur = 7
    t_rounds = time.perf_counter() - t
    return {"value": round(rounds / t_rounds, 4), "unit": "blocks/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model(), "flushed_ctx_rows_per_s": round(rows / t_flush, 2),
            "sample": f"float64 NumPy oracle (BLAS threads = cores) on the same configuration: {rows} context "
                      f"rows flushed in {wl.commit_rows}-row chunks ({t_flush:.1f} s), then {rounds} rounds of "
                      f"propose (n={n}) + sample (T={wl.temperature}, penalty {wl.rep_penalty}) over a "
                      f"{rows}-slot context ({t_rounds:.1f} s); the workload's context is {wl.context or 'per session'}"
                      f" slots, so the round rate is an upper bound of the oracle's there"}


if __name__ == "__main__":
    main()
