"""Pins of the oracle's Laguna arm (CPU only).

The mlxcel PR "feat(speculative): add the Laguna DFlash drafter" (PR body and
the vLLM-deviation paragraph) fixes the Laguna drafter's extra steps by name:
``aux_hidden_norms`` on the concatenated target taps before ``fc``, every
layer's own ``input_layernorm`` on the context rows before their K/V
projection, fused ``qkv_proj`` attention with a per-head sigmoid gate
(``g_proj``), and a per-query sliding window over [context | block].  No
library ships this variant, so it is pinned here against a forward assembled
by hand from independent parts:

* transformers' ``Qwen3Attention`` / ``Qwen3DecoderLayer`` / ``Qwen3RMSNorm``
  for the attention, q/k norms, RoPE, MLP and residuals (their dense form is
  already pinned against the oracle in ``test_oracle_model.py``);
* ``torch.nn.functional.rms_norm`` applied to each tap slice with that tap's
  own gain row (aux norms);
* each layer's ``input_layernorm`` module fed the context before that layer's
  attention fills the K/V cache (context input norm);
* a pre-hook on ``o_proj`` that multiplies q head h's slice of the attention
  output by sigmoid(x . g_proj[h]), x being the normed layer input the
  attention module received (gate);
* an explicit additive mask with p - s >= W hidden (window).

Every pin is shown to discriminate: the ``test_planted_*`` tests plant one
plausible mistake in the oracle (monkeypatched, CPU only) and require the
comparison against the assembled forward to fail.  The planted mistakes are:
norming the whole taps*Ht row instead of each tap; one gain row for every
tap; gating head h with head h+1's scalar; computing the gate from the input
before ``input_layernorm``'s gain; using ``post_attention_layernorm``'s gain,
or layer 0's gain, for the context input norm.
"""
import re

import numpy as np
import pytest
import torch

import synth
import oracle.model as om
from oracle.model import DraftModel
from oracle.session import OracleSession
from tests.helpers import rel_err


@pytest.fixture(autouse=True)
def _fp64_default():
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(old)


def _cfg(**kw):
    base = dict(name="lag", dtype="fp32", hidden=64, layers=2, q_heads=4, kv_heads=2, head_dim=16,
                taps=5, target_hidden=32, vocab=48, block_size=6, intermediate=96, causal=False,
                flush_rows=8, window=9, gate=True, aux_norms=True, ctx_input_norm=True,
                fused_qkv=True)
    base.update(kw)
    return synth.DraftConfig(**base)


def _T(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def _assembled_forward(cfg, w, feats, F, tokens):
    """Laguna drafter forward from transformers' Qwen3 modules plus the
    variant's steps written in torch; returns per-layer context K/V
    ([F, Hkv, D]), the block's last hidden state and logits of rows 1..n."""
    from transformers import DynamicCache
    from transformers.models.qwen3 import modeling_qwen3 as q3
    from transformers.models.qwen3.configuration_qwen3 import Qwen3Config

    D, Hq, Hkv = cfg.head_dim, cfg.q_heads, cfg.kv_heads
    qd, kd = Hq * D, Hkv * D
    hc = Qwen3Config(vocab_size=cfg.vocab, hidden_size=cfg.hidden,
                     intermediate_size=cfg.intermediate, num_hidden_layers=cfg.layers,
                     num_attention_heads=Hq, num_key_value_heads=Hkv, head_dim=D,
                     rms_norm_eps=cfg.rms_eps, attention_bias=False,
                     rope_parameters={"rope_type": "default", "rope_theta": cfg.rope_theta},
                     max_position_embeddings=4096)
    hc._attn_implementation = "eager"
    layers, in_norms = [], []
    captured = {}
    for l in range(cfg.layers):
        layer = q3.Qwen3DecoderLayer(hc, layer_idx=l).double().eval()
        p = f"layers.{l}."
        qkv = w[p + "qkv_proj"]
        sd = {"input_layernorm.weight": w[p + "input_layernorm"],
              "post_attention_layernorm.weight": w[p + "post_attention_layernorm"],
              "self_attn.q_proj.weight": qkv[:qd], "self_attn.k_proj.weight": qkv[qd:qd + kd],
              "self_attn.v_proj.weight": qkv[qd + kd:], "self_attn.o_proj.weight": w[p + "o_proj"],
              "self_attn.q_norm.weight": w[p + "q_norm"], "self_attn.k_norm.weight": w[p + "k_norm"],
              "mlp.gate_proj.weight": w[p + "gate_proj"], "mlp.up_proj.weight": w[p + "up_proj"],
              "mlp.down_proj.weight": w[p + "down_proj"]}
        layer.load_state_dict({k: _T(v) for k, v in sd.items()})
        g = _T(w[p + "g_proj"])

        def take_x(mod, args, kwargs, l=l):
            captured[l] = kwargs["hidden_states"]

        def gate_o(mod, args, l=l, g=g):
            a = args[0]
            s = torch.sigmoid(captured[l] @ g.T)                       # [1, M, Hq]
            return (a.view(*a.shape[:-1], Hq, D) * s[..., None]).view(a.shape),

        layer.self_attn.register_forward_pre_hook(take_x, with_kwargs=True)
        layer.self_attn.o_proj.register_forward_pre_hook(gate_o)
        layers.append(layer)
        nm = q3.Qwen3RMSNorm(cfg.hidden, eps=cfg.rms_eps).double()
        nm.weight.data = _T(w[p + "input_layernorm"])
        in_norms.append(nm)

    def pe(positions):
        inv = 1.0 / (cfg.rope_theta ** (torch.arange(0, D, 2) / D))
        fr = torch.tensor(positions).double()[:, None] * inv[None, :]
        emb = torch.cat([fr, fr], -1)
        return emb.cos()[None], emb.sin()[None]

    hn = q3.Qwen3RMSNorm(cfg.hidden, eps=cfg.rms_eps).double()
    hn.weight.data = _T(w["hidden_norm"])
    fn = q3.Qwen3RMSNorm(cfg.hidden, eps=cfg.rms_eps).double()
    fn.weight.data = _T(w["norm"])
    aux = _T(w["aux_norms"])
    with torch.no_grad():
        f = _T(feats).view(F, cfg.taps, cfg.target_hidden)
        f = torch.stack([torch.nn.functional.rms_norm(f[:, t], (cfg.target_hidden,), weight=aux[t],
                                                      eps=cfg.rms_eps) for t in range(cfg.taps)], 1)
        c = hn(f.reshape(F, cfg.fc_in) @ _T(w["fc"]).T)[None]          # [1, F, H]
        cache = DynamicCache(config=hc)
        for l, layer in enumerate(layers):
            x = in_norms[l](c)
            captured[l] = x
            layer.self_attn(hidden_states=x, position_embeddings=pe(list(range(F))),
                            attention_mask=None, past_key_values=cache)
        ck = [cache.layers[l].keys[0].transpose(0, 1).numpy().copy() for l in range(cfg.layers)]
        cv = [cache.layers[l].values[0].transpose(0, 1).numpy().copy() for l in range(cfg.layers)]
        M = len(tokens)
        mask = torch.zeros(1, 1, M, F + M)
        for i in range(M):
            p = F + i
            for s in range(F + M):
                if (cfg.window and p - s >= cfg.window) or (cfg.causal and s > p):
                    mask[0, 0, i, s] = float("-inf")
        h = _T(w["embed"][np.asarray(tokens)])[None]
        for layer in layers:
            h = layer(h, attention_mask=mask, position_embeddings=pe(list(range(F, F + M))),
                      past_key_values=cache)
            if isinstance(h, tuple):
                h = h[0]
        z = fn(h[0, 1:]) @ _T(w["lm_head"]).T
    return ck, cv, h[0].numpy(), z.numpy()


def _oracle_run(cfg, w, F, anchor=5, seed=0):
    """Oracle session: F context rows committed and flushed, then a full-width
    propose.  Returns the session, the propose result and the features."""
    fs = synth.FeatureSource(cfg, seed)
    s = OracleSession(DraftModel(cfg, w))
    s.committed(fs.tokens(0, F), fs.features(0, F), 0)
    s.flush()
    out = s.propose(anchor, cfg.block_size - 1)
    return s, out, fs.features(0, F)


def _errors(cfg, w, F=14, seed=0):
    """Largest relative error of the oracle against the assembled forward
    over the visible context K/V, the block hidden state and the logits."""
    s, out, feats = _oracle_run(cfg, w, F, seed=seed)
    tokens = [5] + [cfg.mask_id] * out["n"]
    ck, cv, hh, z = _assembled_forward(cfg, w, feats, F, tokens)
    lo = max(0, F - (cfg.window - 1)) if cfg.window else 0
    errs = {}
    for l in range(cfg.layers):
        K, V = s.cache_kv(l, np.arange(lo, F))
        errs[f"k{l}"] = rel_err(K, ck[l][lo:])
        errs[f"v{l}"] = rel_err(V, cv[l][lo:])
    errs["hidden"] = rel_err(out["hidden"], hh)
    errs["logits"] = rel_err(out["logits"], z)
    return errs


# --------------------------------------------------------------------------
# the pins
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_laguna_forward_matches_assembled_forward(causal):
    """Aux norms, context input norm, fused qkv, gate and window together:
    cache K/V of every visible slot, hidden state and logits within 1e-6
    (transformers' RMSNorm modules take the variance in float32)."""
    cfg = _cfg(causal=causal)
    w = synth.make_weights(cfg, seed=21, gains="random")
    errs = _errors(cfg, w)
    assert max(errs.values()) < 1e-6, errs


def test_laguna_forward_with_no_window_drop():
    """Context shorter than the window: nothing dropped, every slot visible."""
    cfg = _cfg(window=64)
    w = synth.make_weights(cfg, seed=22, gains="random")
    errs = _errors(cfg, w, F=11)
    assert max(errs.values()) < 1e-6, errs


def test_swapping_aux_gain_rows_changes_context():
    """Each tap has its own gain row: exchanging two rows changes K/V."""
    cfg = _cfg()
    w = synth.make_weights(cfg, seed=23, gains="random")
    m = DraftModel(cfg, w)
    f = synth.FeatureSource(cfg, 23).features(0, 6)
    a = m.context_kv(f, np.arange(6))
    w2 = dict(w)
    w2["aux_norms"] = w["aux_norms"][[1, 0, 2, 3, 4]]
    b = DraftModel(cfg, w2).context_kv(f, np.arange(6))
    assert rel_err(b[0][0], a[0][0]) > 1e-3


def test_aux_norms_scale_invariance_per_tap():
    """Per-tap RMSNorm makes the context independent of each tap's scale:
    multiplying one tap's slice by 7 leaves K/V unchanged (a whole-row norm
    would not)."""
    cfg = _cfg()
    w = synth.make_weights(cfg, seed=24, gains="random")
    m = DraftModel(cfg, w)
    f = synth.FeatureSource(cfg, 24).features(0, 6).astype(np.float64)
    g = f.copy()
    g[:, 2 * cfg.target_hidden:3 * cfg.target_hidden] *= 7.0
    a = m.context_kv(f, np.arange(6))
    b = m.context_kv(g, np.arange(6))
    for (K, V), (K2, V2) in zip(a, b):
        assert rel_err(K2, K) < 1e-6 and rel_err(V2, V) < 1e-6


def test_gate_closed_form_one_head_off():
    """sigmoid -> 0 on q head h and -> 1 on the others equals the ungated model
    with o_proj's columns of head h zeroed.

    A large constant on embedding coordinate 0 makes that coordinate dominate
    every layer's normed input x (x_0 ~ +sqrt(H)), so g_proj rows
    -1e4 * e_0 and +1e4 * e_0 drive the gate to exactly 0 and 1."""
    cfgg = _cfg(window=0)
    cfgn = _cfg(window=0, gate=False)
    w = synth.make_weights(cfgg, seed=25, gains="random")
    w["embed"] = w["embed"].copy()
    w["embed"][:, 0] = 10.0
    off = 2
    D = cfgg.head_dim
    for l in range(cfgg.layers):
        gp = np.zeros_like(w[f"layers.{l}.g_proj"])
        gp[:, 0] = 1e4
        gp[off, 0] = -1e4
        w[f"layers.{l}.g_proj"] = gp
    wn = {k: v for k, v in w.items() if "g_proj" not in k}
    for l in range(cfgg.layers):
        o = w[f"layers.{l}.o_proj"].copy()
        o[:, off * D:(off + 1) * D] = 0.0
        wn[f"layers.{l}.o_proj"] = o
    with np.errstate(over="ignore"):
        _, a, _ = _oracle_run(cfgg, w, 9)
    _, b, _ = _oracle_run(cfgn, wn, 9)
    np.testing.assert_allclose(a["logits"], b["logits"], rtol=1e-12, atol=1e-12)
    _, c, _ = _oracle_run(cfgn, {k: v for k, v in w.items() if "g_proj" not in k}, 9)
    assert not np.allclose(a["logits"], c["logits"], rtol=1e-6)


def test_context_input_norm_uses_each_layers_own_gain():
    """Context K/V of layer l change when layer l's input_layernorm gain
    changes and stay put when another layer's or the post-attention gain
    changes."""
    cfg = _cfg()
    w = synth.make_weights(cfg, seed=26, gains="random")
    f = synth.FeatureSource(cfg, 26).features(0, 6)
    base = DraftModel(cfg, w).context_kv(f, np.arange(6))
    w1 = dict(w)
    w1["layers.1.input_layernorm"] = w["layers.1.input_layernorm"][::-1].copy()
    a = DraftModel(cfg, w1).context_kv(f, np.arange(6))
    np.testing.assert_array_equal(a[0][0], base[0][0])
    assert rel_err(a[1][0], base[1][0]) > 1e-3
    w2 = dict(w)
    w2["layers.0.post_attention_layernorm"] = w["layers.0.post_attention_layernorm"] * 3.0
    b = DraftModel(cfg, w2).context_kv(f, np.arange(6))
    np.testing.assert_array_equal(b[0][0], base[0][0])


# --------------------------------------------------------------------------
# planted mistakes: each must make the pin fail
# --------------------------------------------------------------------------

def _fails(monkeypatch_fn, monkeypatch, seed):
    cfg = _cfg()
    w = synth.make_weights(cfg, seed=seed, gains="random")
    assert max(_errors(cfg, w).values()) < 1e-6
    monkeypatch_fn(monkeypatch)
    errs = _errors(cfg, w)
    return max(errs.values())


def test_planted_whole_row_aux_norm_is_caught(monkeypatch):
    orig = om.rms_norm

    def plant(mp):
        def whole_row(x, gain, eps):
            x = np.asarray(x)
            gain = np.asarray(gain)
            if x.ndim == 3 and gain.ndim == 2:
                P = x.shape[0]
                return orig(x.reshape(P, -1), gain.reshape(-1), eps).reshape(x.shape)
            return orig(x, gain, eps)
        mp.setattr(om, "rms_norm", whole_row)

    assert _fails(plant, monkeypatch, 31) > 1e-3


def test_planted_single_aux_gain_row_is_caught(monkeypatch):
    orig = om.rms_norm

    def plant(mp):
        def one_row(x, gain, eps):
            gain = np.asarray(gain)
            if gain.ndim == 2:
                gain = np.broadcast_to(gain[0], gain.shape)
            return orig(x, gain, eps)
        mp.setattr(om, "rms_norm", one_row)

    assert _fails(plant, monkeypatch, 32) > 1e-3


def test_planted_gate_on_wrong_head_is_caught(monkeypatch):
    orig = om.sigmoid

    def plant(mp):
        mp.setattr(om, "sigmoid", lambda z: np.roll(orig(z), 1, axis=-1))

    assert _fails(plant, monkeypatch, 33) > 1e-3


def test_planted_gate_from_ungained_input_is_caught(monkeypatch):
    orig = DraftModel.lin

    def plant(mp):
        def lin(self, x, name, row0=0, rows=None):
            m = re.match(r"layers\.(\d+)\.g_proj$", name)
            if m:
                x = x / self.g(f"layers.{m.group(1)}.input_layernorm")
            return orig(self, x, name, row0, rows)
        mp.setattr(DraftModel, "lin", lin)

    assert _fails(plant, monkeypatch, 34) > 1e-3


@pytest.mark.parametrize("wrong", ["post_attention", "layer0"])
def test_planted_context_input_norm_gain_is_caught(monkeypatch, wrong):
    orig_ctx = DraftModel.context_kv

    def plant(mp):
        def ctx(self, feats, positions):
            orig_g = DraftModel.g

            def g(name):
                if wrong == "post_attention":
                    name = name.replace("input_layernorm", "post_attention_layernorm")
                else:
                    name = re.sub(r"layers\.\d+\.input_layernorm", "layers.0.input_layernorm", name)
                return orig_g(self, name)
            self.g = g
            try:
                return orig_ctx(self, feats, positions)
            finally:
                del self.g
        mp.setattr(DraftModel, "context_kv", ctx)

    assert _fails(plant, monkeypatch, 35) > 1e-3
