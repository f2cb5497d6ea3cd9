"""Pins of the oracle's whole decoder.

* A layer whose output projections are zero is the identity on the residual.
* The KV-cached incremental path equals the cache-free full recompute.
* The whole tiny decoder equals an independent fp64 formulation written with
  torch library routines (matmul, softmax) on the CPU, within fp32 error.
"""
import math

import numpy as np
import pytest
import torch

import synth

TINY = synth.CONFIGS["tiny_2l_d256"]


@pytest.fixture(scope="module")
def tiny_weights():
    return synth.model_weights(TINY)


def test_layer_with_zero_outputs_is_identity(orc, tiny_weights):
    w = {k: v for k, v in tiny_weights.items()}
    w["layers"] = [dict(l) for l in tiny_weights["layers"]]
    w["layers"][0]["wo"] = np.zeros_like(w["layers"][0]["wo"])
    w["layers"][0]["w_down"] = np.zeros_like(w["layers"][0]["w_down"])
    m = orc.Model(TINY, w)
    x = synth.hidden(TINY)
    for pos in (0, 3):
        y = m.layer_forward(0, x, pos)
        assert np.array_equal(y, x)


def test_layer_writes_rope_key_and_value_at_pos(orc, tiny_weights):
    """The cache row written at pos is fp16 of (rope(Wk h), Wv h) with h the normed input."""
    m = orc.Model(TINY, tiny_weights)
    lw = tiny_weights["layers"][1]
    x = synth.hidden(TINY)
    pos = 11
    m.layer_forward(1, x, pos)
    h = orc.rmsnorm(x, lw["attn_norm"], TINY["rms_eps"])
    k = orc.gemv(lw["wk"], h).reshape(TINY["n_kv_heads"], TINY["head_dim"])
    v = orc.gemv(lw["wv"], h).reshape(TINY["n_kv_heads"], TINY["head_dim"])
    k = np.stack([orc.rope(r, pos) for r in k])
    assert np.array_equal(m.kcache[1, pos], k.astype(np.float16))
    assert np.array_equal(m.vcache[1, pos], v.astype(np.float16))
    assert not m.kcache[1, pos + 1].any() and not m.kcache[0].any()


def test_cached_decode_equals_nocache_recompute(orc, tiny_weights):
    m = orc.Model(TINY, tiny_weights)
    toks = synth.prompt(TINY, 12)
    for pos, t in enumerate(toks):
        got = m.decode_step(int(t), pos)
        if pos in (0, 1, 6, 11):
            ref = m.forward_nocache(toks[: pos + 1])
            assert np.allclose(got, ref, rtol=0, atol=1e-6 * np.abs(ref).max()), pos


def _torch_fp64_logits(cfg, w, tokens):
    """Independent fp64 formulation: whole-prefix causal forward with library ops.
    Keys/values are rounded to fp16 like the cache; everything else is fp64."""
    T = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    d, hq, hkv, dh = cfg["d_model"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    n = len(tokens)
    eps = cfg["rms_eps"]
    x = T(w["tok_emb"].astype(np.float64))[torch.as_tensor(tokens, dtype=torch.long)]
    half = dh // 2
    inv = torch.tensor([cfg["rope_base"] ** (-2.0 * i / dh) for i in range(half)], dtype=torch.float64)
    ang = torch.arange(n, dtype=torch.float64)[:, None] * inv[None, :]
    cos, sin = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]

    def rope(t):
        a, b = t[..., :half], t[..., half:]
        return torch.cat([a * cos - b * sin, b * cos + a * sin], dim=-1)

    def rms(v, g):
        return T(g.astype(np.float64)) * v / torch.sqrt((v * v).mean(-1, keepdim=True) + eps)

    mask = torch.triu(torch.full((n, n), float("-inf"), dtype=torch.float64), diagonal=1)
    for lw in w["layers"]:
        h = rms(x, lw["attn_norm"])
        q = rope((h @ T(lw["wq"]).T).reshape(n, hq, dh))
        k = rope((h @ T(lw["wk"]).T).reshape(n, hkv, dh)).to(torch.float16).to(torch.float64)
        v = (h @ T(lw["wv"]).T).reshape(n, hkv, dh).to(torch.float16).to(torch.float64)
        k = k.repeat_interleave(hq // hkv, dim=1)
        v = v.repeat_interleave(hq // hkv, dim=1)
        s = torch.matmul(q.permute(1, 0, 2), k.permute(1, 2, 0).contiguous()) / math.sqrt(dh)
        a = torch.softmax(s + mask, dim=-1)
        o = torch.matmul(a, v.permute(1, 0, 2).contiguous()).permute(1, 0, 2).reshape(n, hq * dh)
        x = x + o @ T(lw["wo"]).T
        h = rms(x, lw["ffn_norm"])
        g = h @ T(lw["w_gate"]).T
        x = x + ((g * torch.sigmoid(g)) * (h @ T(lw["w_up"]).T)) @ T(lw["w_down"]).T
    return (rms(x[-1], w["final_norm"]) @ T(w["lm_head"]).T).numpy()


def test_oracle_matches_independent_fp64_formulation(orc, tiny_weights):
    m = orc.Model(TINY, tiny_weights)
    toks = synth.prompt(TINY, 10)
    for pos, t in enumerate(toks):
        got = m.decode_step(int(t), pos).astype(np.float64)
    ref = _torch_fp64_logits(TINY, tiny_weights, toks)
    err = np.abs(got - ref).max()
    assert err <= 2e-4 * np.abs(ref).max(), err
    assert int(np.argmax(ref)) == orc.argmax(got.astype(np.float32))


def test_gqa_oracle_matches_fp64_formulation(orc):
    cfg = synth.scaled_config("tiny_2l_d256", n_heads=8, n_kv_heads=2, head_dim=32, vocab=512)
    w = synth.model_weights(cfg, seed=5)
    m = orc.Model(cfg, w)
    toks = synth.prompt(cfg, 7)
    for pos, t in enumerate(toks):
        got = m.decode_step(int(t), pos).astype(np.float64)
    ref = _torch_fp64_logits(cfg, w, toks)
    assert np.abs(got - ref).max() <= 2e-4 * np.abs(ref).max()


def test_logit_scale_under_unit_gains(orc, tiny_weights):
    """With unit RMSNorm gains and N(0, 0.02) weights the logits are about N(0, 1)
    (std 0.02 * sqrt(d)), which keeps near-ties rare in the greedy checks."""
    m = orc.Model(TINY, tiny_weights)
    logits = m.decode_step(5, 0)
    sd = float(np.std(logits))
    assert 0.02 * math.sqrt(TINY["d_model"]) * 0.5 < sd < 0.02 * math.sqrt(TINY["d_model"]) * 2


def test_generate_equals_stepwise_greedy(orc, tiny_weights):
    m1 = orc.Model(TINY, tiny_weights)
    m2 = orc.Model(TINY, tiny_weights)
    out = m1.generate(17, 0, 6)
    tok = 17
    for i in range(6):
        tok = orc.argmax(m2.decode_step(tok, i))
        assert tok == out[i]


def test_decode_rejects_bad_arguments(orc, tiny_weights):
    m = orc.Model(TINY, tiny_weights)
    with pytest.raises(ValueError):
        m.decode_step(TINY["vocab"], 0)
    with pytest.raises(ValueError):
        m.decode_step(0, TINY["max_seq"])
    with pytest.raises(ValueError):
        m.decode_step(-1, 0)


def test_sliding_window_cached_equals_nocache_and_matters(orc, tiny_weights):
    """Window 4 on layer 0 only: the cached decode equals the no-cache recompute
    (two separate code paths) past the window, and differs from full attention."""
    cfg = dict(TINY, sliding_window=4, window_layers=0b01)
    m, full = orc.Model(cfg, tiny_weights), orc.Model(TINY, tiny_weights)
    toks = synth.prompt(TINY, 10)
    for pos, t in enumerate(toks):
        got, ref_full = m.decode_step(int(t), pos), full.decode_step(int(t), pos)
        if pos in (2, 3, 4, 9):
            ref = m.forward_nocache(toks[: pos + 1])
            assert np.allclose(got, ref, rtol=0, atol=1e-6 * np.abs(ref).max()), pos
        if pos < 4:
            assert np.array_equal(got, ref_full), pos
    assert not np.allclose(got, ref_full, rtol=0, atol=1e-4)
