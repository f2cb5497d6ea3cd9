"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Tolerance (floating point): per step, max_v |logit_gpu - logit_oracle| <=
1e-2 * max_v |logit_oracle| + 1e-3; the same form on the residual vector of the
single-layer workload.  Greedy tokens must agree wherever the oracle's top-2
margin is at least 1e-2.  Integer work (the defined exponential's bits, the
sampler's token given the same logits and counters) must be bit-exact.
"""
import os

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the -m gpu tests must run on an MI355X")


@pytest.fixture(scope="module")
def lf():
    _need_gpu()
    from persistent_runtime_amd import lf as mod
    mod.lib()
    return mod


def close(gpu, ref, rel=1e-2, atol=1e-3):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref).max()
    return err <= rel * np.abs(ref).max() + atol, err


def margin(logits):
    top = np.sort(np.asarray(logits, np.float64))[-2:]
    return top[1] - top[0]


def replay_generate(eng, m, tok0, pos0, n, kc, vc):
    """One generate launch of n steps from pos0, replayed through the oracle
    (restarted from the cache snapshot kc / vc): each kernel token must be an
    argmax of the oracle's logits within twice the logit tolerance (the unique
    argmax where the top-2 margin is at least 1e-2), and the launch's last
    logits must match the oracle's."""
    eng.set_position(tok0, pos0)
    got = eng.generate(n)
    last = eng.logits().cpu().numpy()
    m.kcache[...] = kc
    m.vcache[...] = vc
    tok = tok0
    for i in range(n):
        ref = m.decode_step(tok, pos0 + i)
        tol = 1e-2 * np.abs(ref).max() + 1e-3
        assert ref[int(got[i])] >= ref.max() - 2 * tol, i
        if margin(ref) >= 1e-2:
            assert int(got[i]) == int(np.argmax(ref)), i
        tok = int(got[i])
    ok, err = close(last, ref)
    assert ok, err


def teacher_forced(lf, orc, cfg, weights, tokens, pos0=0, engine=None, model=None):
    """Feed the same tokens to both sides; check logits and greedy choice each step."""
    eng = engine or lf.Engine(cfg, lf.upload_weights(weights))
    m = model or orc.Model(cfg, weights)
    worst = 0.0
    for i, t in enumerate(tokens):
        pos = pos0 + i
        nxt = eng.decode_step(int(t), pos)
        ref = m.decode_step(int(t), pos)
        got = eng.logits().cpu().numpy()
        ok, err = close(got, ref)
        worst = max(worst, err / (np.abs(ref).max() + 1e-30))
        assert ok, (pos, err, np.abs(ref).max())
        if margin(ref) >= 1e-2:
            assert nxt == orc.argmax(ref), pos
            assert nxt == int(np.argmax(got)), pos
    return eng, m, worst


# ---------------------------------------------------------------- sampler pieces

def test_expdef_bit_exact_against_oracle(lf, orc):
    import torch
    # every 37th binary32 in [-23, 0] plus edges: ~29M values
    hi = np.float32(-23.0).view(np.uint32)
    bits = np.arange(0x80000000, hi + 1, 37, dtype=np.uint64).astype(np.uint32)
    x = np.concatenate([bits.view(np.float32), np.float32([0.0, -0.0, -23.0, -1e-38, -0.5, -0.34657359])])
    y_gpu = lf.test_expdef(torch.from_numpy(x).cuda()).cpu().numpy()
    y_cpu = orc.expdef(x)
    assert np.array_equal(y_gpu.view(np.uint32), y_cpu.view(np.uint32))


@pytest.mark.parametrize("V,scale,top_p,T", [(32768, 1.0, 0.9, 0.8), (32768, 4.0, 0.9, 0.8),
                                             (4096, 0.2, 0.5, 1.0), (128256, 1.0, 0.9, 0.8),
                                             (16, 3.0, 0.9, 0.8), (2, 1.0, 0.9, 0.8),
                                             (4096, 1.0, 1.0, 1.0), (4096, 1.0, 1e-6, 0.8)])
def test_sampler_bit_exact_against_oracle(lf, orc, V, scale, top_p, T):
    import torch
    rng = np.random.default_rng(V + int(scale * 10))
    m = 24
    logits = (rng.standard_normal((m, V)) * scale).astype(np.float32)
    logits[1] = np.round(logits[1])                  # many exact ties
    logits[2] = 0.0                                   # all equal
    logits[3, :] = -40.0
    logits[3, V // 2] = 0.0                           # one token carries all mass
    pos = np.arange(16384, 16384 + m, dtype=np.int32)
    tok = lf.test_sample(torch.from_numpy(logits).cuda(), T, top_p, 1234,
                         torch.from_numpy(pos).cuda()).cpu().numpy()
    for c in range(m):
        assert tok[c] == orc.sample(logits[c], T, top_p, 1234, int(pos[c])), c


def test_logdef_bit_exact_against_oracle(lf, orc):
    import torch
    # every 37th binary32 from the smallest normal up to 17 (the Gumbel noise's
    # inputs lie in [2^-24, 1) and (0, 16.7]), plus edges: ~29M values
    lo, hi = np.float32(2.0 ** -126).view(np.uint32), np.float32(17.0).view(np.uint32)
    bits = np.arange(lo, hi + 1, 37, dtype=np.uint64).astype(np.uint32)
    x = np.concatenate([bits.view(np.float32),
                        np.float32([1.0, 2.0 ** -24, 1.0 - 2.0 ** -24, 0.5, 2.0, 1.4142135, 1.4142137])])
    y_gpu = lf.test_logdef(torch.from_numpy(x).cuda()).cpu().numpy()
    y_cpu = orc.logdef(x)
    assert np.array_equal(y_gpu.view(np.uint32), y_cpu.view(np.uint32))


@pytest.mark.parametrize("V,scale,T", [(32768, 1.0, 0.8), (32768, 4.0, 1.0), (128256, 1.0, 0.7),
                                       (37, 2.0, 1.3), (2, 1.0, 0.8), (1000, 0.05, 0.25)])
def test_gumbel_sampler_bit_exact_against_oracle(lf, orc, V, scale, T):
    import torch
    rng = np.random.default_rng(V + int(scale * 100))
    m = 24
    logits = (rng.standard_normal((m, V)) * scale).astype(np.float32)
    logits[1] = np.round(logits[1])                  # many exact ties
    logits[2] = 0.0                                   # all equal: the noise alone decides
    logits[3, :] = -40.0
    logits[3, V // 2] = 0.0                           # one token far ahead
    pos = np.concatenate([np.arange(16384, 16384 + m - 2), [0, 2 ** 31 - 1]]).astype(np.int32)
    seed = 0x9E3779B97F4A7C15
    tok = lf.test_sample_gumbel(torch.from_numpy(logits).cuda(), T, seed,
                                torch.from_numpy(pos).cuda()).cpu().numpy()
    for c in range(m):
        assert tok[c] == orc.sample_gumbel(logits[c], T, seed, int(pos[c])), c
    assert tok[3] == V // 2


# ---------------------------------------------------------------- tiny decoder

@pytest.fixture(scope="module")
def tiny():
    cfg = synth.CONFIGS["tiny_2l_d256"]
    return cfg, synth.model_weights(cfg)


def test_tiny_teacher_forced_logits_and_kv(lf, orc, tiny):
    import torch
    cfg, w = tiny
    prompt = synth.prompt(cfg, cfg["prompt_len"])
    m = orc.Model(cfg, w)
    ref_tokens = list(prompt)
    # oracle's own continuation fixes the teacher-forced sequence
    out = orc.Model(cfg, w)
    for p, t in enumerate(prompt[:-1]):
        out.decode_step(int(t), p)
    gen = out.generate(int(prompt[-1]), len(prompt) - 1, cfg["n_decode"])
    seq = list(prompt) + list(gen[:-1])
    eng, m, worst = teacher_forced(lf, orc, cfg, w, seq)
    n = len(seq)
    for l in range(cfg["n_layers"]):
        k, v = eng.kv_read(l, 0, n)
        k, v = k.cpu().numpy().astype(np.float32), v.cpu().numpy().astype(np.float32)
        rk, rv = m.kcache[l, :n].astype(np.float32), m.vcache[l, :n].astype(np.float32)
        assert np.abs(k - rk).max() <= 2e-2 * np.abs(rk).max() + 1e-3
        assert np.abs(v - rv).max() <= 2e-2 * np.abs(rv).max() + 1e-3


def test_tiny_free_running_greedy_stream(lf, orc, tiny):
    cfg, w = tiny
    prompt = synth.prompt(cfg, cfg["prompt_len"])
    eng = lf.Engine(cfg, lf.upload_weights(w))
    m = orc.Model(cfg, w)
    for p, t in enumerate(prompt[:-1]):
        eng.decode_step(int(t), p)
        m.decode_step(int(t), p)
    pos0 = len(prompt) - 1
    eng.set_position(int(prompt[-1]), pos0)
    got = eng.generate(cfg["n_decode"])
    ref, hist = m.generate(int(prompt[-1]), pos0, cfg["n_decode"], keep_logits=True)
    for i in range(cfg["n_decode"]):
        if margin(hist[i]) < 1e-2:
            break                     # later tokens are not compared
        assert got[i] == ref[i], i


def test_generate_equals_stepwise_decode(lf, tiny):
    cfg, w = tiny
    dw = lf.upload_weights(w)
    a, b = lf.Engine(cfg, dw), lf.Engine(cfg, dw)
    a.decode_step(5, 0)
    ga = a.generate(20)
    tok = b.decode_step(5, 0)
    gb = []
    for i in range(20):
        tok = b.decode_step(tok, 1 + i)
        gb.append(tok)
    assert list(ga) == gb


def test_tiny_smaller_grid_same_results(lf, orc, tiny, monkeypatch):
    """A grid smaller than the attention unit count (units loop per workgroup)."""
    cfg, w = tiny
    monkeypatch.setenv("LF_GRID", "7")
    eng = lf.Engine(cfg, lf.upload_weights(w))
    assert eng.grid == 7
    teacher_forced(lf, orc, cfg, w, synth.prompt(cfg, 6), engine=eng)


@pytest.mark.parametrize("pieces,kind", [(16, 2), (3, 2), (16, 1), (3, 1)])
def test_lds_prefetch(lf, orc, tiny, monkeypatch, pieces, kind):
    """The LDS prefetch of a projection's first pieces, forced on gate/up (kind
    2) or the output projection (kind 1): the tiny model's rows of 32 vectors
    (one masked piece per row, whole wave shares in LDS) and the 2.2B layer
    shape, whose 16- or 3-piece prefetch ends inside a row of five pieces, so
    the ring part goes on with the running row sum."""
    monkeypatch.setenv("LF_GU_PF", str(pieces))
    monkeypatch.setenv("LF_PF_KIND", str(kind))
    cfg, w = tiny
    eng = lf.Engine(cfg, lf.upload_weights(w))
    assert eng.query(lf.LF_Q_GU_PF) == pieces
    assert eng.query(lf.LF_Q_PF_KIND) == kind
    teacher_forced(lf, orc, cfg, w, synth.prompt(cfg, 6), engine=eng)
    layer_d2560_at(lf, orc, 200)


def layer_d2560_at(lf, orc, P):
    """One 2.2B-shaped layer (hidden vector in and out) at position P over a
    synthetic cache, against the oracle's layer."""
    import torch
    cfg = synth.CONFIGS["layer_d2560_kv1024"]
    w = synth.model_weights(cfg)
    k, v = synth.kv_prefill(cfg, P)
    x = synth.hidden(cfg)
    eng = lf.Engine(cfg, lf.upload_weights(w))
    eng.kv_fill(0, 0, torch.from_numpy(k[0]).cuda(), torch.from_numpy(v[0]).cuda())
    eng.set_hidden(torch.from_numpy(x).cuda())
    eng.decode_step(0, P)
    got = eng.get_hidden().cpu().numpy()
    m = orc.Model(cfg, w)
    m.kv_fill(k, v, 0)
    ok, err = close(got, m.layer_forward(0, x, P))
    assert ok, err
    return eng


def test_output_projection_prefetch_rule(lf, orc, monkeypatch):
    """By default the output projection is prefetched into LDS only where a
    stream wave's share is more than one ring round and fits LDS whole: not at
    the 2.2B layer shape (about 8 pieces a wave, one round)."""
    monkeypatch.delenv("LF_GU_PF", raising=False)
    eng = layer_d2560_at(lf, orc, 300)
    assert eng.query(lf.LF_Q_PF_KIND) == 1
    assert eng.query(lf.LF_Q_GU_PF) == 0


@pytest.mark.parametrize("ww,grid", [("1024:64:64:64:64:64:1024", None), ("64:1024:64:1024:64:1024:64", None),
                                     ("1024:64:64:64:64:64:1024", "64"), ("256:256:256:256:256:256:256", None)])
def test_wave_shares_uneven_weights(lf, orc, tiny, monkeypatch, ww, grid):
    """A workgroup's rows split over its stream waves by extreme weights: the
    heavy waves hit the cap of whole rounds and the light waves take what is
    left, so every row is still summed exactly once.  Tiny model teacher-forced
    and the 2.2B layer shape at position 700 (1-5 rounds of 8 pieces per wave;
    on a 64-workgroup grid gate/up has 19, where the cap allows one round more
    than an equal share), and equal weights."""
    monkeypatch.setenv("LF_WAVE_W", ww)
    if grid:
        monkeypatch.setenv("LF_GRID", grid)
    cfg, w = tiny
    eng = lf.Engine(cfg, lf.upload_weights(w))
    want = [int(s) for s in ww.split(":")]
    assert [eng.query(lf.LF_Q_WAVE_W + k) for k in range(7)] == want
    assert eng.query(lf.LF_Q_WAVE_W_KINDS) == 31
    teacher_forced(lf, orc, cfg, w, synth.prompt(cfg, 6), engine=eng)
    eng = layer_d2560_at(lf, orc, 700)
    assert [eng.query(lf.LF_Q_WAVE_W + k) for k in range(7)] == want


@pytest.mark.parametrize("waves", [7, 2])
def test_attention_tile_prefetch(lf, orc, monkeypatch, waves):
    """The K/V tile prefetch into LDS (off by default): the workgroups that run
    attention stream no QKV rows and copy their stream waves' first tile into LDS
    during the QKV phase.  With 2 waves prefetching, the other waves' tiles come
    from the cache as usual.  GQA 8/2 x 64 (three tiles at the last positions) and
    the 2.2B layer shape at position 200 (four tiles, one unit per head)."""
    import torch
    monkeypatch.setenv("LF_KV_PF", str(waves))
    cfg = synth.scaled_config("tiny_2l_d256", n_heads=8, n_kv_heads=2, head_dim=64, max_seq=256)
    w = synth.model_weights(cfg, seed=4)
    eng = lf.Engine(cfg, lf.upload_weights(w))
    assert eng.query(lf.LF_Q_KV_PF) == waves
    teacher_forced(lf, orc, cfg, w, synth.prompt(cfg, 150), engine=eng)
    cfg = synth.CONFIGS["layer_d2560_kv1024"]
    w = synth.model_weights(cfg)
    P = 200
    k, v = synth.kv_prefill(cfg, P)
    x = synth.hidden(cfg)
    eng = lf.Engine(cfg, lf.upload_weights(w))
    eng.kv_fill(0, 0, torch.from_numpy(k[0]).cuda(), torch.from_numpy(v[0]).cuda())
    eng.set_hidden(torch.from_numpy(x).cuda())
    eng.decode_step(0, P)
    got = eng.get_hidden().cpu().numpy()
    m = orc.Model(cfg, w)
    m.kv_fill(k, v, 0)
    ok, err = close(got, m.layer_forward(0, x, P))
    assert ok, err


@pytest.mark.parametrize("qsplit", ["1", "0"])
def test_gqa_and_head64_variants(lf, orc, monkeypatch, qsplit):
    """GQA 8/2 at head dim 64, 8/1 at 128 and MHA 2/2: logits against the oracle,
    with short heads split into one attention unit per query head (the default)
    and with one unit per KV head."""
    monkeypatch.setenv("LF_ATTN_QSPLIT", qsplit)
    for kw in (dict(n_heads=8, n_kv_heads=2, head_dim=64), dict(n_heads=8, n_kv_heads=1, head_dim=128),
               dict(n_heads=2, n_kv_heads=2, head_dim=128, d_model=512, ffn_dim=1376, vocab=1000)):
        cfg = synth.scaled_config("tiny_2l_d256", **kw)
        w = synth.model_weights(cfg, seed=3)
        teacher_forced(lf, orc, cfg, w, synth.prompt(cfg, 5))


@pytest.mark.parametrize("path", ["grid", "grid7", "wg0"])
def test_sampling_model_tokens_match_oracle_sampler(lf, orc, tiny, monkeypatch, path):
    """Temperature / top-p in the kernel: for the GPU's own logits and counters the
    oracle sampler picks the same token at every step.  grid: the draw spread over
    the lm_head workgroups; grid7: the same on a 7-workgroup grid (fewer
    workgroups than bins, so each sums several bins); wg0: workgroup 0 alone."""
    cfg, w = tiny
    cfg = dict(cfg, temperature=0.8, top_p=0.9, seed=1234)
    if path == "grid7":
        monkeypatch.setenv("LF_GRID", "7")
    if path == "wg0":
        monkeypatch.setenv("LF_NUC_WG0", "1")
    eng = lf.Engine(cfg, lf.upload_weights(w))
    tok, pos = 7, 0
    for _ in range(20):
        nxt = eng.decode_step(tok, pos)
        logits = eng.logits().cpu().numpy()
        assert nxt == orc.sample(logits, 0.8, 0.9, 1234, pos)
        tok, pos = nxt, pos + 1


@pytest.mark.parametrize("path", ["grid", "grid7", "wg0"])
def test_nucleus_generate_equals_stepwise(lf, tiny, monkeypatch, path):
    """Top-p tokens drawn inside one launch of 20 tokens (each token's draw at six
    levels of its own over the grid) equal those of 20 one-token launches."""
    cfg, w = tiny
    cfg = dict(cfg, temperature=0.8, top_p=0.9, seed=99)
    if path == "grid7":
        monkeypatch.setenv("LF_GRID", "7")
    if path == "wg0":
        monkeypatch.setenv("LF_NUC_WG0", "1")
    dw = lf.upload_weights(w)
    a, b = lf.Engine(cfg, dw), lf.Engine(cfg, dw)
    a.decode_step(5, 0)
    ga = a.generate(20)
    tok = b.decode_step(5, 0)
    gb = []
    for i in range(20):
        tok = b.decode_step(tok, 1 + i)
        gb.append(tok)
    assert list(ga) == gb


@pytest.mark.parametrize("path", ["grid", "wg0"])
def test_nucleus_flat_logits(lf, orc, tiny, monkeypatch, path):
    """A zero lm_head: every logit is 0, all 4096 tokens tie in the first bin, more
    candidates than the list holds, so the boundary key is found by scanning
    every logit of the bin; the token still equals the oracle sampler's."""
    cfg, w = tiny
    cfg = dict(cfg, temperature=0.8, top_p=0.9, seed=7)
    w = dict(w, lm_head=np.zeros_like(w["lm_head"]))
    if path == "wg0":
        monkeypatch.setenv("LF_NUC_WG0", "1")
    eng = lf.Engine(cfg, lf.upload_weights(w))
    tok = 3
    for pos in range(4):
        nxt = eng.decode_step(tok, pos)
        logits = eng.logits().cpu().numpy()
        assert not logits.any()
        assert nxt == orc.sample(logits, 0.8, 0.9, 7, pos)
        tok = nxt


def test_gumbel_model_tokens_match_oracle_sampler(lf, orc, tiny):
    """Gumbel-max in the decode kernel (each lm_head workgroup publishes its best
    noised score): for the GPU's own logits and counters the oracle's Gumbel-max
    picks the same token at every step, stepwise and in one multi-token launch."""
    cfg, w = tiny
    cfg = dict(cfg, temperature=0.8, top_p=0.0, seed=987654321, sampler="gumbel")
    dw = lf.upload_weights(w)
    eng = lf.Engine(cfg, dw)
    tok, pos, steps = 7, 0, []
    for _ in range(20):
        nxt = eng.decode_step(tok, pos)
        logits = eng.logits().cpu().numpy()
        assert nxt == orc.sample_gumbel(logits, 0.8, 987654321, pos), pos
        steps.append(nxt)
        tok, pos = nxt, pos + 1
    other = lf.Engine(cfg, dw)
    other.decode_step(7, 0)
    assert list(other.generate(19)) == steps[1:]
    del dw


# ---------------------------------------------------------------- edges

def test_position_zero_and_last_position(lf, orc, tiny):
    cfg, w = tiny
    eng, m, _ = teacher_forced(lf, orc, cfg, w, [3])                # pos 0: a single key
    last = cfg["max_seq"] - 1
    k = synth.kv_prefill(cfg, last)
    import torch
    for l in range(cfg["n_layers"]):
        eng.kv_fill(l, 0, torch.from_numpy(k[0][l]).cuda(), torch.from_numpy(k[1][l]).cuda())
    m.kv_fill(k[0], k[1], 0)
    teacher_forced(lf, orc, cfg, w, [11], pos0=last, engine=eng, model=m)


def test_errors(lf, tiny):
    cfg, w = tiny
    eng = lf.Engine(cfg, lf.upload_weights(w))
    with pytest.raises(lf.LfError) as e:
        eng.decode_step(0, cfg["max_seq"])
    assert e.value.code == lf.LF_ERANGE
    with pytest.raises(lf.LfError) as e:
        eng.decode_step(cfg["vocab"], 0)
    assert e.value.code == lf.LF_ERANGE
    eng.decode_step(1, cfg["max_seq"] - 3)
    with pytest.raises(lf.LfError) as e:
        eng.generate(5)                           # runs past max_seq
    assert e.value.code == lf.LF_ERANGE
    assert len(eng.generate(2)) == 2


def test_timeout_path_exits_cleanly(lf, tiny, monkeypatch):
    """A tiny bound on the in-kernel waits makes them expire: the kernel must
    drain and report LF_ETIMEOUT, and a normal state must work afterwards."""
    cfg, w = tiny
    dw = lf.upload_weights(w)
    monkeypatch.setenv("LF_TIMEOUT_MS", "0.0001")
    eng = lf.Engine(cfg, dw)
    codes = set()
    for i in range(3):
        try:
            eng.decode_step(1, i)
            codes.add(0)
        except lf.LfError as e:
            codes.add(e.code)
    assert codes <= {0, lf.LF_ETIMEOUT} and lf.LF_ETIMEOUT in codes
    monkeypatch.delenv("LF_TIMEOUT_MS")
    ok = lf.Engine(cfg, dw)
    assert ok.decode_step(1, 0) >= 0


def test_non_unit_norm_gains(lf, orc):
    """Gains other than 1: the library folds each RMSNorm gain vector into the
    columns of the projection after it (QKV, gate/up, lm_head) and scales the row
    sums by 1/rms; the oracle applies RMSNorm as defined."""
    cfg = synth.CONFIGS["tiny_2l_d256"]
    w = synth.model_weights(cfg, seed=5)
    d = cfg["d_model"]

    def gains(tid):
        return (1.0 + 0.25 * synth.normal_f32(d, 77, tid)).astype(np.float16)

    for l, lw in enumerate(w["layers"]):
        lw["attn_norm"], lw["ffn_norm"] = gains(2 * l), gains(2 * l + 1)
    w["final_norm"] = gains(99)
    teacher_forced(lf, orc, cfg, w, synth.prompt(cfg, 12))


def test_large_activations_across_chunks(lf, orc):
    """Weights at 5x the usual scale give residual and SwiGLU values well above
    1, which the kernel stages unnormalised as fp16; positions up to 40 split the
    attention over several chunks, whose keys past the chunk must contribute
    nothing (regression: a current-row patch past the chunk produced NaN)."""
    cfg = synth.CONFIGS["tiny_2l_d256"]
    w = synth.model_weights(cfg, seed=9, scale=0.1)
    eng, m, worst = teacher_forced(lf, orc, cfg, w, synth.prompt(cfg, 40))
    assert np.isfinite(eng.logits().cpu().numpy()).all()


# ---------------------------------------------------------------- full-size shapes

def test_single_layer_2b_shape_hidden_io(lf, orc):
    """One d2560 / 20x128 / F6912 layer, KV prefilled to 1024, one step at pos 1024."""
    import torch
    cfg = synth.CONFIGS["layer_d2560_kv1024"]
    w = synth.model_weights(cfg)
    k, v = synth.kv_prefill(cfg, cfg["kv_prefill"])
    x = synth.hidden(cfg)
    eng = lf.Engine(cfg, lf.upload_weights(w))
    eng.kv_fill(0, 0, torch.from_numpy(k[0]).cuda(), torch.from_numpy(v[0]).cuda())
    eng.set_hidden(torch.from_numpy(x).cuda())
    eng.decode_step(0, cfg["kv_prefill"])
    got = eng.get_hidden().cpu().numpy()
    m = orc.Model(cfg, w)
    m.kv_fill(k, v, 0)
    ref = m.layer_forward(0, x, cfg["kv_prefill"])
    ok, err = close(got, ref)
    assert ok, err
    gk, gv = eng.kv_read(0, cfg["kv_prefill"], 1)
    assert np.abs(gv.cpu().numpy().astype(np.float32) - m.vcache[0, 1024].astype(np.float32)).max() < 2e-2


@pytest.fixture(scope="module")
def dec2b():
    cfg = synth.CONFIGS["dec2b_25l_greedy"]
    return cfg, synth.model_weights(cfg)


def test_dec2b_teacher_forced_and_generate_launch(lf, orc, dec2b):
    """The ~2.2B decoder at full size: teacher-forced steps against the oracle, then
    the multi-token launch the benchmark times, checked against the step-by-step
    launches of the same engine and the oracle's greedy continuation."""
    cfg, w = dec2b
    orc.set_threads(min(16, os.cpu_count() or 1))
    dw = lf.upload_weights(w)
    prompt = synth.prompt(cfg, 6)
    eng, m, _ = teacher_forced(lf, orc, cfg, w, prompt, engine=lf.Engine(cfg, dw))
    n = 6
    eng.set_position(int(prompt[-1]), len(prompt) - 1)
    # restart from the last prompt position: the cache rows beyond it are rewritten
    got = eng.generate(n)
    m2 = orc.Model(cfg, w)
    for p, t in enumerate(prompt[:-1]):
        m2.decode_step(int(t), p)
    ref, hist = m2.generate(int(prompt[-1]), len(prompt) - 1, n, keep_logits=True)
    for i in range(n):
        if margin(hist[i]) < 1e-2:
            break
        assert got[i] == ref[i], i
    del dw


@pytest.mark.timeout(900)
def test_dec2b_timed_positions_prefill_and_generate(lf, orc, dec2b):
    """The benchmark's own path at the ~2.2B shape: the 127-token prompt in one
    teacher-forced launch, then steps at the timed positions 127.. against the
    oracle (logits within tolerance every step), then one generate launch from
    position 127 replayed through the oracle."""
    cfg, w = dec2b
    orc.set_threads(min(16, os.cpu_count() or 1))
    prompt = synth.prompt(cfg, cfg["prompt_len"])
    P = len(prompt) - 1
    eng = lf.Engine(cfg, lf.upload_weights(w))
    eng.prefill(prompt[:P], 0)
    m = orc.Model(cfg, w)
    for p in range(P):
        m.decode_step(int(prompt[p]), p)
    # snapshot the oracle's cache so that the generate check restarts from pos P
    kc, vc = m.kcache.copy(), m.vcache.copy()
    tok = int(prompt[P])
    for i in range(3):
        pos = P + i
        nxt = eng.decode_step(tok, pos)
        ref = m.decode_step(tok, pos)
        ok, err = close(eng.logits().cpu().numpy(), ref)
        assert ok, (pos, err)
        if margin(ref) >= 1e-2:
            assert nxt == orc.argmax(ref), pos
        tok = orc.argmax(ref)
    replay_generate(eng, m, int(prompt[P]), P, 8, kc, vc)


@pytest.fixture(scope="module")
def dec8b():
    cfg = synth.CONFIGS["dec8b_32l_gqa"]
    return cfg, synth.model_weights(cfg)


@pytest.mark.timeout(900)
def test_dec8b_gqa_full_shape(lf, orc, dec8b):
    """The ~8B GQA decoder at full size (32 layers, d 4096, 32 query / 8 KV heads of
    dim 128, F 14336, untied vocabulary of 128,256 over the lm_head workgroups):
    teacher-forced steps from position 0; then the cache is filled with 255
    synthetic rows and the steps at positions 255.. attend over them (4 tiles per
    KV head: one attention unit per query head); then one generate launch
    replayed through the oracle.  Logits within tolerance at every step, greedy
    tokens equal where the oracle's top-2 margin is at least 1e-2.  The output
    projection is prefetched into LDS in part (11 of 24 pieces a wave)."""
    import torch
    cfg, w = dec8b
    orc.set_threads(min(16, os.cpu_count() or 1))
    dw = lf.upload_weights(w)
    eng = lf.Engine(cfg, dw)
    del dw
    torch.cuda.empty_cache()
    assert eng.query(lf.LF_Q_PF_KIND) == 1 and eng.query(lf.LF_Q_GU_PF) >= 8
    m = orc.Model(cfg, w)
    prompt = synth.prompt(cfg, 3)
    teacher_forced(lf, orc, cfg, w, prompt, engine=eng, model=m)
    P = 255
    k, v = synth.kv_prefill(cfg, P)
    for l in range(cfg["n_layers"]):
        eng.kv_fill(l, 0, torch.from_numpy(k[l]).cuda(), torch.from_numpy(v[l]).cuda())
    m.kv_fill(k, v, 0)
    del k, v
    kc, vc = m.kcache.copy(), m.vcache.copy()
    tok0 = int(synth.prompt(cfg, 4)[3])
    tok = tok0
    for i in range(3):
        pos = P + i
        nxt = eng.decode_step(tok, pos)
        ref = m.decode_step(tok, pos)
        got = eng.logits().cpu().numpy()
        ok, err = close(got, ref)
        assert ok, (pos, err, np.abs(ref).max())
        if margin(ref) >= 1e-2:
            assert nxt == orc.argmax(ref), pos
        tok = orc.argmax(ref)
    replay_generate(eng, m, tok0, P, 6, kc, vc)


@pytest.mark.timeout(600)
def test_dec8b_nucleus_full_vocab(lf, orc, dec8b):
    """Temperature 0.8 / top-p 0.9 on the 8B model: the nucleus draw over the grid
    at a 128,256-row vocabulary (about 500 lm_head rows per workgroup, listed as
    16-bit offsets).  For the kernel's own logits and counter, the oracle sampler
    picks the same token at every step."""
    import torch
    cfg, w = dec8b
    cfg = dict(cfg, temperature=0.8, top_p=0.9, seed=4321)
    dw = lf.upload_weights(w)
    eng = lf.Engine(cfg, dw)
    del dw
    torch.cuda.empty_cache()
    tok = int(synth.prompt(cfg, 1)[0])
    for pos in range(6):
        nxt = eng.decode_step(tok, pos)
        logits = eng.logits().cpu().numpy()
        assert nxt == orc.sample(logits, 0.8, 0.9, 4321, pos), pos
        tok = nxt
    eng.close()


def test_dec2b_long_context_sampling(lf, orc, dec2b):
    """16K prefilled cache, temperature 0.8 / top-p 0.9 Philox sampling at pos 16384..:
    GPU logits within tolerance of the oracle's, and the token the kernel samples
    equals the oracle sampler's on the GPU's own logits."""
    import torch
    cfg = synth.CONFIGS["dec2b_25l_kv16k_topp"]
    _, w = dec2b
    orc.set_threads(min(16, os.cpu_count() or 1))
    P = cfg["kv_prefill"]
    k, v = synth.kv_prefill(cfg, P)
    eng = lf.Engine(cfg, lf.upload_weights(w))
    for l in range(cfg["n_layers"]):
        eng.kv_fill(l, 0, torch.from_numpy(k[l]).cuda(), torch.from_numpy(v[l]).cuda())
    m = orc.Model(cfg, w)
    m.kv_fill(k, v, 0)
    del k, v
    tok = int(synth.prompt(dict(cfg, prompt_len=1), 1)[0])
    for i in range(3):
        pos = P + i
        nxt = eng.decode_step(tok, pos)
        got = eng.logits().cpu().numpy()
        ref = m.decode_step(tok, pos)
        ok, err = close(got, ref)
        assert ok, (pos, err)
        assert nxt == orc.sample(got, 0.8, 0.9, 1234, pos)
        tok = nxt


def test_dec2b_gumbel_sampling(lf, orc, dec2b):
    """The ~2.2B decoder with Gumbel-max sampling (V = 32768 over 256 lm_head
    workgroups): GPU logits within tolerance of the oracle's, and the sampled
    token equals the oracle's Gumbel-max on the GPU's own logits."""
    cfg, w = dec2b
    cfg = dict(cfg, temperature=0.8, sampler="gumbel", seed=4242)
    orc.set_threads(min(16, os.cpu_count() or 1))
    eng = lf.Engine(cfg, lf.upload_weights(w))
    m = orc.Model(cfg, w)
    tok = int(synth.prompt(cfg, 1)[0])
    for pos in range(4):
        nxt = eng.decode_step(tok, pos)
        got = eng.logits().cpu().numpy()
        ok, err = close(got, m.decode_step(tok, pos))
        assert ok, (pos, err)
        assert nxt == orc.sample_gumbel(got, 0.8, 4242, pos), pos
        tok = nxt


def test_gqa_query_split_then_tile_split(lf, orc):
    """GQA 8/2 heads of dim 64 teacher-forced through position 469.  While a KV
    head's cached keys fit in one unit (at most 7 tiles of 64 keys: positions up
    to 448), attention runs one unit per query head.  Past that, each KV head is
    split into units of about 3 tiles, each with its 4 query heads, and the
    units' partials are merged.  Logits are checked against the oracle at every
    position."""
    cfg = synth.scaled_config("tiny_2l_d256", n_heads=8, n_kv_heads=2, head_dim=64, max_seq=512)
    w = synth.model_weights(cfg, seed=11)
    teacher_forced(lf, orc, cfg, w, synth.prompt(cfg, 470))


@pytest.mark.parametrize("qsplit", ["1", "0"])
def test_sliding_window_gqa_head96_teacher_forced(lf, orc, monkeypatch, qsplit):
    """Sliding-window attention on layers 0 and 2 of three (window 36: the windowed
    layers split 3 ways, the full layer 4 ways at the end), GQA 4/2 heads of dim 96:
    logits against the oracle at every position, most of them past the window;
    short heads split by query heads or not."""
    monkeypatch.setenv("LF_ATTN_QSPLIT", qsplit)
    cfg = synth.scaled_config("tiny_2l_d256", n_layers=3, d_model=384, n_heads=4, n_kv_heads=2,
                              head_dim=96, ffn_dim=1024, vocab=2000, max_seq=64,
                              sliding_window=36, window_layers=0b101)
    w = synth.model_weights(cfg, seed=5)
    prompt = synth.prompt(cfg, 60)
    teacher_forced(lf, orc, cfg, w, prompt)
    # the check is decisive: full attention in every layer misses the tolerance
    a, b = orc.Model(cfg, w), orc.Model(dict(cfg, sliding_window=0, window_layers=0), w)
    for pos, t in enumerate(prompt):
        la, lb = a.decode_step(int(t), pos), b.decode_step(int(t), pos)
    assert not close(la, lb)[0]


def test_laneformer_shape_sliding_window_long_context(lf, orc):
    """The LaneFormer-2B-shaped decoder (15 layers, 32/16 heads of dim 96, window
    1024 in 10 layers) with its cache prefilled to 2048: GPU logits within
    tolerance of the oracle's and the greedy token equal where the margin allows
    (with the output projection prefetched into LDS, as by default at this
    shape); then one 8-token generate launch from 2048, as the benchmark times
    it, replayed through the oracle."""
    import torch
    cfg = synth.CONFIGS["laneformer_15l_swa"]
    w = synth.model_weights(cfg)
    orc.set_threads(min(16, os.cpu_count() or 1))
    P = cfg["kv_prefill"]
    k, v = synth.kv_prefill(cfg, P)
    eng = lf.Engine(cfg, lf.upload_weights(w))
    # a stream wave's share of the output projection (13 rows of 6 pieces per
    # workgroup) is more than one ring round: prefetched into LDS whole
    assert eng.query(lf.LF_Q_PF_KIND) == 1
    assert eng.query(lf.LF_Q_GU_PF) >= 12
    for l in range(cfg["n_layers"]):
        eng.kv_fill(l, 0, torch.from_numpy(k[l]).cuda(), torch.from_numpy(v[l]).cuda())
    m = orc.Model(cfg, w)
    m.kv_fill(k, v, 0)
    del k, v
    # snapshot the oracle's cache so that the generate check restarts from pos P
    kc, vc = m.kcache.copy(), m.vcache.copy()
    tok0 = int(synth.prompt(dict(cfg, prompt_len=1), 1)[0])
    tok = tok0
    for i in range(3):
        pos = P + i
        nxt = eng.decode_step(tok, pos)
        got = eng.logits().cpu().numpy()
        ref = m.decode_step(tok, pos)
        ok, err = close(got, ref)
        assert ok, (pos, err)
        if margin(ref) >= 1e-2:
            assert nxt == int(np.argmax(ref)), pos
        tok = int(np.argmax(ref))
    # the benchmark's launch: one generate from position P
    replay_generate(eng, m, tok0, P, 8, kc, vc)


def test_prefill_one_launch_matches_oracle(lf, orc, tiny):
    """Teacher-forced prompt in one launch: the cache it leaves and the step after
    it agree with the oracle."""
    cfg, w = tiny
    prompt = synth.prompt(cfg, cfg["prompt_len"])
    eng = lf.Engine(cfg, lf.upload_weights(w))
    m = orc.Model(cfg, w)
    n = len(prompt) - 1
    eng.prefill(prompt[:n], 0)
    for p in range(n):
        m.decode_step(int(prompt[p]), p)
    for l in range(cfg["n_layers"]):
        k, v = eng.kv_read(l, 0, n)
        assert np.abs(k.cpu().numpy().astype(np.float32) - m.kcache[l, :n].astype(np.float32)).max() < 2e-2
        assert np.abs(v.cpu().numpy().astype(np.float32) - m.vcache[l, :n].astype(np.float32)).max() < 2e-2
    teacher_forced(lf, orc, cfg, w, [int(prompt[n])], pos0=n, engine=eng, model=m)
