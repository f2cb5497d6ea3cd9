"""lf_generate_noalloc (the entry point that allocates nothing) against
lf_generate on the same state: the same kernel over the static scratch array
instead of the state's buffers, so tokens and the last step's logits must be
identical bit for bit.  Two calls in a row, the second shorter, so that the
second runs over the first one's leftover scratch contents."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lf():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the -m gpu tests must run on an MI355X")
    from persistent_runtime_amd import lf as mod
    mod.lib()
    return mod


CASES = {
    "tiny_mha": synth.CONFIGS["tiny_2l_d256"],
    # temperature / top-p: the nucleus draw's exchange buffers live in the array too
    "tiny_topp": dict(synth.CONFIGS["tiny_2l_d256"], temperature=0.8, top_p=0.9, seed=99),
    # GQA 4/2 heads of dim 96 with a sliding window on two of three layers: other
    # exchange-buffer sizes and several attention chunks per KV head
    "gqa_window": synth.scaled_config("tiny_2l_d256", n_layers=3, d_model=384, n_heads=4, n_kv_heads=2,
                                      head_dim=96, ffn_dim=1024, vocab=2000, max_seq=96,
                                      sliding_window=36, window_layers=0b101),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_noalloc_generate_equals_generate(lf, name):
    import torch
    cfg = CASES[name]
    w = synth.model_weights(cfg, seed=3)
    eng = lf.Engine(cfg, lf.upload_weights(w))
    need, cap = eng.query(lf.LF_Q_SCRATCH_BYTES), eng.query(lf.LF_Q_SCRATCH_MAX)
    assert 0 < need <= cap == 4 << 20
    prompt = synth.prompt(cfg, 20)
    P = len(prompt) - 1
    eng.prefill(prompt[:P], 0)
    out = torch.full((40,), -1, dtype=torch.int32, device="cuda")
    first = None
    for n in (40, 11):   # the second call is shorter and starts over the first one's scratch
        eng.set_position(int(prompt[P]), P)
        ref = eng.generate(n)
        ref_logits = eng.logits().cpu().numpy()
        eng.set_position(int(prompt[P]), P)
        got = eng.generate_noalloc(n, out)
        torch.cuda.synchronize()
        assert np.array_equal(got[:n].cpu().numpy(), ref), (name, n)
        assert np.array_equal(eng.logits().cpu().numpy().view(np.uint32), ref_logits.view(np.uint32)), (name, n)
        if first is None:
            first = got.cpu().numpy().copy()
        else:   # entries past n belong to the caller: this call left them as they were
            assert np.array_equal(got[n:].cpu().numpy(), first[n:])
    # the pending position advanced like lf_generate's: the next call continues
    nxt = eng.generate_noalloc(3)
    eng.set_position(int(prompt[P]), P)
    full = eng.generate(14)
    assert np.array_equal(nxt.cpu().numpy(), full[11:14])
    eng.close()


def test_noalloc_rejects_a_state_beyond_the_array(lf):
    """64 query heads over 8 KV heads of dim 128: the split-attention partials
    alone exceed the 4 MiB array, so the entry point refuses before launching."""
    cfg = synth.scaled_config("tiny_2l_d256", n_layers=1, d_model=512, n_heads=64, n_kv_heads=8,
                              head_dim=128, ffn_dim=512, vocab=256, max_seq=32)
    eng = lf.Engine(cfg, lf.upload_weights(synth.model_weights(cfg)))
    assert eng.query(lf.LF_Q_SCRATCH_BYTES) > eng.query(lf.LF_Q_SCRATCH_MAX)
    eng.decode_step(1, 0)
    with pytest.raises(lf.LfError) as ei:
        eng.generate_noalloc(2)
    assert ei.value.code == lf.LF_EUNSUPPORTED and "scratch" in str(ei.value)
    eng.close()
