"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point include/lf.h declares, and rejects bad configurations before
touching the device."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "lf.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lf_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lf():
    from persistent_runtime_amd import lf as mod
    if not os.path.exists(mod.LIB_PATH):
        pytest.fail("liblf.so is not built (run __graft_entry__.build())")
    mod.lib()
    return mod


def test_library_exports_every_declared_symbol(lf):
    declared = _declared()
    assert len(declared) >= 15
    lib = C.CDLL(lf.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(lf.EXPORTS) == declared


def _cfg(**kw):
    import synth
    c = dict(synth.CONFIGS["tiny_2l_d256"])
    c.update(kw)
    return c


def _create(lf, cfg, weights_ptr_ok=True):
    c = lf.make_config(cfg)
    L = cfg["n_layers"]
    layers = (lf.LfLayerWeights * L)()
    fake = 0x1000 if weights_ptr_ok else None
    for i in range(L):
        for n in lf.LAYER_NAMES:
            setattr(layers[i], n, fake)
    w = lf.LfWeights(fake, fake, fake, layers)
    st = C.c_void_p()
    rc = lf.lib().lf_model_create(C.byref(c), C.byref(w), None, C.byref(st))
    return rc, lf.lib().lf_last_error(None).decode()


@pytest.mark.parametrize("kw,code", [
    (dict(n_heads=4, n_kv_heads=3), -1),           # heads not a multiple of KV heads
    (dict(head_dim=80), -6),                        # unsupported head size
    (dict(sliding_window=-1), -1),
    (dict(d_model=250), -1),                        # d_model not a multiple of 8
    (dict(vocab=4095), -1),                         # odd vocabulary
    (dict(n_layers=0), -1),
    (dict(temperature=0.8, top_p=0.0), -1),
    (dict(n_heads=36, n_kv_heads=4), -6),           # 9 query heads per KV head
    (dict(sliding_window=16, window_layers=0b100), -1),   # mask bit at or above n_layers (2)
    (dict(sliding_window=16, n_layers=65, window_layers=1), -6),   # the mask word covers 64 layers
])
def test_create_rejects_bad_config_without_device(lf, kw, code):
    rc, msg = _create(lf, _cfg(**kw))
    assert rc == code and msg


def test_create_rejects_null_weights(lf):
    rc, msg = _create(lf, _cfg(), weights_ptr_ok=False)
    assert rc == -1 and msg


def test_null_state_calls_fail_cleanly(lf):
    L = lf.lib()
    nxt = C.c_int32()
    assert L.lf_decode_step(None, 0, 0, C.byref(nxt)) == -1
    assert L.lf_generate(None, 1, None) == -1
    assert L.lf_query(None, 0) == -1
    L.lf_model_destroy(None)
