"""ctypes front end of the CPU oracle (``liblf_oracle.so``).

TEST INFRASTRUCTURE ONLY.  The plain fp32 CPU decoder in ``lf_oracle.cpp`` is
the reference the GPU path is checked against.  Only the tests, the smoke check
and the CPU-baseline leg of the benchmark may import this package; the product
package never does, and this package imports nothing from it.

Inputs are host numpy arrays (fp16 weights as ``numpy.float16``; the KV cache
as ``[L][max_seq][n_kv_heads][head_dim]`` float16 arrays owned by ``Model``).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblf_oracle.so")


class OrcConfig(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_layers", "d_model", "n_heads", "n_kv_heads",
                                         "head_dim", "ffn_dim", "vocab", "max_seq")] + \
               [("rms_eps", C.c_float), ("rope_base", C.c_float), ("sliding_window", C.c_int32),
                ("reserved", C.c_int32), ("window_layers", C.c_uint64)]


_LAYER_NAMES = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")


class OrcLayer(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in _LAYER_NAMES]


class OrcWeights(C.Structure):
    _fields_ = [("tok_emb", C.c_void_p), ("final_norm", C.c_void_p), ("lm_head", C.c_void_p),
                ("layers", C.POINTER(OrcLayer))]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(LIB_PATH)
        P = C.c_void_p
        L.orc_f16_to_f32.restype = C.c_float
        L.orc_f16_to_f32.argtypes = [C.c_uint16]
        L.orc_f32_to_f16.restype = C.c_uint16
        L.orc_f32_to_f16.argtypes = [C.c_float]
        L.orc_f16_to_f32_n.argtypes = [P, P, C.c_size_t]
        L.orc_f32_to_f16_n.argtypes = [P, P, C.c_size_t]
        L.orc_gemv.argtypes = [P, P, C.c_int32, C.c_int32, P]
        L.orc_rmsnorm.argtypes = [P, P, C.c_int32, C.c_float, P]
        L.orc_rope.argtypes = [P, C.c_int32, C.c_int32, C.c_float]
        L.orc_attention.argtypes = [P, P, P, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, P]
        L.orc_silu.restype = C.c_float
        L.orc_silu.argtypes = [C.c_float]
        L.orc_layer_forward.argtypes = [P, P, P, P, P, C.c_int32, C.c_int32]
        L.orc_decode_step.argtypes = [P, P, P, P, C.c_int32, C.c_int32, P]
        L.orc_forward_nocache.argtypes = [P, P, P, C.c_int32, P]
        L.orc_argmax.restype = C.c_int32
        L.orc_argmax.argtypes = [P, C.c_int32]
        L.orc_expdef.restype = C.c_float
        L.orc_expdef.argtypes = [C.c_float]
        L.orc_expdef_constants.argtypes = [P]
        L.orc_expdef_n.argtypes = [P, P, C.c_size_t]
        L.orc_philox4x32_10.argtypes = [P, P, P]
        L.orc_logdef.restype = C.c_float
        L.orc_logdef.argtypes = [C.c_float]
        L.orc_logdef_n.argtypes = [P, P, C.c_size_t]
        L.orc_gumbel_noise.restype = C.c_float
        L.orc_gumbel_noise.argtypes = [C.c_uint64, C.c_int32, C.c_int32]
        L.orc_sample_gumbel.restype = C.c_int32
        L.orc_sample_gumbel.argtypes = [P, C.c_int32, C.c_float, C.c_uint64, C.c_int32]
        L.orc_sample.restype = C.c_int32
        L.orc_sample.argtypes = [P, C.c_int32, C.c_float, C.c_float, C.c_uint64, C.c_int32]
        L.orc_sample_detail.restype = C.c_int32
        L.orc_sample_detail.argtypes = [P, C.c_int32, C.c_float, C.c_float, C.c_uint64, C.c_int32,
                                        P, P, P, P, P, P]
        L.orc_generate.argtypes = [P, P, P, P, C.c_int32, C.c_int32, C.c_int32, C.c_float,
                                   C.c_float, C.c_uint64, P, P]
        L.orc_set_threads.argtypes = [C.c_int32]
        L.orc_get_threads.restype = C.c_int32
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


# ---------------------------------------------------------------- building blocks

def f16_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().orc_f16_to_f32_n(_p(h), _p(out), h.size)
    return out


def f32_to_f16(f: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, dtype=np.uint16)
    lib().orc_f32_to_f16_n(_p(f), _p(out), f.size)
    return out


def gemv(W: np.ndarray, x: np.ndarray) -> np.ndarray:
    W = np.ascontiguousarray(W, dtype=np.float16)
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(W.shape[0], dtype=np.float32)
    lib().orc_gemv(_p(W), _p(x), W.shape[0], W.shape[1], _p(y))
    return y


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    g = np.ascontiguousarray(g, dtype=np.float16)
    y = np.empty_like(x)
    lib().orc_rmsnorm(_p(x), _p(g), x.size, eps, _p(y))
    return y


def rope(v: np.ndarray, pos: int, base: float = 10000.0) -> np.ndarray:
    v = np.array(v, dtype=np.float32, copy=True)
    lib().orc_rope(_p(v), v.size, pos, base)
    return v


def attention(q: np.ndarray, kc: np.ndarray, vc: np.ndarray, pos: int, window: int = 0) -> np.ndarray:
    """q [Hq][dh] fp32; kc, vc [max_seq][Hkv][dh] fp16 (one layer); window > 0: the last
    `window` positions only."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    kc = np.ascontiguousarray(kc, dtype=np.float16)
    vc = np.ascontiguousarray(vc, dtype=np.float16)
    hq, dh = q.shape
    hkv = kc.shape[1]
    o = np.empty_like(q)
    lib().orc_attention(_p(q), _p(kc), _p(vc), pos, hq, hkv, dh, window, _p(o))
    return o


def silu(z: float) -> float:
    return lib().orc_silu(float(z))


def argmax(logits: np.ndarray) -> int:
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    return lib().orc_argmax(_p(logits), logits.size)


def expdef(x) -> np.ndarray:
    x = np.ascontiguousarray(np.atleast_1d(np.asarray(x, dtype=np.float32)))
    y = np.empty_like(x)
    lib().orc_expdef_n(_p(x), _p(y), x.size)
    return y


def expdef_constants() -> np.ndarray:
    out = np.zeros(11, dtype=np.float32)
    lib().orc_expdef_constants(_p(out))
    return out


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def logdef(x) -> np.ndarray:
    x = np.ascontiguousarray(np.atleast_1d(np.asarray(x, dtype=np.float32)))
    y = np.empty_like(x)
    lib().orc_logdef_n(_p(x), _p(y), x.size)
    return y


def gumbel_noise(seed: int, pos: int, i: int) -> float:
    return lib().orc_gumbel_noise(seed, pos, i)


def sample_gumbel(logits: np.ndarray, temperature: float, seed: int, pos: int) -> int:
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    return lib().orc_sample_gumbel(_p(logits), logits.size, temperature, seed, pos)


def sample(logits: np.ndarray, temperature: float, top_p: float, seed: int, pos: int) -> int:
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    return lib().orc_sample(_p(logits), logits.size, temperature, top_p, seed, pos)


def sample_detail(logits: np.ndarray, temperature: float, top_p: float, seed: int, pos: int) -> dict:
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    n = logits.size
    q = np.zeros(n, dtype=np.uint64)
    K = np.zeros(1, dtype=np.int32)
    cv = np.zeros(1, dtype=np.uint64)
    cn = np.zeros(1, dtype=np.uint64)
    t = np.zeros(1, dtype=np.uint64)
    inn = np.zeros(n, dtype=np.uint8)
    tok = lib().orc_sample_detail(_p(logits), n, temperature, top_p, seed, pos, _p(q), _p(K),
                                  _p(cv), _p(cn), _p(t), _p(inn))
    return dict(token=tok, q=q, nucleus_size=int(K[0]), c_v=int(cv[0]), c_n=int(cn[0]),
                t=int(t[0]), in_nucleus=inn.astype(bool))


# ---------------------------------------------------------------- the decoder

def _cfg_struct(cfg: dict) -> OrcConfig:
    return OrcConfig(cfg["n_layers"], cfg["d_model"], cfg["n_heads"], cfg["n_kv_heads"],
                     cfg["head_dim"], cfg["ffn_dim"], cfg.get("vocab", 0), cfg["max_seq"],
                     cfg.get("rms_eps", 1e-5), cfg.get("rope_base", 10000.0),
                     cfg.get("sliding_window", 0), 0, cfg.get("window_layers", 0))


class Model:
    """The oracle decoder over host fp16 weights, with its own fp16 KV cache."""

    def __init__(self, cfg: dict, weights: dict):
        self.cfg = dict(cfg)
        self.w = weights
        self._keep = []
        L = cfg["n_layers"]
        self._layers = (OrcLayer * L)()
        for i, lw in enumerate(weights["layers"]):
            vals = []
            for n in _LAYER_NAMES:
                a = np.ascontiguousarray(lw[n], dtype=np.float16)
                self._keep.append(a)
                vals.append(_p(a))
            self._layers[i] = OrcLayer(*vals)

        def ptr(name):
            a = weights.get(name)
            if a is None:
                return None
            a = np.ascontiguousarray(a, dtype=np.float16)
            self._keep.append(a)
            return _p(a)

        self._w = OrcWeights(ptr("tok_emb"), ptr("final_norm"), ptr("lm_head"), self._layers)
        self._c = _cfg_struct(cfg)
        shp = (L, cfg["max_seq"], cfg["n_kv_heads"], cfg["head_dim"])
        self.kcache = np.zeros(shp, dtype=np.float16)
        self.vcache = np.zeros(shp, dtype=np.float16)

    def kv_fill(self, k: np.ndarray, v: np.ndarray, pos0: int = 0) -> None:
        n = k.shape[1]
        self.kcache[:, pos0:pos0 + n] = k
        self.vcache[:, pos0:pos0 + n] = v

    def decode_step(self, token: int, pos: int) -> np.ndarray:
        logits = np.empty(self.cfg["vocab"], dtype=np.float32)
        rc = lib().orc_decode_step(C.byref(self._c), C.byref(self._w), _p(self.kcache),
                                   _p(self.vcache), int(token), int(pos), _p(logits))
        if rc:
            raise ValueError(f"orc_decode_step failed ({rc})")
        return logits

    def layer_forward(self, layer: int, x: np.ndarray, pos: int) -> np.ndarray:
        x = np.array(x, dtype=np.float32, copy=True)
        rc = lib().orc_layer_forward(C.byref(self._c), C.byref(self._layers[layer]),
                                     _p(self.kcache[layer]), _p(self.vcache[layer]), _p(x), int(pos),
                                     int(layer))
        if rc:
            raise ValueError(f"orc_layer_forward failed ({rc})")
        return x

    def forward_nocache(self, tokens) -> np.ndarray:
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        logits = np.empty(self.cfg["vocab"], dtype=np.float32)
        rc = lib().orc_forward_nocache(C.byref(self._c), C.byref(self._w), _p(t), t.size, _p(logits))
        if rc:
            raise ValueError(f"orc_forward_nocache failed ({rc})")
        return logits

    def generate(self, token: int, pos: int, n: int, temperature: float = 0.0, top_p: float = 1.0,
                 seed: int = 1234, keep_logits: bool = False):
        out = np.zeros(n, dtype=np.int32)
        hist = np.zeros((n, self.cfg["vocab"]), dtype=np.float32) if keep_logits else None
        rc = lib().orc_generate(C.byref(self._c), C.byref(self._w), _p(self.kcache), _p(self.vcache),
                                int(token), int(pos), int(n), temperature, top_p, seed, _p(out),
                                _p(hist) if hist is not None else None)
        if rc:
            raise ValueError(f"orc_generate failed ({rc})")
        return (out, hist) if keep_logits else out
