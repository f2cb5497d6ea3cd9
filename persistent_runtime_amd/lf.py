"""Python binding of ``liblf.so`` (the C ABI in ``include/lf.h``).

Argument marshalling only: every step of the decode path runs in the HIP
library.  torch provides device memory and the stream; nothing here computes.
The native library is required: importing this module on a machine where
``liblf.so`` has not been built raises, there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# LF_LIB selects another build of the same library (e.g. one compiled with a
# different LDS ring depth); by default the in-tree build is used.
LIB_PATH = os.environ.get("LF_LIB") or os.path.join(HERE, "liblf.so")

LF_OK, LF_EINVAL, LF_ENOMEM, LF_EHIP, LF_ERANGE, LF_ETIMEOUT, LF_EUNSUPPORTED = 0, -1, -2, -3, -4, -5, -6
LF_HIDDEN_IO, LF_STATS, LF_GUMBEL = 1, 4, 8
LF_Q_GRID, LF_Q_THREADS, LF_Q_LDS_BYTES, LF_Q_SCRATCH_BYTES, LF_Q_SCRATCH_MAX = 0, 1, 2, 3, 4
LF_Q_KV_PF, LF_Q_GU_PF, LF_Q_WAVE_W, LF_Q_WAVE_W_KINDS, LF_Q_PF_KIND = 5, 6, 7, 14, 15
LAYER_NAMES = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")

# every symbol include/lf.h declares
EXPORTS = ("lf_model_create", "lf_model_destroy", "lf_decode_step", "lf_generate", "lf_generate_noalloc",
           "lf_prefill", "lf_set_position",
           "lf_last_error", "lf_get_logits", "lf_kv_fill", "lf_kv_read", "lf_set_hidden", "lf_get_hidden",
           "lf_get_stats", "lf_query", "lf_test_expdef", "lf_test_sample",
           "lf_test_logdef", "lf_test_sample_gumbel")


class LfError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"liblf error {code}: {msg}")
        self.code = code


class LfConfig(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_layers", "d_model", "n_heads", "n_kv_heads", "head_dim",
                                         "ffn_dim", "vocab", "max_seq")] + \
               [("rms_eps", C.c_float), ("rope_base", C.c_float), ("temperature", C.c_float),
                ("top_p", C.c_float), ("seed", C.c_uint64), ("flags", C.c_uint32),
                ("sliding_window", C.c_int32), ("window_layers", C.c_uint64)]


class LfLayerWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in LAYER_NAMES]


class LfWeights(C.Structure):
    _fields_ = [("tok_emb", C.c_void_p), ("final_norm", C.c_void_p), ("lm_head", C.c_void_p),
                ("layers", C.POINTER(LfLayerWeights))]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with persistent_runtime_amd/build.py "
                              "(the HIP library is required; there is no fallback)")
        L = C.CDLL(LIB_PATH)
        P, I32, U64 = C.c_void_p, C.c_int32, C.c_uint64
        L.lf_model_create.argtypes = [C.POINTER(LfConfig), C.POINTER(LfWeights), P, C.POINTER(P)]
        L.lf_model_destroy.argtypes = [P]
        L.lf_model_destroy.restype = None
        L.lf_decode_step.argtypes = [P, I32, I32, C.POINTER(I32)]
        L.lf_generate.argtypes = [P, I32, P]
        L.lf_generate_noalloc.argtypes = [P, I32, P]
        L.lf_set_position.argtypes = [P, I32, I32]
        L.lf_prefill.argtypes = [P, P, I32, I32]
        L.lf_last_error.argtypes = [P]
        L.lf_last_error.restype = C.c_char_p
        L.lf_get_logits.argtypes = [P, P, C.c_int]
        L.lf_kv_fill.argtypes = [P, I32, I32, I32, P, P]
        L.lf_kv_read.argtypes = [P, I32, I32, I32, P, P]
        L.lf_set_hidden.argtypes = [P, P]
        L.lf_get_hidden.argtypes = [P, P]
        L.lf_get_stats.argtypes = [P, P, C.c_size_t]
        L.lf_query.argtypes = [P, I32]
        L.lf_test_expdef.argtypes = [P, P, C.c_int64, P]
        L.lf_test_sample.argtypes = [P, I32, C.c_float, C.c_float, U64, P, I32, P, P]
        L.lf_test_logdef.argtypes = [P, P, C.c_int64, P]
        L.lf_test_sample_gumbel.argtypes = [P, I32, C.c_float, U64, P, I32, P, P]
        _lib = L
    return _lib


def _check(rc: int, st=None) -> None:
    if rc != LF_OK:
        msg = lib().lf_last_error(st)
        raise LfError(rc, msg.decode() if msg else "")


def _stream_handle(stream) -> int | None:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def make_config(cfg: dict, flags: int = 0) -> LfConfig:
    return LfConfig(cfg["n_layers"], cfg["d_model"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"],
                    cfg["ffn_dim"], cfg.get("vocab", 0), cfg["max_seq"], cfg.get("rms_eps", 1e-5),
                    cfg.get("rope_base", 10000.0), cfg.get("temperature", 0.0), cfg.get("top_p", 1.0),
                    cfg.get("seed", 1234), flags | (LF_HIDDEN_IO if cfg.get("vocab", 0) == 0 else 0)
                    | (LF_GUMBEL if cfg.get("sampler", "nucleus") == "gumbel" else 0),
                    cfg.get("sliding_window", 0), cfg.get("window_layers", 0))


def upload_weights(weights: dict, device="cuda") -> dict:
    """Host fp16 numpy weights -> torch device tensors (same structure)."""
    import torch

    def up(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device)

    return dict(tok_emb=up(weights.get("tok_emb")), final_norm=up(weights.get("final_norm")),
                lm_head=up(weights.get("lm_head")),
                layers=[{k: up(v) for k, v in lw.items()} for lw in weights["layers"]])


class Engine:
    """One decode state (``lf_state``): packed weights, KV cache, activations."""

    def __init__(self, cfg: dict, dev_weights: dict, flags: int = 0, stream=None):
        import torch
        self.cfg = dict(cfg)
        self._stream = stream
        self._c = make_config(cfg, flags)
        L = cfg["n_layers"]
        layers = (LfLayerWeights * L)()
        for i, lw in enumerate(dev_weights["layers"]):
            for n in LAYER_NAMES:
                t = lw[n]
                assert t.is_cuda and t.dtype == torch.float16 and t.is_contiguous(), n
                setattr(layers[i], n, t.data_ptr())

        def ptr(name):
            t = dev_weights.get(name)
            return None if t is None else t.data_ptr()

        w = LfWeights(ptr("tok_emb"), ptr("final_norm"), ptr("lm_head"), layers)
        st = C.c_void_p()
        _check(lib().lf_model_create(C.byref(self._c), C.byref(w), _stream_handle(stream), C.byref(st)))
        self._st = st
        self.grid = lib().lf_query(st, LF_Q_GRID)
        self.lds_bytes = lib().lf_query(st, LF_Q_LDS_BYTES)

    def close(self) -> None:
        if getattr(self, "_st", None):
            lib().lf_model_destroy(self._st)
            self._st = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def decode_step(self, token: int, pos: int) -> int:
        nxt = C.c_int32(-1)
        _check(lib().lf_decode_step(self._st, int(token), int(pos), C.byref(nxt)), self._st)
        return nxt.value

    def prefill(self, tokens, pos0: int = 0) -> None:
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        _check(lib().lf_prefill(self._st, t.ctypes.data, t.size, int(pos0)), self._st)

    def set_position(self, token: int, pos: int) -> None:
        _check(lib().lf_set_position(self._st, int(token), int(pos)), self._st)

    def generate(self, n: int) -> np.ndarray:
        out = np.zeros(n, dtype=np.int32)
        _check(lib().lf_generate(self._st, int(n), out.ctypes.data), self._st)
        return out

    def generate_noalloc(self, n: int, out=None):
        """lf_generate_noalloc: tokens into a caller-owned int32 device tensor (allocated
        here, on the caller's side, when `out` is None)."""
        import torch
        if out is None:
            out = torch.empty(n, dtype=torch.int32, device="cuda")
        assert out.is_cuda and out.dtype == torch.int32 and out.is_contiguous() and out.numel() >= n
        _check(lib().lf_generate_noalloc(self._st, int(n), out.data_ptr()), self._st)
        return out

    def query(self, what: int) -> int:
        return lib().lf_query(self._st, int(what))

    def logits(self):
        import torch
        t = torch.empty(self.cfg["vocab"], dtype=torch.float32, device="cuda")
        _check(lib().lf_get_logits(self._st, t.data_ptr(), 1), self._st)
        return t

    def kv_fill(self, layer: int, pos0: int, k, v) -> None:
        assert k.is_cuda and v.is_cuda and k.is_contiguous() and v.is_contiguous()
        _check(lib().lf_kv_fill(self._st, layer, pos0, k.shape[0], k.data_ptr(), v.data_ptr()), self._st)

    def kv_read(self, layer: int, pos0: int, n: int):
        import torch
        shp = (n, self.cfg["n_kv_heads"], self.cfg["head_dim"])
        k = torch.empty(shp, dtype=torch.float16, device="cuda")
        v = torch.empty(shp, dtype=torch.float16, device="cuda")
        _check(lib().lf_kv_read(self._st, layer, pos0, n, k.data_ptr(), v.data_ptr()), self._st)
        return k, v

    def set_hidden(self, x) -> None:
        _check(lib().lf_set_hidden(self._st, x.data_ptr()), self._st)

    def get_hidden(self):
        import torch
        x = torch.empty(self.cfg["d_model"], dtype=torch.float32, device="cuda")
        _check(lib().lf_get_hidden(self._st, x.data_ptr()), self._st)
        return x

    def stats(self) -> np.ndarray:
        out = np.zeros((self.grid, 16), dtype=np.uint64)
        _check(lib().lf_get_stats(self._st, out.ctypes.data, out.nbytes), self._st)
        return out


def test_expdef(x):
    """Defined exponential on the GPU (test hook); x: fp32 cuda tensor."""
    import torch
    y = torch.empty_like(x)
    _check(lib().lf_test_expdef(x.data_ptr(), y.data_ptr(), x.numel(), _stream_handle(None)))
    return y


def test_sample(logits, temperature: float, top_p: float, seed: int, pos):
    """In-kernel nucleus sampler on m cases (test hook): logits [m, n] fp32 cuda, pos [m] int32 cuda."""
    import torch
    m, n = logits.shape
    tokens = torch.empty(m, dtype=torch.int32, device=logits.device)
    _check(lib().lf_test_sample(logits.data_ptr(), n, temperature, top_p, seed, pos.data_ptr(), m,
                                tokens.data_ptr(), _stream_handle(None)))
    return tokens


def test_logdef(x):
    """Defined natural logarithm on the GPU (test hook); x: positive fp32 cuda tensor."""
    import torch
    y = torch.empty_like(x)
    _check(lib().lf_test_logdef(x.data_ptr(), y.data_ptr(), x.numel(), _stream_handle(None)))
    return y


def test_sample_gumbel(logits, temperature: float, seed: int, pos):
    """In-kernel Gumbel-max choice on m cases (test hook): logits [m, n] fp32 cuda, pos [m] int32 cuda."""
    import torch
    m, n = logits.shape
    tokens = torch.empty(m, dtype=torch.int32, device=logits.device)
    _check(lib().lf_test_sample_gumbel(logits.data_ptr(), n, temperature, seed, pos.data_ptr(), m,
                                       tokens.data_ptr(), _stream_handle(None)))
    return tokens
