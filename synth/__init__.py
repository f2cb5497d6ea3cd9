"""Seeded synthetic inputs for the batch-1 decode workloads.

This module only draws random numbers and lays them out as host arrays.  It
holds none of the decoder's arithmetic, imports nothing from the product
package or from the oracle, and is the one place both sides take their inputs
from, so the GPU path and the CPU oracle always see the same bytes.

Recipe (every tensor is independent of every other tensor):
  * a tensor is split into chunks of ``CHUNK`` elements; chunk ``c`` of tensor
    number ``tid`` under base seed ``s`` is drawn from
    ``numpy.random.Generator(numpy.random.Philox(SeedSequence([s, tid, c])))``
    as float32 ``standard_normal`` values;
  * matrices and the embedding are ``0.02 * N(0, 1)`` rounded to fp16 (RNE);
  * RMSNorm gains are exactly 1.0 (only matrices and embeddings are random);
  * prompt tokens are uniform integers in ``[0, vocab)`` (seed 1);
  * prefilled K/V cache entries are ``N(0, 1)`` rounded to fp16 (seed 2);
  * the single-layer hidden input is ``N(0, 1)`` in fp32 (seed 3);
  * weights use seed 0.

Shapes follow the Llama-style boundary layout: every matrix is row-major
``[out][in]`` fp16, ``wq`` rows are head-major (row ``h*head_dim + j``).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

CHUNK = 1 << 22
SEED_WEIGHTS, SEED_PROMPT, SEED_KV, SEED_HIDDEN, SEED_SAMPLER = 0, 1, 2, 3, 1234

# Workload presets.  Names describe the workload; sizes are the full ones.
CONFIGS = {
    # tiny decoder, checkable on a CPU in seconds
    "tiny_2l_d256": dict(n_layers=2, d_model=256, n_heads=4, n_kv_heads=4, head_dim=64,
                         ffn_dim=1024, vocab=4096, max_seq=64,
                         prompt_len=8, n_decode=32, temperature=0.0, top_p=1.0),
    # one decoder layer at the 2B-class shape, hidden vector in / out, KV prefilled to 1024
    "layer_d2560_kv1024": dict(n_layers=1, d_model=2560, n_heads=20, n_kv_heads=20, head_dim=128,
                               ffn_dim=6912, vocab=0, max_seq=1040,
                               kv_prefill=1024, temperature=0.0, top_p=1.0),
    # ~2.2B decoder: 25 such layers, untied 32768-token vocabulary, greedy
    "dec2b_25l_greedy": dict(n_layers=25, d_model=2560, n_heads=20, n_kv_heads=20, head_dim=128,
                             ffn_dim=6912, vocab=32768, max_seq=384,
                             prompt_len=128, n_decode=256, temperature=0.0, top_p=1.0),
    # the same model at 16K context with temperature / top-p sampling
    "dec2b_25l_kv16k_topp": dict(n_layers=25, d_model=2560, n_heads=20, n_kv_heads=20, head_dim=128,
                                 ffn_dim=6912, vocab=32768, max_seq=16512,
                                 kv_prefill=16384, n_decode=128, temperature=0.8, top_p=0.9),
    # LaneFormer-2B-shaped decoder: 15 layers, GQA 32 query / 16 KV heads of dim 96,
    # sliding window in 10 of the 15 layers (every third layer attends globally),
    # 4096-token context; d_model, ffn_dim, window and vocabulary are readings
    "laneformer_15l_swa": dict(n_layers=15, d_model=3072, n_heads=32, n_kv_heads=16, head_dim=96,
                               ffn_dim=12288, vocab=32000, max_seq=4096, sliding_window=1024,
                               window_layers=sum(1 << l for l in range(15) if l % 3 != 2),
                               kv_prefill=2048, n_decode=128, temperature=0.0, top_p=1.0),
    # ~8B dense GQA decoder
    "dec8b_32l_gqa": dict(n_layers=32, d_model=4096, n_heads=32, n_kv_heads=8, head_dim=128,
                          ffn_dim=14336, vocab=128256, max_seq=768,
                          prompt_len=256, n_decode=512, temperature=0.0, top_p=1.0),
}
for _cfg in CONFIGS.values():
    _cfg.setdefault("rms_eps", 1e-5)
    _cfg.setdefault("rope_base", 10000.0)
    _cfg.setdefault("seed", SEED_SAMPLER)

LAYER_TENSORS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_f32(n: int, seed: int, tid: int, scale: float = 1.0) -> np.ndarray:
    """``n`` float32 draws ``scale * N(0,1)`` for tensor number ``tid`` (chunked recipe)."""
    out = np.empty(n, dtype=np.float32)

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        rng = np.random.Generator(np.random.Philox(np.random.SeedSequence([seed, tid, c])))
        blk = rng.standard_normal(hi - lo, dtype=np.float32)
        if scale != 1.0:
            blk *= np.float32(scale)
        out[lo:hi] = blk

    nchunks = (n + CHUNK - 1) // CHUNK
    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def normal_f16(shape, seed: int, tid: int, scale: float) -> np.ndarray:
    n = int(np.prod(shape))
    return normal_f32(n, seed, tid, scale).astype(np.float16).reshape(shape)


def layer_shapes(cfg: dict) -> dict:
    d, hq, hkv, dh, f = cfg["d_model"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["ffn_dim"]
    return dict(attn_norm=(d,), wq=(hq * dh, d), wk=(hkv * dh, d), wv=(hkv * dh, d),
                wo=(d, hq * dh), ffn_norm=(d,), w_gate=(f, d), w_up=(f, d), w_down=(d, f))


def model_weights(cfg: dict, seed: int = SEED_WEIGHTS, scale: float = 0.02) -> dict:
    """All weights of a config as host fp16 arrays.

    Returns ``{"tok_emb", "final_norm", "lm_head", "layers": [ {name: array} ]}``;
    the three top-level entries are ``None`` when ``vocab == 0`` (single-layer
    hidden-vector workload).
    """
    d, v = cfg["d_model"], cfg["vocab"]
    shapes = layer_shapes(cfg)
    layers = []
    tid = 0
    for _ in range(cfg["n_layers"]):
        lw = {}
        for name in LAYER_TENSORS:
            shp = shapes[name]
            if name.endswith("_norm"):
                lw[name] = np.ones(shp, dtype=np.float16)
            else:
                lw[name] = normal_f16(shp, seed, tid, scale)
            tid += 1
        layers.append(lw)
    w = dict(layers=layers, tok_emb=None, final_norm=None, lm_head=None)
    if v > 0:
        w["tok_emb"] = normal_f16((v, d), seed, 100000, scale)
        w["lm_head"] = normal_f16((v, d), seed, 100001, scale)
        w["final_norm"] = np.ones((d,), dtype=np.float16)
    return w


def prompt(cfg: dict, n: int | None = None, seed: int = SEED_PROMPT) -> np.ndarray:
    n = cfg.get("prompt_len", 1) if n is None else n
    rng = np.random.Generator(np.random.Philox(np.random.SeedSequence([seed, 0])))
    return rng.integers(0, cfg["vocab"], size=n, dtype=np.int64).astype(np.int32)


def kv_prefill(cfg: dict, n_pos: int, seed: int = SEED_KV, layers=None) -> tuple[np.ndarray, np.ndarray]:
    """Prefilled cache contents ``[L][n_pos][n_kv_heads][head_dim]`` fp16 for K and for V."""
    L = cfg["n_layers"] if layers is None else layers
    shp = (L, n_pos, cfg["n_kv_heads"], cfg["head_dim"])
    k = np.empty(shp, dtype=np.float16)
    v = np.empty(shp, dtype=np.float16)
    per = int(np.prod(shp[1:]))
    for l in range(L):
        k[l] = normal_f32(per, seed, 2 * l, 1.0).astype(np.float16).reshape(shp[1:])
        v[l] = normal_f32(per, seed, 2 * l + 1, 1.0).astype(np.float16).reshape(shp[1:])
    return k, v


def hidden(cfg: dict, seed: int = SEED_HIDDEN) -> np.ndarray:
    return normal_f32(cfg["d_model"], seed, 0, 1.0)


def scaled_config(name: str, **overrides) -> dict:
    """A copy of a preset with some fields replaced (used for small parity cases)."""
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    return cfg
