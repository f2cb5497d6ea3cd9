"""Algorithmic byte / flop model of one batch-1 decode step, and the ceilings it implies.

Batch-1 decode reads every active weight once per token and does about one
multiply-add per weight, so its floor is memory traffic: tokens/s <= B / (P*b)
for P parameters of b bytes at bandwidth B ("KOG LaneFormer-2B & the
monokernel", sections "A worked bandwidth ceiling" and "Technical takeaways").

Bytes counted per token at position ``pos`` (algorithmic, not measured):
  * every layer matrix and RMSNorm gain, the final gain and the lm_head (fp16);
  * one embedding row (the table is gathered, not streamed);
  * K and V of positions 0..pos for every layer (attention reads them all,
    the current one included; a sliding-window layer reads the last W only),
    and the K/V row written at ``pos``.
Activations (a few KB per phase, cache resident) are not counted.
"""
from __future__ import annotations

HBM_PEAK_BYTES_PER_S = 8.0e12        # MI355X published HBM3E peak
FP16 = 2


def qkv_rows(n_heads: int, n_kv_heads: int, head_dim: int) -> int:
    return (n_heads + 2 * n_kv_heads) * head_dim


def layer_weight_elems(cfg: dict) -> int:
    d, hq, hkv, dh, f = cfg["d_model"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["ffn_dim"]
    return qkv_rows(hq, hkv, dh) * d + d * hq * dh + 3 * d * f + 2 * d


def weight_bytes(cfg: dict) -> int:
    """Weights streamed per token: all layers, final gain and lm_head, plus one embedding row."""
    d, v = cfg["d_model"], cfg.get("vocab", 0)
    elems = cfg["n_layers"] * layer_weight_elems(cfg)
    if v > 0:
        elems += v * d + d + d      # lm_head, final gain, gathered embedding row
    return FP16 * elems


def kv_bytes(cfg: dict, pos: int) -> int:
    """K/V read over positions 0..pos (the last ``sliding_window`` of them in the
    layers of ``window_layers``) plus the row written at pos, all layers."""
    row = cfg["n_kv_heads"] * cfg["head_dim"] * FP16
    W, mask = cfg.get("sliding_window", 0), cfg.get("window_layers", 0)
    rows = 0
    for l in range(cfg["n_layers"]):
        keys = min(pos + 1, W) if W > 0 and l < 64 and (mask >> l) & 1 else pos + 1
        rows += keys + 1
    return 2 * row * rows


def bytes_per_token(cfg: dict, pos: int) -> int:
    return weight_bytes(cfg) + kv_bytes(cfg, pos)


def bytes_for_steps(cfg: dict, pos0: int, n: int) -> int:
    return sum(bytes_per_token(cfg, pos0 + i) for i in range(n))


def flops_per_token(cfg: dict, pos: int) -> int:
    d, hq, dh, v = cfg["d_model"], cfg["n_heads"], cfg["head_dim"], cfg.get("vocab", 0)
    gemv = cfg["n_layers"] * (layer_weight_elems(cfg) - 2 * d) + v * d
    return 2 * gemv + 4 * cfg["n_layers"] * hq * dh * (pos + 1)


# ---- the pages' own arithmetic (context figures, reproduced as checks) ----

def weight_only_ceiling_tok_s(params: float, bytes_per_param: float, bandwidth_bytes_per_s: float) -> float:
    """P*b/B floor per token, inverted: tokens/s <= B / (P*b)."""
    return bandwidth_bytes_per_s / (params * bytes_per_param)


def launch_bound_tok_s(overhead_us_per_token: float) -> float:
    """Tokens/s if per-token launch overhead were the only cost."""
    return 1e6 / overhead_us_per_token
