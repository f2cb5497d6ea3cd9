"""Per-phase timeline of one decode token, from the LF_TRACE build of the library.

    python3 persistent_runtime_amd/build.py --trace
    LF_LIB=persistent_runtime_amd/liblf_trace.so python3 -m persistent_runtime_amd.phase_trace \\
        dec2b_25l_greedy 16 12

decodes N tokens of a synthetic workload (after its teacher-forced prompt or
its synthetic cache), twice, and prints for one layer of the middle token the
median and maximum over the workgroups of each timestamp the kernel took,
in microseconds from the median start of that layer's QKV staging, and per
exchange the producers' last publish, the consumers' first poll back and their
poll round trips.  Diagnostics only: it needs the trace build."""
from __future__ import annotations

import os
import sys

import numpy as np

from . import lf

PHASES = {0: "QKV", 1: "attention", 2: "output projection", 3: "gate/up", 4: "down"}
SYNC = {6: "staging started", 7: "tagged input in", 0: "input staged", 1: "stream waves done", 2: "published"}
WAVE1 = {3: "input seen", 5: "done"}
ATT = {8: "unit entered", 6: "unit start", 2: "first tile issue starts", 0: "first tile requested", 1: "queries polled (last wave)", 3: "queries staged",
       10: "first scores", 4: "keys done", 9: "waves' states in LDS", 5: "partial stored",
       11: "merge start", 12: "folded", 13: "merged"}


def run(workload: str, n: int):
    import torch

    import synth
    if "trace" not in os.path.basename(lf.LIB_PATH):
        raise SystemExit("load the LF_TRACE build: LF_LIB=persistent_runtime_amd/liblf_trace.so")
    cfg = dict(synth.CONFIGS[workload])
    kv = "prompt_len" not in cfg
    P = cfg["kv_prefill"] if kv else cfg["prompt_len"]
    pos0 = P if kv else P - 1
    cfg["max_seq"] = max(cfg["max_seq"], pos0 + n + 1)
    eng = lf.Engine(cfg, lf.upload_weights(synth.model_weights(cfg)))
    if kv:
        k, v = synth.kv_prefill(cfg, P)
        for l in range(cfg["n_layers"]):
            eng.kv_fill(l, 0, torch.from_numpy(k[l]).cuda(), torch.from_numpy(v[l]).cuda())
        first = int(synth.prompt(dict(cfg, prompt_len=1), 1)[0])
    else:
        pr = synth.prompt(cfg, P)
        eng.prefill(pr[:pos0], 0)
        first = int(pr[pos0])
    for _ in range(2):
        eng.set_position(first, pos0)
        eng.generate(n)
    G, L = eng.grid, cfg["n_layers"]
    nslot = 5 * L + 2
    buf = np.zeros((G, 16 + 16 * nslot), np.uint64)
    rc = lf.lib().lf_get_stats(eng._st, buf.ctypes.data, buf.nbytes)
    if rc != 0:
        raise SystemExit(f"lf_get_stats failed ({rc})")
    eng.close()
    return buf[:, 16:].reshape(G, nslot, 16).astype(np.int64), L


def report(tr: np.ndarray, l: int) -> None:
    base = tr[:, 5 * l, 6]
    t0 = np.median(base[base > 0])

    def row(name, v):
        v = v[v > 0]
        if len(v):
            d = (v - t0) / 100.0
            print(f"    {name:28s} n={len(v):3d} median {np.median(d):7.2f} max {d.max():7.2f}")

    print(f"layer {l}: us from the median start of its QKV staging")
    for k, name in PHASES.items():
        s = 5 * l + k
        print(f"  {name}")
        for j, nm in (ATT if k == 1 else SYNC).items():
            row(("" if k == 1 else "sync wave: ") + nm, tr[:, s, j])
        if k != 1:
            for j, nm in WAVE1.items():
                row("stream wave 1: " + nm, tr[:, s, j])
    nb = tr[:, 5 * (l + 1), 6]
    if (nb > 0).any():
        print(f"  next layer's QKV staging starts: median {(np.median(nb[nb > 0]) - t0) / 100.0:.2f}")
    print("  exchanges (sync wave): producers' last publish -> first poll back -> tagged input in; poll round trips")
    prev = {0: (5 * (l - 1) + 4, 2), 2: (5 * l + 1, 5), 3: (5 * l + 2, 2), 4: (5 * l + 3, 2)}
    for k, (ps, pj) in prev.items():
        if ps < 0:
            continue
        s = 5 * l + k
        pub = tr[:, ps, pj]
        pub = pub[pub > 0]
        first, tin, polls = tr[:, s, 8], tr[:, s, 7], tr[:, s, 9]
        ok = (first > 0) & (tin > 0)
        if not len(pub) or not ok.any():
            continue
        print(f"    {PHASES[k]:18s} last publish {(pub.max() - t0) / 100:7.2f}  first poll back "
              f"{(np.median(first[ok]) - t0) / 100:7.2f}  input in {(np.median(tin[ok]) - t0) / 100:7.2f}  "
              f"round trips median {np.median(polls[ok]):.0f} max {polls[ok].max():.0f}")


def main() -> int:
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    if len(sys.argv) < 3:
        print(__doc__)
        return 2
    workload, n = sys.argv[1], int(sys.argv[2])
    tr, L = run(workload, n)
    layer = int(sys.argv[3]) if len(sys.argv) > 3 else L // 2
    print(f"{workload}: {n} tokens, token {n // 2} traced")
    report(tr, layer)
    return 0


if __name__ == "__main__":
    sys.exit(main())
