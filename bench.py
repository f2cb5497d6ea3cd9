"""Batch-1 decode benchmark on one MI355X: tokens/s and HBM-roofline fraction.

Workload (default ``dec2b_25l_greedy``): the synthetic ~2.2B fp16 decoder (25
layers, d 2560, 20 heads x 128, SwiGLU 6912, vocab 32768 untied, weights
N(0, 0.02) from seed 0), a 128-token random prompt, greedy decode.  The prompt's
first 127 tokens go through one teacher-forced launch (timed on its own and
reported as ``prompt``, never part of the decode rate); a step is one decoded
token.  The W warmup steps run as one more teacher-forced launch of the same
layer stack from the first decode position (so every dispatch of the decode
kernel is a timed one and a profiler's per-kernel average is their mean); then
R repetitions each reset the position to the first decode position and run
EXACTLY K steps in ONE lf_generate launch, timed with HIP events on the stream
the kernel is launched on, bracketed by device synchronisations.  ``value`` is
K / the median launch time.  Inputs are resident in HBM before timing starts.

Other workloads: ``dec2b_25l_kv16k_topp`` (16K prefilled cache, nucleus
sampling), ``dec8b_32l_gqa`` (~8B GQA), ``laneformer_15l_swa`` (sliding
windows), and ``layer_d2560_kv1024`` (one 2B-class layer step: the model is
``--rotate`` distinct copies of the layer run in one launch so that the weights
cannot stay in the 256 MB last-level cache; reported per layer).

Prints one JSON line.  ``roofline.achieved`` = algorithmic bytes of one launch
(every weight once per token, the KV rows read and written; see
persistent_runtime_amd/roofline.py) / the median launch duration.
``cpu_baseline`` is the CPU oracle timed on this host on a bounded sample of the
same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0
METRIC = "batch-1 decode tokens/s + % of HBM-bandwidth roofline (MBU), 1x MI355X"


def kernel_name(cfg: dict) -> str:
    """The decode kernel's instance: one per attention variant (query heads per
    KV head rounded up to 1, 2, 4 or 8)."""
    qpg = cfg["n_heads"] // cfg["n_kv_heads"]
    kq = 1 if qpg <= 1 else 2 if qpg == 2 else 4 if qpg <= 4 else 8
    return f"lf_monokernel<false, {kq}>"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("lf_kernel.hip", "lf_internal.h", "lf_api.cpp"):
        with open(os.path.join(ROOT, "persistent_runtime_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def host_threads() -> int:
    """Threads the host share allows: OMP_NUM_THREADS when set, else the CPUs this
    process may run on."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def host_info() -> dict:
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = None
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity_cpus": aff,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


# ---------------------------------------------------------------- workloads

def setup(workload: str, K: int, W: int, rotate: int):
    """(cfg, kind, P, pos0): kind 'prompt' decodes after a teacher-forced prompt
    of P tokens (from position P-1), 'kv' after a synthetic cache of P rows (from
    position P), 'hidden' runs one layer step per copy on a hidden vector."""
    import synth
    cfg = dict(synth.CONFIGS[workload])
    if cfg.get("vocab", 0) == 0:
        cfg["n_layers"] = rotate
        P = cfg["kv_prefill"]
        return cfg, "hidden", P, P
    if "prompt_len" in cfg:
        P = cfg["prompt_len"]
        pos0 = P - 1
        kind = "prompt"
    else:
        P = cfg["kv_prefill"]
        pos0 = P
        kind = "kv"
    cfg["max_seq"] = max(cfg["max_seq"], pos0 + max(K, W) + 1)
    return cfg, kind, P, pos0


def launch_bytes(cfg: dict, kind: str, pos0: int, K: int) -> int:
    from persistent_runtime_amd import roofline
    if kind == "hidden":
        return roofline.bytes_per_token(cfg, pos0)   # every layer copy once, no embedding / lm_head
    return roofline.bytes_for_steps(cfg, pos0, K)


# ---------------------------------------------------------------- HBM traffic from counters

def measured_traffic(workload: str, nbytes: int):
    """HBM bytes of one launch from the committed rocprofv3 counter record, if it
    was taken on the current kernel source and this workload: the counted bytes
    per algorithmic byte of the profiled launch, times this launch's algorithmic
    bytes (the ratio is a property of the kernel and the workload, not of the
    step count)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None, None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None, None
    if d.get("kernel_source_hash") != kernel_source_hash() or "measured_over_algorithmic" not in d:
        return None, None
    r = float(d["measured_over_algorithmic"])
    return int(round(r * nbytes)), d


def _counter_rows(path: str, counter: str):
    import csv
    import glob
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {path}")
    rows = []
    with open(files[0], newline="") as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    return sorted(rows)


def write_traffic(d: str, workload: str, K: int, W: int, rotate: int) -> int:
    """HBM bytes of the timed decode launches from counter runs of this command
    (DIR/fetch, DIR/write), each counter scaled by its reading for a device copy
    of 1 GiB (DIR/cfetch, DIR/cwrite: 1 GiB read, 1 GiB written)."""
    cfg, kind, _, pos0 = setup(workload, K, W, rotate)
    copy_bytes = 1 << 30
    cal = {}
    for c, sub in (("FETCH_SIZE", "cfetch"), ("WRITE_SIZE", "cwrite")):
        copies = [v for _, k, v in _counter_rows(os.path.join(d, sub), c) if "copyBuffer" in k]
        cal[c] = copy_bytes / max(copies)   # bytes per counted KiB
    got = {}
    kname = kernel_name(cfg)
    for c, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        mine = [v for _, k, v in _counter_rows(os.path.join(d, sub), c) if kname in k]
        if not mine:
            raise SystemExit(f"no {kname} dispatch in {sub}")
        got[c] = sum(mine) / len(mine)   # every decode dispatch is a timed repetition
    alg = launch_bytes(cfg, kind, pos0, K)
    rec = {"workload": workload, "steps": K, "kernel": kname, "kernel_source_hash": kernel_source_hash(),
           "dispatches": len(mine),
           "fetch_kib_counted": got["FETCH_SIZE"], "write_kib_counted": got["WRITE_SIZE"],
           "fetch_bytes_per_counted_kib": cal["FETCH_SIZE"], "write_bytes_per_counted_kib": cal["WRITE_SIZE"],
           "hbm_read_bytes_per_launch": int(got["FETCH_SIZE"] * cal["FETCH_SIZE"]),
           "hbm_write_bytes_per_launch": int(got["WRITE_SIZE"] * cal["WRITE_SIZE"]),
           "algorithmic_bytes_per_launch": alg}
    rec["hbm_bytes_per_launch"] = rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]
    rec["measured_over_algorithmic"] = rec["hbm_bytes_per_launch"] / alg
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    out = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))
    return 0


# ---------------------------------------------------------------- CPU oracle baseline

def cpu_baseline(cfg, weights, kind: str, P: int, pos0: int, seconds: float):
    """The oracle timed on this host's threads on a bounded sample of the workload:
    teacher-forced steps from position 0 for prompt workloads; for a prefilled
    cache, the same synthetic rows filled into the oracle's cache and steps from
    the first decode position; for the layer workload, single-layer steps."""
    import numpy as np

    import oracle
    import synth
    threads = host_threads()
    oracle.set_threads(threads)
    times = []
    t_start = time.perf_counter()
    if kind == "hidden":
        one = dict(cfg, n_layers=1)
        lw = dict(weights, layers=weights["layers"][:1])
        m = oracle.Model(one, lw)
        k, v = synth.kv_prefill(one, P)
        m.kv_fill(k, v, 0)
        x = synth.hidden(one)
        while True:
            t0 = time.perf_counter()
            m.layer_forward(0, x, pos0)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_start > seconds and len(times) >= 2:
                break
        per = sorted(times)[len(times) // 2]
        return {"value": round(per * 1e6, 1), "unit": "us per layer step", "cores": threads, "kind": "oracle",
                "sample": f"{len(times)} single-layer steps at position {pos0} over {P} cached rows, "
                          f"median {per * 1e3:.2f} ms", "host": host_info()}
    m = oracle.Model(cfg, weights)
    if kind == "kv":
        k, v = synth.kv_prefill(cfg, P)
        m.kv_fill(k, v, 0)
        del k, v
        tok = int(synth.prompt(dict(cfg, prompt_len=1), 1)[0])
        p = pos0
        while True:
            t0 = time.perf_counter()
            logits = m.decode_step(tok, p)
            times.append(time.perf_counter() - t0)
            tok, p = int(np.argmax(logits)), p + 1
            if time.perf_counter() - t_start > seconds and len(times) >= 2:
                break
        where = f"positions {pos0}..{p - 1} over the same {P}-row synthetic cache"
    else:
        prompt = synth.prompt(cfg, P)
        for pos, tok in enumerate(prompt):
            t0 = time.perf_counter()
            m.decode_step(int(tok), pos)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_start > seconds and len(times) >= 2:
                break
        where = f"positions 0..{len(times) - 1} (teacher-forced prompt tokens)"
    per = sorted(times)[len(times) // 2]
    return {"value": round(1.0 / per, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(times)} decode steps of the same model at {where}, median step {per * 1e3:.1f} ms",
            "host": host_info()}


# ---------------------------------------------------------------- timing

def time_launches(fn, reps: int, stream):
    import torch
    ms = []
    out = None
    for _ in range(reps):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        out = fn()
        ev1.record(stream)
        torch.cuda.synchronize()
        ms.append(ev0.elapsed_time(ev1))
    s = sorted(ms)
    return out, {"median": round(s[len(s) // 2], 4), "min": round(s[0], 4), "max": round(s[-1], 4),
                 "mean": round(sum(s) / len(s), 4), "reps": len(s), "all": [round(x, 4) for x in ms]}


def wait_stats(eng, steps: int) -> dict:
    import numpy as np
    s = eng.stats().astype(np.float64)
    tot = np.maximum(s[:, 3], 1)

    def frac(k):
        return round(float((s[:, k] / tot).mean()), 4)

    return {"wait_fraction_mean": frac(0), "wait_fraction_max": round(float((s[:, 0] / tot).max()), 4),
            "waits_per_step": round(float(s[:, 1].mean()) / steps, 2),
            "sync_wave_fraction": {"poll": frac(0), "stage": frac(4), "wait_streams": frac(5),
                                   "epilogue": frac(6), "attention": frac(7), "lm_sample": frac(8)},
            "stream_wave1_fraction": {"wait_input": frac(9), "consume": frac(10)},
            "stream_wave1_ns_per_piece": round(float((s[:, 10] * 10.0 / np.maximum(s[:, 11], 1)).mean()), 1),
            "xcd_ids": sorted(set(int(x) for x in s[:, 2]))}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--reps", type=int, default=5, help="timed launches of K steps each (median reported)")
    ap.add_argument("--workload", default="dec2b_25l_greedy")
    ap.add_argument("--rotate", type=int, default=16,
                    help="layer workload: distinct copies of the layer run in one launch")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--stats", action="store_true", help="build the state with LF_STATS (wait-time counters)")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="write profiles/traffic_<workload>.json from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE CSVs "
                         "of this command (DIR/fetch, DIR/write) and of --copy-calibration 1024 (DIR/cfetch, "
                         "DIR/cwrite), then exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of MIB MiB (a known-size kernel for scaling "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE readings) and exit")
    args = ap.parse_args()
    if args.traffic_from:
        return write_traffic(args.traffic_from, args.workload, args.steps, args.warmup, args.rotate)
    if args.copy_calibration:
        import torch
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 3}), flush=True)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library runs on one GPU only (no sharding, no collectives); "
              "--gpus N with N > 1 is not supported", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth
    from persistent_runtime_amd import lf

    K, W, R = args.steps, args.warmup, max(1, args.reps)
    cfg, kind, P, pos0 = setup(args.workload, K, W, args.rotate)
    torch.cuda.set_device(0)
    t0 = time.time()
    weights = synth.model_weights(cfg)
    log(f"weights generated in {time.time() - t0:.1f}s")
    dev = lf.upload_weights(weights)
    eng = lf.Engine(cfg, dev, flags=lf.LF_STATS if args.stats else 0)
    del dev
    torch.cuda.empty_cache()
    log(f"engine: grid={eng.grid} lds={eng.lds_bytes}")
    stream = torch.cuda.current_stream()
    prompt_rec = None
    extra = {}
    if kind in ("kv", "hidden"):
        k, v = synth.kv_prefill(cfg, P)
        for l in range(cfg["n_layers"]):
            eng.kv_fill(l, 0, torch.from_numpy(k[l]).cuda(), torch.from_numpy(v[l]).cuda())
        del k, v
    if kind == "hidden":
        x = torch.from_numpy(synth.hidden(cfg)).cuda()
        eng.set_hidden(x)
        for _ in range(max(1, W)):
            eng.decode_step(0, pos0)
        _, t = time_launches(lambda: eng.decode_step(0, pos0), R, stream)
        # one cold single-layer step: a one-layer engine after a 1 GiB read has
        # displaced the last-level cache
        one = dict(cfg, n_layers=1)
        e1 = lf.Engine(one, lf.upload_weights(dict(weights, layers=weights["layers"][:1])))
        k1, v1 = synth.kv_prefill(one, P)
        e1.kv_fill(0, 0, torch.from_numpy(k1[0]).cuda(), torch.from_numpy(v1[0]).cuda())
        e1.set_hidden(x)
        e1.decode_step(0, pos0)
        junk = torch.ones((1 << 30) // 4, dtype=torch.float32, device="cuda")
        float(junk.sum())
        _, tc = time_launches(lambda: e1.decode_step(0, pos0), 1, stream)
        e1.close()
        del junk
        extra["cold_single_layer_launch_us"] = round(tc["median"] * 1e3, 2)
        out = None
    else:
        if kind == "prompt":
            prompt = synth.prompt(cfg, P)
            _, tp = time_launches(lambda: eng.prefill(prompt[:pos0], 0), 1, stream)
            prompt_rec = {"tokens": pos0, "launches": 1, "ms": tp["median"],
                          "tokens_per_s": round(pos0 / (tp["median"] * 1e-3), 1),
                          "note": "teacher-forced prompt in one lf_prefill launch; not part of the decode rate"}
            first = int(prompt[pos0])
        else:
            first = int(synth.prompt(dict(cfg, prompt_len=1), 1)[0])
        torch.cuda.synchronize()
        if W > 0:
            src = prompt if kind == "prompt" else synth.prompt(dict(cfg, prompt_len=W), W)
            eng.prefill(np.resize(src, W).astype(np.int32), pos0)   # any in-vocabulary tokens

        def run():
            eng.set_position(first, pos0)
            return eng.generate(K)

        out, t = time_launches(run, R, stream)
        log(f"timed launches: {K} tokens each, ms {t['all']}; first tokens {out[:8].tolist()}")

    ms = t["median"]
    nbytes = launch_bytes(cfg, kind, pos0, K)
    achieved = nbytes / (ms * 1e-3) / 1e9
    traffic, trec = measured_traffic(args.workload, nbytes)
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_GBS, 4), "traffic": traffic,
            "algorithmic_bytes_per_launch": nbytes, "kernel": kernel_name(cfg), "launch_ms": t}
    if trec is not None:
        roof["traffic_source"] = (f"rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE of {trec['dispatches']} launch(es) of "
                                  f"{trec['steps']} steps on this kernel source, copy-calibrated: measured / "
                                  f"algorithmic = {trec['measured_over_algorithmic']:.4f}, applied to this launch")
    sampling = "greedy" if cfg.get("temperature", 0) == 0 else f"T={cfg['temperature']} top_p={cfg['top_p']}"
    conf = {"workload": args.workload, "n_layers": cfg["n_layers"], "d_model": cfg["d_model"],
            "n_heads": cfg["n_heads"], "n_kv_heads": cfg["n_kv_heads"], "head_dim": cfg["head_dim"],
            "ffn_dim": cfg["ffn_dim"], "vocab": cfg["vocab"], "batch": 1,
            ("kv_prefill" if kind != "prompt" else "prompt_len"): P,
            "sliding_window": cfg.get("sliding_window", 0), "window_layers": bin(cfg.get("window_layers", 0)),
            "parallelism": "single GPU"}
    if kind == "hidden":
        per_layer_us = ms * 1e3 / cfg["n_layers"]
        conf.update({"layer_copies_per_launch": cfg["n_layers"], "position": pos0})
        res = {"metric": "single-layer decode step time (2B-class layer, KV 1024), 1x MI355X",
               "value": round(per_layer_us, 3), "unit": "us per layer step", "n_gpus": 1,
               "steps": cfg["n_layers"], "warmup": W, "ms_per_step": round(per_layer_us * 1e-3, 6),
               "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
               "data": "synthetic", "config": conf, "roofline": roof}
        res.update(extra)
    else:
        conf.update({"positions": f"{pos0}..{pos0 + K - 1}", "sampling": sampling})
        res = {"metric": METRIC, "value": round(K / (ms * 1e-3), 2), "unit": "tokens/s", "n_gpus": 1,
               "steps": K, "warmup": W, "ms_per_step": round(ms / K, 5), "higher_is_better": True,
               "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic", "config": conf,
               "roofline": roof, "prompt": prompt_rec}
    if args.stats:
        res["wait_stats"] = wait_stats(eng, K if kind != "hidden" else 1)
        log(f"stats: {res['wait_stats']}")
    eng.close()
    torch.cuda.empty_cache()
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(cfg, weights, kind, P, pos0, args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
