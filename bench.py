"""Benchmark: CSA decode steps per second per layer at a 2^20-token context.

One step = one csa_decode_step of one attention layer (indexer scoring over
262,144 compressed blocks -> causal top-1024 -> gather of 1024 + 128 rows ->
64-head x 512 shared-KV attention), on seeded synthetic inputs already resident
in HBM.  Steps rotate over 30 layer-sized caches (the 30 CSA layers of the
1M-context sizing: 1.9 GiB of indexer keys, 7.5 GiB of compressed KV) so that
every step streams its keys from HBM rather than from the 256 MB last-level
cache.  Timed steps are replayed from HIP graphs, bracketed by device
synchronisation.

Also reported:
  roofline     -- the dominant kernel (indexer scoring): its algorithmic bytes
                  per launch over its mean launch duration measured here with
                  HIP events on its stream, against 8 TB/s;
  cpu_baseline -- the fp64 numpy oracle timed on a bounded sample of the same
                  workload on this host's cores (a reported baseline only).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
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

LAYERS = 30
HBM_PEAK_GBS = 8000.0
METRIC = "CSA decode steps/sec per layer at 1M ctx; achieved HBM GB/s vs peak"


def _kernel_src_hash() -> str:
    h = hashlib.sha256()
    for f in ("index_score.hip", "csa_common.h"):
        with open(os.path.join(ROOT, "sparse_long_context_index_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic_per_launch():
    """HBM bytes per indexer launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "index_score_1m_counters.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("kernel_src_sha256_16") != _kernel_src_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(inp, budget_s: float = 12.0) -> dict:
    """Time the oracle (unchanged) on whole 1M steps until ~budget_s."""
    import numpy as np
    from oracle import csa_token
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    n = 0
    t0 = time.perf_counter()
    while True:
        csa_token(inp, 0)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": n / el, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} full 1M-context CSA decode steps (token 0, layer 0), "
                      f"{el:.1f} s, numpy fp64, BLAS threads={threads}"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3000)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "sharding the path over several GPUs is not built", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from sparse_long_context_index_amd import binding as B
    from sparse_long_context_index_amd import inputs as gen

    dev = torch.device("cuda:0")
    B.load()
    print("bench: generating the 1M-context workload", file=sys.stderr, flush=True)
    inp = gen.ctx1m()
    d0 = B.upload(inp, dev)
    layers = [d0]
    for _ in range(LAYERS - 1):
        dl = dict(d0)
        dl["k_idx"] = d0["k_idx"].clone()
        dl["comp_kv"] = d0["comp_kv"].clone()
        layers.append(dl)
    outs = B.alloc_step_outputs(inp, dev, keep=False, all_kv=False)
    step_args = [B.step_args(inp, dl, outs) for dl in layers]
    ws = B.step_workspace(step_args[0], dev)
    torch.cuda.synchronize()
    print("bench: warmup", file=sys.stderr, flush=True)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            B.csa_decode_step(step_args[i % LAYERS], ws)
    torch.cuda.synchronize()
    if int(outs["err"].item()) != 0:
        raise RuntimeError(f"device error word {int(outs['err'].item()):#x}")

    # Graphs: one replay = LAYERS consecutive steps (+ a remainder graph).
    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                B.csa_decode_step(step_args[i % LAYERS], ws)
        return g
    g_full = capture(LAYERS)
    rem = args.steps % LAYERS
    g_rem = capture(rem) if rem else None
    torch.cuda.synchronize()

    print("bench: timed steps", file=sys.stderr, flush=True)
    with torch.cuda.stream(stream):
        for _ in range(2):
            g_full.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(args.steps // LAYERS):
            g_full.replay()
        if g_rem is not None:
            g_rem.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = gpu_ms / args.steps
    steps_per_s = args.steps / (gpu_ms / 1e3)
    if int(outs["err"].item()) != 0:
        raise RuntimeError(f"device error word {int(outs['err'].item()):#x}")

    # Dominant kernel: indexer scoring, launched through csa_index_score on
    # `stream` back to back over the rotated layers (as the kernels of the
    # step run), between two HIP events recorded on that stream.
    print("bench: indexer kernel timing", file=sys.stderr, flush=True)
    n_vis = inp.max_visible()
    scores = torch.empty((1, n_vis), dtype=torch.float32, device=dev)
    reps = LAYERS * 8

    def index_launch(i):
        dl = layers[i % LAYERS]
        B.csa_index_score(dl["q_idx"], dl["w"], dl["k_idx"], dl["pos"], dl["seq_kv"],
                          dl["n_comp"], inp.n_ih, inp.ihd, inp.ratio, scores, n_vis)

    with torch.cuda.stream(stream):
        for i in range(LAYERS):
            index_launch(i)
        k0 = torch.cuda.Event(enable_timing=True)
        k1 = torch.cuda.Event(enable_timing=True)
        k0.record(stream)
        for i in range(reps):
            index_launch(i)
        k1.record(stream)
    torch.cuda.synchronize()
    k_ms = k0.elapsed_time(k1) / reps
    # algorithmic bytes of one indexer launch: keys + queries + weights read,
    # one fp32 score per visible block written
    idx_bytes = n_vis * inp.ihd * 2 + inp.n_ih * inp.ihd * 2 + inp.n_ih * 4 + n_vis * 4
    achieved = idx_bytes / (k_ms * 1e-3) / 1e9
    traffic = _traffic_per_launch()

    # Secondary denominator: a plain device copy of 1 GiB on the same stream
    # (its rocprofv3 FETCH_SIZE / WRITE_SIZE also calibrate the counters).
    print("bench: device copy bandwidth", file=sys.stderr, flush=True)
    csrc = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    with torch.cuda.stream(stream):
        cdst.copy_(csrc)
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(10):
            cdst.copy_(csrc)
        c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 10 * 2 * csrc.numel() / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del csrc, cdst

    # minimum bytes of a whole step (keys, indexer q and w, selected rows, SWA
    # rows, attention q, output)
    step_bytes = (n_vis * inp.ihd * 2 + inp.n_ih * inp.ihd * 2 + inp.n_ih * 4
                  + inp.top_k * inp.head_dim * 2 + inp.window * inp.head_dim * 2
                  + 2 * inp.n_heads * inp.head_dim * 2)
    step_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu:
        print("bench: CPU oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(inp)

    line = {
        "metric": METRIC,
        "value": round(steps_per_s, 1),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "1M-context CSA decode step, one layer: 262,144 blocks, "
                               "n_ih 64 x ihd 128, top_k 1024, window 128, 64 heads x 512",
                   "layers_rotated": LAYERS, "batch": 1, "context_tokens": 1 << 20},
        "step_min_bytes": step_bytes,
        "step_effective_gbs": round(step_gbs, 1),
        "step_roofline_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "kernel": "index_score_kernel<128,2>",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": idx_bytes, "mean_launch_us": round(k_ms * 1e3, 3)},
        "device_copy_gbs": round(copy_gbs, 1),
        "cpu_baseline": cpu,
        "wall_s": round(wall, 3),
    }
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
