#!/usr/bin/env python3
"""Benchmark of the MLA decode step on one MI355X.

A step is one pass of the decode hot path over the batch (one mla_decode_step
call): append the B new tokens' latent rows (kv_a projection, RMSNorm, RoPE,
scatter) and decode them (query projection, absorbed query, split-S latent
attention core, combine, value un-absorb, output projection).  Inputs are synthetic and seeded
(``mla_latent_kv_decode_amd.synth``), resident in HBM before timing; the cache
is filled through the library's own append.  Two copies of the cache are used
alternately so consecutive steps do not find the previous step's cache in the
256 MB Infinity Cache.  The K timed steps are captured once into a HIP graph
(one replay = K steps).  Events recorded inside a captured graph do not time
the kernels between them, so right after the timed replay the same K steps are
run eagerly with HIP events that the library records on its own stream around
every split-S core launch (created without the system-scope fence, so they do
not flush caches); their mean is the core kernel's duration.

Prints ONE JSON line.  Default workload: V2-Lite shapes, B = 64 sequences with
cached lengths ~ U{512..8192} (``v2lite_decode_b64``).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
ROW_BYTES = 1152               # one bf16 latent row: 512 + 64 values
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_core_v2lite_b64_traffic.json")
CORE_SRC = os.path.join(ROOT, "mla_latent_kv_decode_amd", "csrc", "k_decode_ring.hip")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="v2lite_decode_b64")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the oracle (CPU baseline) sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time eager calls, no HIP graph")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for HBM counter calibration)")
    return ap.parse_args()


def copy_calibration(steps: int):
    """A plain device-to-device copy of 1 GiB, repeated: rocprofv3's FETCH_SIZE
    and WRITE_SIZE for it read 1 GiB each per dispatch if the counters are exact,
    which calibrates the traffic figures of the MLA kernels."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"copy_bytes": n, "ms": dt * 1e3, "GBps_read_plus_write": 2 * n / dt / 1e9}))


def src_hash(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def traffic_from_profile(n_launch_bytes: float):
    """HBM bytes per launch of the core kernel from the committed rocprofv3
    counter summary, or None if absent or taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        t = json.load(open(TRAFFIC_FILE))
    except Exception:
        return None
    if t.get("kernel_src_sha") != src_hash(CORE_SRC):
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(wl, w, lens, budget_s: float):
    """The fp64 oracle (as it stands) on a bounded sample of the same workload:
    whole sequences from the start of the batch until the time budget is used.
    Per sequence the cached rows are prepared untimed; the timed part is the
    decode step (append of the new token + the non-absorbed attention)."""
    from oracle import mla as O
    from mla_latent_kv_decode_amd import synth
    d = wl.dims
    shp = O.MLAShape(hidden=d.hidden, n_heads=d.n_heads, qk_nope=d.qk_nope,
                     qk_rope=d.qk_rope, v_head=d.v_head, kv_lora=d.kv_lora, q_lora=d.q_lora,
                     rope_base=d.rope_base, rms_eps=d.rms_eps)
    spent, rows, toks, passes = 0.0, 0, 0, 0
    prepared = {}
    while spent < budget_s:  # whole passes over the batch until the budget is used
        for b in range(len(lens)):
            L = int(lens[b])
            if b not in prepared:
                x = synth.hidden_states(b, L + 1, d.hidden, wl.dtype)
                prepared[b] = (x, O.latent_rows(x[:L], np.arange(L), w["w_kva"], w["kv_norm_g"],
                                                shp))
            x, prior = prepared[b]
            t0 = time.perf_counter()
            O.mla_step(x[L:], np.array([L]), prior, w, shp)
            spent += time.perf_counter() - t0
            rows += L + 1
            toks += 1
            if spent >= budget_s:
                break
        passes += 1
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count()
    return {"value": rows * ROW_BYTES / spent / 1e9, "unit": "GB/s", "cores": int(cores),
            "kind": "oracle", "tokens_per_s": toks / spent,
            "sample": f"{toks} sequence decodes over {passes} pass(es) of the {len(lens)}-sequence "
                      f"batch ({rows} latent rows), fp64 non-absorbed oracle, {spent:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the sharded "
              "design is described in DESIGN.md and is not run here", file=sys.stderr)
        sys.exit(2)

    import torch
    from mla_latent_kv_decode_amd import synth
    from mla_latent_kv_decode_amd.lib import MLALayer

    if args.copy_calibration:
        copy_calibration(args.steps)
        return

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    wl = synth.WORKLOADS[args.workload]
    assert wl.kind == "decode" and wl.dtype == "bf16"
    d = wl.dims
    tdt = torch.bfloat16

    # ---- set-up (untimed): weights, caches filled by append
    w = synth.make_weights(d, wl.weight_std, wl.dtype)
    layer = MLALayer(d, wl.dtype)
    layer.absorb_weights({k: torch.from_numpy(v).cuda().to(tdt) for k, v in w.items()})
    lens = synth.lengths(wl)
    seq_off, seq_len, total = synth.decode_layout(lens)
    B = len(lens)
    caches = [torch.empty((total, d.row), dtype=tdt, device="cuda") for _ in range(2)]
    x_new = np.empty((B, d.hidden), np.float32)
    chunk = 8192
    for b in range(B):
        n = int(lens[b]) + 1
        for s in range(0, n, chunk):
            m = min(chunk, n - s)
            x = synth.hidden_states(b, m, d.hidden, wl.dtype, start=s)
            layer.append(torch.from_numpy(x).cuda().to(tdt), np.arange(s, s + m),
                         int(seq_off[b]) + np.arange(s, s + m), caches[0])
        x_new[b] = x[-1]
    caches[1].copy_(caches[0])
    xd = torch.from_numpy(x_new).cuda().to(tdt)
    pos = (seq_len - 1).astype(np.int32)
    slot = seq_off + pos
    y = torch.empty((B, d.hidden), dtype=tdt, device="cuda")
    torch.cuda.synchronize()

    def step(i):
        # append the B new rows and decode them in one library call
        layer.decode_step(xd, seq_off, seq_len, caches[i % 2], out=y)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps

    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s, capture_error_mode="relaxed"):
                for i in range(K):
                    step(i)
        torch.cuda.current_stream().wait_stream(s)
        graph.replay()  # one untimed replay
        torch.cuda.synchronize()

    def eager_steps_with_core_events():
        layer.core_timing(K)
        for i in range(K):
            step(i)
        core = layer.core_timing_read(K)
        layer.core_timing(0)
        return core

    # ---- timed region: exactly K steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        core = eager_steps_with_core_events()
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / K
    if graph is not None:
        # events recorded inside a captured graph do not time the kernel between
        # them, so the core kernel is timed on the same K steps run eagerly
        core = eager_steps_with_core_events()
        torch.cuda.synchronize()
    assert len(core) == K
    core_ms = float(np.mean(core))
    cache_bytes = float(int(seq_len.sum()) * ROW_BYTES)
    weight_bytes = 2.0 * sum(v.size for v in w.values())
    act_bytes = 2.0 * (2 * B * d.hidden + B * d.row)  # hidden in, y out, appended rows
    gbs = cache_bytes / t_step / 1e9
    core_gbs = cache_bytes / (core_ms * 1e-3) / 1e9
    traffic = traffic_from_profile(cache_bytes)

    res = {
        "metric": "MLA decode latent-KV GB/s + tokens/s (V2-Lite shapes, B=64), % of HBM peak",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 5),
        "tokens_per_s": round(B / t_step, 1),
        "hbm_frac_step": round((cache_bytes + weight_bytes + act_bytes) / t_step / 1e9
                               / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "timing": "eager" if graph is None else "hip-graph replay of the K steps",
        "config": {"workload": wl.name, "batch": B, "len_lo": wl.len_lo, "len_hi": wl.len_hi,
                   "latent_rows": int(seq_len.sum()), "cache_bytes": int(cache_bytes),
                   "weight_bytes": int(weight_bytes), "hidden": d.hidden, "heads": d.n_heads,
                   "kv_lora": d.kv_lora, "qk_rope": d.qk_rope},
        "roofline": {"kernel": "decode_core_ring_k", "bound": "hbm",
                     "kernel_timing": "HIP events (no system fence) around every split-S core "
                                      "launch, K eager steps",
                     "achieved": round(core_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(core_gbs / HBM_PEAK_GBS, 4),
                     "kernel_ms": round(core_ms, 5),
                     "algorithmic_bytes_per_launch": int(cache_bytes),
                     "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, w, lens, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
