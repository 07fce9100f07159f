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

``--workload v2lite_decode_b64_fp8`` is the same decode batch on an FP8 latent
cache (656-byte rows: E4M3 codes, bf16 RoPE key, per-row scale); its GB/s
count those bytes.

``--workload v2lite_decode_b64_paged`` is the same batch on a paged cache
(64-row pages handed out in a seeded random order, mla_decode_step_paged).

``--workload v2lite_decode_b64_q2``: the same sequences decoding two new tokens
each per step (mla_decode_ex with the append; 128 query rows).

``--workload v3_prefill_4x4096`` measures the chunked causal prefill instead
(V3 shapes, 4 sequences of 4096 new tokens after 0 / 2048 cached rows): a step
is the append of the new tokens' latent rows plus one mla_prefill call over the
batch, timed eagerly; the figure is expanded-form TFLOP/s against the bf16
MFMA peak, with the attention kernel's own rate (library events around its
launches) as the roofline entry.
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
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, vendor figure
ROW_BYTES = 1152               # one bf16 latent row: 512 + 64 values
FP8_ROW_BYTES = 656            # one FP8 row: 512 codes, 64 bf16 rope values, scale, pad
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
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="limit the oracle's BLAS threads (0: as configured)")
    ap.add_argument("--cpu-only", action="store_true",
                    help="only time the oracle on the workload's sample (no GPU)")
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


def traffic_from_profile(workload: str, kernel: str):
    """HBM bytes per launch of the core kernel from the committed rocprofv3
    counter summary, or None if absent, taken on another workload or kernel,
    or on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        t = json.load(open(TRAFFIC_FILE))
    except Exception:
        return None
    if str(t.get("workload", "")).split(" ")[0] != workload or t.get("kernel") != kernel:
        return None
    if t.get("kernel_src_sha") != src_hash(CORE_SRC):
        return None
    return t.get("hbm_bytes_per_launch")


def _oracle_threads() -> int:
    """Threads the oracle's BLAS actually runs with."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))
    except Exception:
        return int(os.cpu_count() or 1)


def _cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _thread_limit(n: int):
    """A context limiting the oracle's BLAS pools to n threads (n = 0: none)."""
    import contextlib
    if n <= 0:
        return contextlib.nullcontext()
    from threadpoolctl import threadpool_limits
    return threadpool_limits(limits=n)


def cpu_only(args):
    """The oracle's cpu_baseline of a workload by itself, on the host only."""
    from mla_latent_kv_decode_amd import synth
    wl = synth.WORKLOADS[args.workload]
    w = synth.make_weights(wl.dims, wl.weight_std, wl.dtype)
    with _thread_limit(args.cpu_threads):
        if wl.kind == "prefill":
            base = cpu_baseline_prefill(wl, w, args.cpu_seconds)
        else:
            base = cpu_baseline(wl, w, synth.lengths(wl), args.cpu_seconds)
    print(json.dumps({"workload": wl.name, "cpu_baseline": base}), flush=True)


def cpu_baseline(wl, w, lens, budget_s: float):
    """The fp64 oracle (as it stands) on a bounded sample of the same workload:
    whole sequences from the start of the batch until the time budget is used.
    Per sequence the cached rows are prepared untimed; the timed part is the
    decode step (append of the new token + the non-absorbed attention)."""
    from oracle import mla as O
    from mla_latent_kv_decode_amd import synth
    d = wl.dims
    store = None
    row_bytes = d.row * (4 if wl.dtype == "f32" else 2)  # the GPU cache's row
    if wl.kv == "fp8":
        from oracle import fp8 as F8
        store = lambda r: F8.fp8_rows(r, d.kv_lora)  # noqa: E731
        row_bytes = FP8_ROW_BYTES
    shp = O.MLAShape(hidden=d.hidden, n_heads=d.n_heads, qk_nope=d.qk_nope,
                     qk_rope=d.qk_rope, v_head=d.v_head, kv_lora=d.kv_lora, q_lora=d.q_lora,
                     rope_base=d.rope_base, rms_eps=d.rms_eps)
    spent, rows, toks, passes = 0.0, 0, 0, 0
    prepared = {}
    while spent < budget_s:  # whole passes over the batch until the budget is used
        for b in range(len(lens)):
            L = int(lens[b])
            q = wl.q_len
            if b not in prepared:
                x = synth.hidden_states(b, L + q, d.hidden, wl.dtype)
                prepared[b] = (x, O.latent_rows(x[:L], np.arange(L), w["w_kva"], w["kv_norm_g"],
                                                shp))
            x, prior = prepared[b]
            t0 = time.perf_counter()
            O.mla_step(x[L:], np.arange(L, L + q), prior, w, shp, kv_store=store)
            spent += time.perf_counter() - t0
            rows += L + q
            toks += q
            if spent >= budget_s:
                break
        passes += 1
    return {"value": rows * row_bytes / spent / 1e9, "unit": "GB/s", "cores": _oracle_threads(),
            "cpu_model": _cpu_model(), "kind": "oracle", "tokens_per_s": toks / spent,
            "sample": f"{toks} sequence decodes over {passes} pass(es) of the {len(lens)}-sequence "
                      f"batch ({rows} latent rows), fp64 non-absorbed oracle, {spent:.1f} s"}


def prefill_flops(d, T, key_rows, pairs):
    """Expanded-form flops of one prefill step: the projections of the T new
    tokens (q_a / q_b or q, kv_a), the K_nope / V expansion of every key row,
    causal attention over the (query, key) pairs, and the output projection."""
    H, dn, dr, dv, dc, D, dq = (d.n_heads, d.qk_nope, d.qk_rope, d.v_head, d.kv_lora, d.hidden,
                                d.q_lora)
    qw = H * (dn + dr)
    proj = 2.0 * T * D * (dc + dr)                               # kv_a (append)
    proj += 2.0 * T * (D * dq + dq * qw) if dq else 2.0 * T * D * qw
    expand = 2.0 * key_rows * dc * H * (dn + dv)
    attn = 2.0 * H * (dn + dr + dv) * pairs
    out = 2.0 * T * H * dv * D
    return proj + expand + attn + out, attn


def cpu_baseline_prefill(wl, w, budget_s: float):
    """The fp64 oracle (as it stands) on a bounded sample of the same workload:
    chunks of 512 new tokens of sequence 0 (no cached rows) until the time
    budget is used; TFLOP/s over the same expanded-form flop count."""
    from oracle import mla as O
    from mla_latent_kv_decode_amd import synth
    d = wl.dims
    store = None
    row_bytes = ROW_BYTES
    if wl.kv == "fp8":
        from oracle import fp8 as F8
        store = lambda r: F8.fp8_rows(r, d.kv_lora)  # noqa: E731
        row_bytes = FP8_ROW_BYTES
    shp = O.MLAShape(hidden=d.hidden, n_heads=d.n_heads, qk_nope=d.qk_nope,
                     qk_rope=d.qk_rope, v_head=d.v_head, kv_lora=d.kv_lora, q_lora=d.q_lora,
                     rope_base=d.rope_base, rms_eps=d.rms_eps)
    n = 512
    x = synth.hidden_states(0, n, d.hidden, wl.dtype)
    spent, chunks, flops = 0.0, 0, 0.0
    while spent < budget_s:
        t0 = time.perf_counter()
        O.mla_step(x, np.arange(n), np.zeros((0, shp.row)), w, shp)
        spent += time.perf_counter() - t0
        chunks += 1
        flops += prefill_flops(d, n, n, n * (n + 1) // 2)[0]
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": _oracle_threads(),
            "cpu_model": _cpu_model(),
            "kind": "oracle", "tokens_per_s": chunks * n / spent,
            "sample": f"{chunks} prefill(s) of {n} new tokens with no cached rows (sequence 0), "
                      f"fp64 non-absorbed oracle, {spent:.1f} s"}


def bench_prefill(args, wl):
    import torch
    from mla_latent_kv_decode_amd import synth
    from mla_latent_kv_decode_amd.lib import MLALayer
    d = wl.dims
    tdt = torch.bfloat16
    w = synth.make_weights(d, wl.weight_std, wl.dtype)
    layer = MLALayer(d, wl.dtype)
    layer.absorb_weights({k: torch.from_numpy(v).cuda().to(tdt) for k, v in w.items()})
    seq_off, prior, cu_new, total = synth.prefill_layout(wl)
    B = wl.batch
    T = int(cu_new[-1])
    # cached rows before the chunk: latent rows appended from seeded hidden states
    cache = torch.zeros((total, d.row), dtype=tdt, device="cuda")
    for b in range(B):
        if prior[b]:
            xp = synth.hidden_states(b, int(prior[b]), d.hidden, wl.dtype)
            layer.append(torch.from_numpy(xp).cuda().to(tdt), np.arange(prior[b]),
                         int(seq_off[b]) + np.arange(prior[b]), cache)
    x = np.concatenate([synth.hidden_states(b, wl.new_tokens, d.hidden, wl.dtype,
                                            start=int(prior[b])) for b in range(B)])
    xd = torch.from_numpy(x).cuda().to(tdt)
    y = torch.empty((T, d.hidden), dtype=tdt, device="cuda")

    def step():
        # append of the new tokens' latent rows + the prefill, in one call
        layer.prefill_step(xd, cu_new, prior, seq_off, cache, out=y)

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    K = args.steps
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / K
    layer.core_timing(K)
    for _ in range(K):
        step()
    attn = layer.core_timing_read(K)
    layer.core_timing(0)
    torch.cuda.synchronize()
    attn_ms = float(np.mean(attn))
    key_rows = int(sum(int(prior[b]) + int(cu_new[b + 1] - cu_new[b]) for b in range(B)))
    pairs = int(sum(int(prior[b]) * int(cu_new[b + 1] - cu_new[b])
                    + int(cu_new[b + 1] - cu_new[b]) * int(cu_new[b + 1] - cu_new[b] + 1) // 2
                    for b in range(B)))
    flops, attn_flops = prefill_flops(d, T, key_rows, pairs)
    tfs = flops / t_step / 1e12
    attn_tfs = attn_flops / (attn_ms * 1e-3) / 1e12
    res = {
        "metric": "MLA chunked prefill TFLOP/s (V3 shapes, 4 x 4096 new tokens), % of bf16 "
                  "MFMA peak",
        "value": round(tfs, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "tokens_per_s": round(T / t_step, 1),
        "mfma_frac_step": round(tfs / MFMA_BF16_PEAK_TFLOPS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "timing": "eager steps (mla_prefill_step: append + prefill)",
        "config": {"workload": wl.name, "batch": B, "new_tokens": wl.new_tokens,
                   "prior": [int(p) for p in prior], "key_rows": key_rows,
                   "causal_pairs": pairs, "step_tflop": round(flops / 1e12, 4),
                   "hidden": d.hidden, "heads": d.n_heads, "kv_lora": d.kv_lora,
                   "q_lora": d.q_lora},
        "roofline": {"kernel": "prefill_attn_mfma_k", "bound": "mfma",
                     "kernel_timing": "HIP events (no system fence) around every prefill "
                                      "attention launch, K eager steps",
                     "achieved": round(attn_tfs, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tfs / MFMA_BF16_PEAK_TFLOPS, 4),
                     "kernel_ms": round(attn_ms, 4), "algorithmic_flops_per_launch": attn_flops,
                     "traffic": None},
    }
    if not args.no_cpu_baseline:
        with _thread_limit(args.cpu_threads):
            res["cpu_baseline"] = cpu_baseline_prefill(wl, w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the sharded "
              "design shards sequences across GPUs and is not run here", file=sys.stderr)
        sys.exit(2)

    if args.cpu_only:
        cpu_only(args)
        return

    import torch
    from mla_latent_kv_decode_amd import synth
    from mla_latent_kv_decode_amd.lib import MLALayer

    if args.copy_calibration:
        copy_calibration(args.steps)
        return

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    wl = synth.WORKLOADS[args.workload]
    assert wl.dtype == "bf16"
    if wl.kind == "prefill":
        bench_prefill(args, wl)
        return
    assert wl.kind == "decode"
    d = wl.dims
    tdt = torch.bfloat16

    # ---- set-up (untimed): weights, caches filled by append
    w = synth.make_weights(d, wl.weight_std, wl.dtype)
    layer = MLALayer(d, wl.dtype, kv=wl.kv, absorb=wl.absorb)
    layer.absorb_weights({k: torch.from_numpy(v).cuda().to(tdt) for k, v in w.items()})
    lens = synth.lengths(wl)
    q = wl.q_len  # new tokens per sequence and step
    seq_off, seq_len, total = synth.decode_layout(lens, q)
    B = len(lens)
    caches = [layer.new_cache(total) for _ in range(2)]
    row_bytes = layer.row_bytes()
    x_new = np.empty((B * q, d.hidden), np.float32)
    chunk = 8192
    for b in range(B):
        n = int(lens[b]) + q
        for s in range(0, n, chunk):
            m = min(chunk, n - s)
            x = synth.hidden_states(b, m, d.hidden, wl.dtype, start=s)
            layer.append(torch.from_numpy(x).cuda().to(tdt), np.arange(s, s + m),
                         int(seq_off[b]) + np.arange(s, s + m), caches[0])
        x_new[b * q:(b + 1) * q] = x[-q:]
    P = wl.page_rows
    if P:
        # a paged cache: the same rows moved into 64-row pages handed out in a
        # seeded random order (two pools alternate like the two caches)
        table, n_pages = synth.page_table(seq_len, P)
        src, dst = [], []
        for b in range(B):
            t = np.arange(int(seq_len[b]))
            src.append(int(seq_off[b]) + t)
            dst.append(table[b, t // P].astype(np.int64) * P + t % P)
        src_t = torch.as_tensor(np.concatenate(src), device="cuda")
        dst_t = torch.as_tensor(np.concatenate(dst), device="cuda")
        pool = layer.new_cache(n_pages * P)
        pool[dst_t] = caches[0][src_t]
        caches = [pool, pool.clone()]
        del src_t, dst_t
    else:
        caches[1].copy_(caches[0])
    xd = torch.from_numpy(x_new).cuda().to(tdt)
    pos = (seq_len - 1).astype(np.int32)
    slot = seq_off + pos
    y = torch.empty((B * q, d.hidden), dtype=tdt, device="cuda")
    torch.cuda.synchronize()

    def step(i):
        # append the B new rows and decode them in one library call
        if q > 1:
            layer.decode_ex(xd, seq_len, caches[i % 2], q_len=q, seq_off=seq_off, append=True,
                            out=y)
        elif P:
            layer.decode_step_paged(xd, table, P, seq_len, caches[i % 2], out=y)
        else:
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
    cache_bytes = float(int(seq_len.sum()) * row_bytes)
    weight_bytes = 2.0 * sum(v.size for v in w.values())
    if wl.absorb == "materialized":
        # the decode step reads W_kva, [W_qa,] per head [W^KQ_h ; W_q,rope_h] and W^OV
        # (and the norms) in place of the factored query, W_kv_b and W_o weights
        kq = d.q_lora or d.hidden
        weight_bytes = 2.0 * (d.row * d.hidden + d.q_lora * d.hidden
                              + d.n_heads * (d.kv_lora + d.qk_rope) * kq
                              + d.hidden * d.n_heads * d.kv_lora + d.kv_lora + d.q_lora)
    act_bytes = 2.0 * 2 * B * q * d.hidden + B * q * row_bytes  # hidden in, y out, new rows
    gbs = cache_bytes / t_step / 1e9
    core_gbs = cache_bytes / (core_ms * 1e-3) / 1e9
    fp8 = wl.kv == "fp8"
    core_kernel = (("decode_core_wide8_k" if fp8 else "decode_core_wide_k")
                   if d.n_heads % 128 == 0 else
                   "decode_core_ring8_k" if fp8 else "decode_core_ring_k")
    traffic = None if (P or q > 1) else traffic_from_profile(wl.name, core_kernel)

    res = {
        "metric": "MLA decode latent-KV GB/s + tokens/s (V2-Lite shapes, B=64), % of HBM peak"
                  + (", FP8 latent cache" if fp8 else "")
                  + (f", paged cache ({P}-row pages)" if P else "")
                  + (f", {q} new tokens per sequence" if q > 1 else ""),
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 5),
        "tokens_per_s": round(B * q / t_step, 1),
        "hbm_frac_step": round((cache_bytes + weight_bytes + act_bytes) / t_step / 1e9
                               / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "timing": "eager" if graph is None else "hip-graph replay of the K steps",
        "config": {"workload": wl.name, "batch": B, "len_lo": wl.len_lo, "len_hi": wl.len_hi,
                   "latent_rows": int(seq_len.sum()), "cache_row_bytes": row_bytes,
                   "page_rows": P, "q_len": q,
                   "cache_bytes": int(cache_bytes),
                   "weight_bytes": int(weight_bytes), "hidden": d.hidden, "heads": d.n_heads,
                   "kv_lora": d.kv_lora, "qk_rope": d.qk_rope},
        "roofline": {"kernel": core_kernel,
                     "bound": "hbm",
                     "kernel_timing": "HIP events (no system fence) around every split-S core "
                                      "launch, K eager steps",
                     "achieved": round(core_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(core_gbs / HBM_PEAK_GBS, 4),
                     "kernel_ms": round(core_ms, 5),
                     "algorithmic_bytes_per_launch": int(cache_bytes),
                     "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        with _thread_limit(args.cpu_threads):
            res["cpu_baseline"] = cpu_baseline(wl, w, lens, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
