"""Benchmark of the mixed retrieval/streaming KV attention hot path on one GPU.

Default workload: one full-model decode step of a 70B-GQA-shaped model
(80 layers, n_q=64, n_kv=8, d=128, bf16, 128,000-token context, S=64,
W=1024, 2 of 8 KV heads retrieval per layer): per layer, one new token per
KV head is appended and the layer's queries decoded, in one duo_decode_append
call (the same work as duo_append of the token followed by duo_decode).  The
step is captured once in a HIP graph and replayed; each replay is the next
generation step (the kernels read every row's token count when they run), so
the timed steps hold T + warmup .. T + warmup + steps - 1 tokens and the
bytes are taken at their mean.

Prints one JSON line.  `value` is the step's algorithmic KV bytes (held K+V
rows read once per KV head, plus the appended rows, queries and outputs)
divided by the measured step time.  `roofline` is for one duo_decode launch
(the split kernel plus the combine kernel of its partials), timed with HIP
events on the launch stream around graph replays of the layers' decodes.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.

Usage: python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]
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

import numpy as np  # noqa: E402

import workloads as WL  # noqa: E402

METRIC = "mixed-head decode attention: KV GB/s (% HBM peak), µs/step at 128k ctx"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_DENSE_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PROFILES = os.path.join(ROOT, "profiles")
# Cache copies a step rotates through: the batch-8 32k decode reads 294 MB, close
# to the 256 MiB last-level (Infinity) cache, so four copies (1.2 GB) keep its
# rows from being served from that cache between steps.
MALL_COPIES = {"llama3_8b_decode_b8_32k": 4}
# every source the decode kernels are compiled from: counters taken on an
# older version of any of them no longer describe the kernel
KERNEL_SRC = [os.path.join(ROOT, "head_wise_kv_amd", "csrc", f)
              for f in ("duo_kernels.hip", "duo_internal.h", "duo_rows.h", "duo_rope.h", "duo_dma.h")]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def src_hash(paths) -> str:
    h = hashlib.sha256()
    for path in ([paths] if isinstance(paths, str) else paths):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(name: str, kernel_hash: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if there is none or the kernel source changed since it was taken."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    kv = {}
    for ln in open(path):
        if "=" in ln and not ln.startswith("#"):
            k, v = ln.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_src_sha256_16") != kernel_hash:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ decode

def decode_layer_bytes(w: WL.Workload, mask_row, T: int, append: bool) -> int:
    """Algorithmic bytes of one layer's step: every held K and V row once per
    KV head, the queries and outputs, and (if appending) the new K/V rows
    read from the input and written to the cache."""
    n_ret = int(np.sum(mask_row))
    n_str = w.n_kv - n_ret
    rows = w.B * (n_ret * T + n_str * min(T, w.S + w.W))
    if w.forked:  # the prefix's full pages, shared by the B rows, are read once
        shared = (w.T - 1) // w.page_rows * w.page_rows
        rows -= (w.B - 1) * n_ret * shared
    kv = rows * w.kv_row_bytes * 2  # FP8 rows: codes plus the row scale
    qo = 2 * w.B * w.n_q * w.d * w.elem_bytes
    app = 2 * w.B * w.n_kv * (w.d * w.elem_bytes + w.kv_row_bytes) if append else 0
    return kv + qo + app


def _timed_replays(graph, steps: int, stream=None):
    """Replay `graph` `steps` times with a HIP event between replays (on the
    launch stream): (total seconds, list of per-replay seconds)."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    if stream is None:
        evs[0].record()
        for i in range(steps):
            graph.replay()
            evs[i + 1].record()
    else:
        evs[0].record(stream)
        with torch.cuda.stream(stream):
            for i in range(steps):
                graph.replay()
                evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) * 1e-3 for i in range(steps)]
    return evs[0].elapsed_time(evs[steps]) * 1e-3, per


def bench_decode(w: WL.Workload, steps: int, warmup: int, layers: int, copies: int = 1):
    """One step = every layer's decode (or fused append + decode) of `copies`
    separate caches in turn, captured in one HIP graph; per-step figures are
    per cache copy (copies > 1 keeps a working set near the 256 MiB
    last-level cache from being served by it)."""
    import torch
    import head_wise_kv_amd as H

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = layers
    mask = WL.mask_table(w, L)
    append = w.mode == "decode_append"
    T = w.T
    fill = T - 1 if append else T
    # every replay of a fused step appends one more token (the kernels read the
    # rows' counts when they run), so the rows have room for all of them
    T_cap = T + (warmup + steps if append else 0)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    pages = dict(page_rows=w.page_rows, n_pages=w.B * -(-T_cap // w.page_rows)) if w.page_rows else {}
    caches = [H.DuoCache(L, w.B, w.n_q, w.n_kv, w.d, T_cap, w.S, w.W, w.dtype, mask, device=dev,
                         kv_format=w.kv_format, rope_theta=w.rope_theta, **pages) for _ in range(copies)]
    log(f"{w.name}: {copies} x arena {caches[0].arena_bytes / 1e9:.2f} GB, filling {L} layers x {fill} tokens")
    t0 = time.time()
    buf_k = torch.empty(1 if w.forked else w.B, w.n_kv, fill, w.d, dtype=dt, device=dev)
    buf_v = torch.empty_like(buf_k)
    for l in range(L):
        WL.device_fill_normal(buf_k, WL.device_seed(w, l, WL.TENSOR_K), w.S, w.sink_scale)
        WL.device_fill_normal(buf_v, WL.device_seed(w, l, WL.TENSOR_V))
        for cache in caches:
            if w.forked:  # row 0 holds the prefix; the other rows are forks of it
                cache.append_row(l, 0, buf_k, buf_v)
                for b in range(1, w.B):
                    cache.fork_row(l, 0, b)
            else:
                cache.append(l, buf_k, buf_v)
    del buf_k, buf_v
    q = torch.empty(L, w.B, w.n_q, w.d, dtype=dt, device=dev)
    WL.device_fill_normal(q, WL.device_seed(w, 0, WL.TENSOR_Q))
    out = torch.empty_like(q)
    k_new = torch.empty(L, w.B, w.n_kv, 1, w.d, dtype=dt, device=dev)
    v_new = torch.empty_like(k_new)
    WL.device_fill_normal(k_new, WL.device_seed(w, 0, WL.TENSOR_K, 1))
    WL.device_fill_normal(v_new, WL.device_seed(w, 0, WL.TENSOR_V, 1))
    q_l = [q[l] for l in range(L)]
    o_l = [out[l] for l in range(L)]
    kn_l = [k_new[l] for l in range(L)]
    vn_l = [v_new[l] for l in range(L)]
    torch.cuda.synchronize()
    log(f"filled in {time.time() - t0:.1f} s")

    stream = torch.cuda.Stream(device=dev)
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        for cache in caches:
            for l in range(L):
                if append:
                    cache.decode_append(l, kn_l[l], vn_l[l], q_l[l], out=o_l[l], scale=w.scale)
                else:
                    cache.decode(l, q_l[l], out=o_l[l], scale=w.scale)
    torch.cuda.synchronize()
    if append:
        for cache in caches:
            for l in range(L):
                cache.reserve(l, warmup + steps - 1)  # pages for the replays (the capture counted one step)
    # tokens held after the appends of the timed steps: T + warmup .. T + warmup
    # + steps - 1 (replay i of the graph stores position T - 1 + i); bytes at the mean
    T_step = T + warmup + (steps - 1) / 2.0 if append else T
    step_bytes = sum(decode_layer_bytes(w, mask[l], T_step, append) for l in range(L))

    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    total, per = _timed_replays(graph, steps)
    wall = time.perf_counter() - t0
    ms_step = total * 1e3 / (steps * copies)
    per_step = np.asarray(per) / copies
    for cache in caches:
        cache.sync()  # host counts from the device (raises if a step found no room)
    if append:
        assert caches[0].seq_len(0) == T - 1 + warmup + steps, caches[0].seq_len(0)
    log(f"graph: {ms_step * 1e3:.1f} us/step mean, {np.median(per_step) * 1e6:.1f} median, "
        f"{per_step.min() * 1e6:.1f} min (wall {wall / steps * 1e6:.1f} us/replay)")

    # Decode alone: the L duo_decode calls of one step (split kernel + combine
    # kernel each, over the T held rows) captured in a second graph, replayed
    # back to back; HIP events on the launch stream bracket the replays, so
    # the average covers both kernels of a call plus the graph's dispatch gaps.
    dgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(dgraph, stream=stream):
        for cache in caches:
            for l in range(L):
                cache.decode(l, q_l[l], out=o_l[l], scale=w.scale)
    torch.cuda.synchronize()
    reps = max(3, min(steps, 10))
    dgraph.replay()
    dtotal, _ = _timed_replays(dgraph, reps, stream)
    avg_s = dtotal / (reps * L * copies)
    T_dec = caches[0].seq_len(0)  # plain decodes do not append: every replay reads these rows
    avg_bytes = float(np.mean([decode_layer_bytes(w, mask[l], T_dec, False) for l in range(L)]))
    return dict(ms_step=ms_step, median_s=float(np.median(per_step)), min_s=float(per_step.min()),
                step_bytes=step_bytes, decode_avg_s=avg_s, decode_avg_bytes=avg_bytes,
                mask=mask, T=T_step, T_decode=T_dec, layers=L, graph_wall_us=wall / steps * 1e6, copies=copies)


# ------------------------------------------------------------------ prefill (secondary)

def prefill_flops(w: WL.Workload, mask_row) -> float:
    """Visible (query, key) pairs x 4 d flops over the whole sequence."""
    N, S, W, d, g = w.T, w.S, w.W, w.d, w.g
    t = np.arange(N, dtype=np.float64)
    causal = float(np.sum(t + 1))
    lam = float(np.sum(np.minimum(t + 1, np.minimum(S, t + 1) + np.minimum(W, np.maximum(t + 1 - S, 0)))))
    n_ret = int(np.sum(mask_row))
    return 4.0 * d * w.B * g * (n_ret * causal + (w.n_kv - n_ret) * lam)


def bench_prefill(w: WL.Workload, reps: int = 2):
    import torch
    import head_wise_kv_amd as H

    dev = torch.device("cuda:0")
    mask = WL.mask_table(w, 1)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    N, C = w.T, w.chunk
    q = torch.empty(w.B, w.n_q, N, w.d, dtype=dt, device=dev)
    k = torch.empty(w.B, w.n_kv, N, w.d, dtype=dt, device=dev)
    v = torch.empty_like(k)
    WL.device_fill_normal(q, WL.device_seed(w, 0, WL.TENSOR_Q))
    WL.device_fill_normal(k, WL.device_seed(w, 0, WL.TENSOR_K))
    WL.device_fill_normal(v, WL.device_seed(w, 0, WL.TENSOR_V))
    qc = [q[:, :, p:p + C].contiguous() for p in range(0, N, C)]
    kc = [k[:, :, p:p + C].contiguous() for p in range(0, N, C)]
    vc = [v[:, :, p:p + C].contiguous() for p in range(0, N, C)]
    oc = [torch.empty_like(x) for x in qc]
    best = None
    for r in range(reps + 1):
        cache = H.DuoCache(1, w.B, w.n_q, w.n_kv, w.d, N, w.S, w.W, w.dtype, mask, device=dev)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(len(qc)):
            cache.prefill_chunk(0, qc[i], kc[i], vc[i], out=oc[i], scale=w.scale)
        e1.record()
        torch.cuda.synchronize()
        s = e0.elapsed_time(e1) * 1e-3
        if r > 0:
            best = s if best is None else min(best, s)
        del cache
    flops = prefill_flops(w, mask[0])
    tf = flops / best / 1e12
    return dict(workload=w.name, seconds=best, tflops=tf, mfma_frac=tf / BF16_DENSE_TFLOPS, algorithmic_tflop=flops / 1e12)


# ------------------------------------------------------------------ gated forward (secondary)

def gated_flops(w: WL.Workload) -> float:
    """Causal (query, key) pairs x 4 d flops: every pair's score and P V product
    is needed once (the sink+window pairs are a subset of the causal ones)."""
    N = w.T
    return 4.0 * w.d * w.B * w.n_q * (N * (N + 1) / 2.0)


def bench_gated(w: WL.Workload, reps: int = 3):
    import torch
    import head_wise_kv_amd as H

    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q = torch.empty(w.B, w.n_q, w.T, w.d, dtype=dt, device=dev)
    k = torch.empty(w.B, w.n_kv, w.T, w.d, dtype=dt, device=dev)
    v = torch.empty_like(k)
    WL.device_fill_normal(q, WL.device_seed(w, 0, WL.TENSOR_Q))
    WL.device_fill_normal(k, WL.device_seed(w, 0, WL.TENSOR_K))
    WL.device_fill_normal(v, WL.device_seed(w, 0, WL.TENSOR_V))
    alpha = torch.from_numpy(WL.gate_values(w, 0)).to(dev)
    out = torch.empty_like(q)
    H.gated_attention(q, k, v, alpha, w.S, w.W, out=out, scale=w.scale)  # warm-up
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        H.gated_attention(q, k, v, alpha, w.S, w.W, out=out, scale=w.scale)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3)
    best = min(times)
    flops = gated_flops(w)
    tf = flops / best / 1e12
    return dict(workload=w.name, seconds=best, median_s=float(np.median(times)), tflops=tf,
                mfma_frac=tf / BF16_DENSE_TFLOPS, algorithmic_tflop=flops / 1e12)


# ------------------------------------------------------------------ CPU oracle baseline

def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:  # noqa: BLE001
        return os.cpu_count() or 1


def cpu_baseline(w: WL.Workload, budget_s: float = 15.0, prefill_rows: int = 256):
    """The oracle on host cores, on bounded samples (inputs generated on the
    host by the seeded recipe; generation is not timed):
      * decode: as many whole layers of workload `w` as fit in about
        `budget_s` seconds;
      * prefill: the first `prefill_rows` rows of the last 4,096-token chunk
        of the 64k chunked prefill, every query head, against the 61,440
        cached positions plus the chunk."""
    from oracle import attention as OA
    append = w.mode == "decode_append"
    spent, nbytes, layers = 0.0, 0, 0
    for l in range(w.L):
        mask = WL.retrieval_mask(w, l)
        K = WL.round_to_dtype(WL.stacked_rows_f32(w, l, WL.TENSOR_K, w.n_kv, 0, w.T), w.dtype)
        V = WL.round_to_dtype(WL.stacked_rows_f32(w, l, WL.TENSOR_V, w.n_kv, 0, w.T), w.dtype)
        Q = WL.round_to_dtype(WL.stacked_rows_f32(w, l, WL.TENSOR_Q, w.n_q, w.T - 1, w.T)[:, :, 0], w.dtype)
        t0 = time.perf_counter()
        for b in range(w.B):
            OA.decode_step(Q[b], K[b], V[b], mask, w.S, w.W, w.scale)
        spent += time.perf_counter() - t0
        nbytes += decode_layer_bytes(w, mask, w.T, append)
        layers += 1
        del K, V
        if spent >= budget_s:
            break
    pw = WL.WORKLOADS["llama3_8b_prefill_64k"]
    pmask = WL.retrieval_mask(pw, 0)
    N, C = pw.T, pw.chunk
    p0 = N - C
    rows = p0 + np.arange(prefill_rows)
    Qp = WL.round_to_dtype(WL.stacked_rows_f32(pw, 0, WL.TENSOR_Q, pw.n_q, p0, p0 + prefill_rows)[0], pw.dtype)
    hi = int(rows.max()) + 1
    Kp = WL.round_to_dtype(WL.stacked_rows_f32(pw, 0, WL.TENSOR_K, pw.n_kv, 0, hi)[0], pw.dtype)
    Vp = WL.round_to_dtype(WL.stacked_rows_f32(pw, 0, WL.TENSOR_V, pw.n_kv, 0, hi)[0], pw.dtype)
    Qfull = np.zeros((pw.n_q, hi, pw.d))
    Qfull[:, rows] = Qp
    t0 = time.perf_counter()
    OA.prefill_full(Qfull, Kp, Vp, pmask, pw.S, pw.W, pw.scale, rows=rows)
    pspent = time.perf_counter() - t0
    t = rows.astype(np.float64)
    lam = np.minimum(t + 1, np.minimum(pw.S, t + 1) + np.minimum(pw.W, np.maximum(t + 1 - pw.S, 0)))
    n_ret = int(np.sum(pmask))
    pflops = 4.0 * pw.d * pw.g * (n_ret * float(np.sum(t + 1)) + (pw.n_kv - n_ret) * float(np.sum(lam)))
    return dict(value=nbytes / spent / 1e9, unit="GB/s", cores=_blas_threads(), cpu_count=os.cpu_count(),
                kind="oracle",
                sample=f"{layers} of {w.L} layers of {w.name}, fp64 numpy oracle, {spent:.1f} s",
                prefill={"value": pflops / pspent / 1e12, "unit": "TFLOP/s",
                         "sample": f"rows {p0}..{p0 + prefill_rows - 1} (first {prefill_rows} of chunk "
                                   f"{N // C - 1}) of {pw.name}, all {pw.n_q} query heads, {pspent:.1f} s",
                         "algorithmic_tflop": pflops / 1e12})


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa70b_decode_128k",
                    choices=[n for n, w in WL.WORKLOADS.items() if w.mode in ("decode", "decode_append")])
    ap.add_argument("--layers", type=int, default=0, help="limit layers (profiling only; 0 = all)")
    ap.add_argument("--also", default="tiny_decode,llama3_8b_decode_b8_32k,"
                                      "mha7b_decode_128k,gqa70b_decode_128k_fp8,mha7b_decode_128k_fp8,"
                                      "gqa70b_decode_128k_int4,mha7b_decode_128k_int4,"
                                      "gqa70b_decode_128k_paged,gqa70b_decode_128k_rope,"
                                      "gqa70b_decode_128k_full,mha7b_decode_128k_full,"
                                      "gqa70b_decode_128k_b2_forked,gqa70b_decode_128k_b2_paged",
                    help="comma-separated extra decode workloads reported under 'also' ('' for none)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-gated", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the decode and prefill kernels run on one device); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    w = WL.WORKLOADS[args.workload]
    L = args.layers if args.layers > 0 else w.L
    if args.calibrate_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log("calibration copy: 1073741824 bytes read, 1073741824 bytes written")
        del a, b
    r = bench_decode(w, args.steps, args.warmup, L, copies=MALL_COPIES.get(w.name, 1))
    value = r["step_bytes"] / (r["ms_step"] * 1e-3) / 1e9
    achieved = r["decode_avg_bytes"] / r["decode_avg_s"] / 1e9
    traffic = stored_traffic(f"decode_{w.name}_traffic.txt", src_hash(KERNEL_SRC))
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_step"], 4),
        "us_per_step": round(r["ms_step"] * 1e3, 1),
        "us_per_step_median": round(r["median_s"] * 1e6, 1),
        "us_per_step_min": round(r["min_s"] * 1e6, 1),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) on device; mask seeded per layer)",
        "config": {"workload": w.name, "layers": L, "batch": w.B, "n_q": w.n_q, "n_kv": w.n_kv, "d_head": w.d,
                   "context": w.T, "context_mean_timed": r["T"], "sink": w.S, "recent": w.W, "retrieval_kv_heads_per_layer": w.n_ret,
                   "step": ("append 1 token + decode, every layer (duo_decode_append)" if w.mode == "decode_append"
                            else "decode, every layer"),
                   "parallelism": "single GPU"},
        "roofline": {"kernel": "duo_decode: decode_kernel + combine_kernel", "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "avg_launch_us": round(r["decode_avg_s"] * 1e6, 2),
                     "algorithmic_bytes_per_launch": int(r["decode_avg_bytes"])},
    }
    also = []
    for name in [x for x in args.also.split(",") if x and x != w.name]:
        import gc
        gc.collect()
        torch.cuda.empty_cache()
        wa = WL.WORKLOADS[name]
        copies = MALL_COPIES.get(name, 1)
        ra = bench_decode(wa, max(args.steps, 20), args.warmup, wa.L, copies=copies)
        va = ra["step_bytes"] / (ra["ms_step"] * 1e-3) / 1e9
        also.append({"workload": name, "kv_rows": wa.kv_format or wa.dtype, "page_rows": wa.page_rows,
                     "rope_theta": wa.rope_theta, "cache_copies": copies,
                     "value": round(va, 2), "unit": "GB/s", "us_per_step": round(ra["ms_step"] * 1e3, 2),
                     "us_per_step_median": round(ra["median_s"] * 1e6, 2),
                     "us_per_step_min": round(ra["min_s"] * 1e6, 2),
                     "hbm_frac": round(va / HBM_PEAK_GBS, 4),
                     "decode_kernel_gbs": round(ra["decode_avg_bytes"] / ra["decode_avg_s"] / 1e9, 2),
                     "decode_kernel_us": round(ra["decode_avg_s"] * 1e6, 2)})
    if also:
        line["also"] = also
        # decode speedup of the mixed cache over full attention (every head a
        # retrieval head) through the same kernels, attention only
        steps_us = {x["workload"]: x["us_per_step"] for x in also}
        if L == w.L:  # the whole model, like the entries above
            steps_us[w.name] = round(r["ms_step"] * 1e3, 1)
        vs_full = {n: {"mixed_us_per_step": steps_us[n], "full_us_per_step": steps_us[n + "_full"],
                       "speedup": round(steps_us[n + "_full"] / steps_us[n], 3)}
                   for n in steps_us if n + "_full" in steps_us}
        if vs_full:
            line["duo_vs_full_attention"] = vs_full
        # two requests sharing a 128k prefix (forked rows: its pages stored and
        # read once) against the same two rows held apart
        if "gqa70b_decode_128k_b2_forked" in steps_us and "gqa70b_decode_128k_b2_paged" in steps_us:
            f, p = steps_us["gqa70b_decode_128k_b2_forked"], steps_us["gqa70b_decode_128k_b2_paged"]
            line["shared_prefix"] = {"forked_us_per_step": f, "apart_us_per_step": p, "speedup": round(p / f, 3)}
    if not args.no_prefill:
        pw = WL.WORKLOADS["llama3_8b_prefill_64k"]
        p = bench_prefill(pw)
        line["prefill"] = {"workload": p["workload"], "ms": round(p["seconds"] * 1e3, 3),
                           "tflops": round(p["tflops"], 2), "mfma_frac": round(p["mfma_frac"], 4),
                           "peak_tflops": BF16_DENSE_TFLOPS, "algorithmic_tflop": round(p["algorithmic_tflop"], 4)}
    if not args.no_gated:
        gw = WL.WORKLOADS["llama3_8b_gated_32k"]
        gr = bench_gated(gw)
        line["gated"] = {"workload": gr["workload"], "ms": round(gr["seconds"] * 1e3, 3),
                         "ms_median": round(gr["median_s"] * 1e3, 3), "tflops": round(gr["tflops"], 2),
                         "mfma_frac": round(gr["mfma_frac"], 4), "peak_tflops": BF16_DENSE_TFLOPS,
                         "algorithmic_tflop": round(gr["algorithmic_tflop"], 4)}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
