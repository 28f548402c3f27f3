#!/usr/bin/env python3
"""Benchmark of one paged decode step on one MI355X.

A step is the whole hot path over one batch: write each sequence's new token
into its cache slot (pa_reshape_and_cache), then decode attention over the
paged cache (pa_decode: block-table gather, scores, softmax, weighted V sum and
the split-context log-sum-exp merge).  The default workload is the largest
decode configuration one GPU holds: 4 sequences of 131072 tokens each, 32
heads, head_dim 128, block size 16, fp16, 8192 randomly scattered blocks per
sequence (an 8 GiB K+V pool), under the library's default split.  The same
run then measures, with fewer steps, the pages' layer shape (8 sequences,
lengths uniform in [1, 2048]), continuous batching (64 sequences, log-normal
lengths, block 32), the 128K context at batch 1, and the 4 x 128K batch with
explicit partitions of 512 tokens (key "configs"); --no-extra skips them.

Timing is cold-cache: the step rotates over enough replicas of the KV pool
(>= 2 GiB in total) that the 256 MB last-level cache cannot hold the working
set from one visit to the next (a pool of 2 GiB or more is its own replica).
Inputs are resident in HBM before the timed region; the steps are replayed
from HIP graphs and HIP events on the stream the kernels run on bracket
exactly --steps steps.

Prints ONE JSON line on stdout (progress goes to stderr).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: achieved HBM GB/s (% of peak) and µs/step, 1 MI355X"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published peak
COLD_BYTES = 2 << 30           # replica footprint that defeats the 256 MB last-level cache
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_186_amd", "csrc", f)
                  for f in ("pa_decode.hip", "pa_decode_balanced.hip", "pa_decode_balanced_gqa2.hip",
                            "pa_decode_balanced_gqa4.hip", "pa_decode_mfma.hip",
                            "pa_balanced_kernel.h", "pa_attend.h", "pa_device.h", "pa_mfma.h", "pa_internal.h",
                            "pa_api.cpp")]


PF_SOURCES = [os.path.join(ROOT, "paged_kv_cache_186_amd", "csrc", f)
              for f in ("pa_prefill.hip", "pa_prefill_tiles.hip", "pa_mla_heads.hip", "pa_decode_mfma.hip", "pa_attend.h",
                        "pa_device.h", "pa_mfma.h", "pa_internal.h", "pa_api.cpp")]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_digest(sources=None) -> str:
    h = hashlib.sha256()
    for p in (sources or KERNEL_SOURCES):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def decode_bytes(lens: np.ndarray, H: int, D: int, e: int, bs: int, e_kv: int = 0,
                 Hkv: int = 0) -> int:
    """Algorithmic bytes of one decode: K+V rows of the Hkv K/V heads read
    (e_kv bytes per element, default e; Hkv defaults to H), q read and out
    written for the H query heads (e bytes), the used block-table entries and
    the lengths; an 8-bit cache (e_kv == 1) also reads the K and V scale of
    every (block, K/V head) it visits."""
    e_kv = e_kv or e
    Hkv = Hkv or H
    lens = lens.astype(np.int64)
    S = len(lens)
    nb = -(-lens // bs)
    scales = 2 * 4 * int(nb.sum()) * Hkv if e_kv == 1 else 0
    return int(lens.sum() * Hkv * D * 2 * e_kv + 2 * S * H * D * e + 4 * nb.sum() + 4 * S + scales)


def reshape_bytes(T: int, H: int, D: int, e: int, e_kv: int = 0) -> int:
    """New K and V rows read (e bytes) and written (e_kv bytes), the slot
    numbers, and for an 8-bit cache the scales of the written blocks."""
    e_kv = e_kv or e
    scales = 2 * 4 * T * H if e_kv == 1 else 0
    return 2 * T * H * D * e + 2 * T * H * D * e_kv + 4 * T + scales


def profile_path(workload: str, kv: str, kv_heads: int = 0) -> str:
    tag = workload if kv == "native" else f"{workload}_fp8_{kv}"
    if kv_heads:
        tag += f"_kvh{kv_heads}"
    return os.path.join(PROFILES, f"pa_decode_{tag}_traffic.txt")


def traffic_from_profile(digest: str, path: str):
    """Counter-measured HBM bytes per pa_decode launch, if a committed
    rocprofv3 record exists for this workload and was taken on this exact
    kernel source; else None."""
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("kernel_source_sha") != digest:
        return None
    try:
        return float(rec["scaled_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def build_workload(name: str, seed: int, dev):
    from paged_kv_cache_186_amd import workloads as W
    if name == "layer_shape":
        return W.layer_shape(seed, device=dev)
    if name == "continuous_batching":
        return W.continuous_batching(seed, device=dev)
    if name == "shared_prefix":
        return W.shared_prefix(seed, device=dev)
    if name == "long_context_b1":
        return W.long_context(seed, batch=1, device=dev)
    if name == "long_context_b4":
        return W.long_context(seed, batch=4, device=dev)
    if name == "tiny":
        return W.tiny(seed, device=dev, poison=False)
    raise SystemExit(f"unknown workload {name}")


def describe(w) -> str:
    lens = w.context_lens_np()
    return (f"{w.name}: {w.num_seqs} seqs, context {int(lens.min())}..{int(lens.max())} "
            f"(total {int(lens.sum())} tokens), {w.num_heads} heads, head_dim {w.head_dim}, "
            f"block {w.block_size}, {str(w.dtype).replace('torch.', '')}, pool {w.num_blocks} blocks")


def capture(enqueue) -> "torch.cuda.CUDAGraph":
    """Capture the kernels `enqueue` launches on the current stream into a graph."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        enqueue()
    torch.cuda.synchronize()
    return g


def time_eager(reshape, decode, n: int, stream) -> dict:
    """Per-call HIP events around eager calls (includes host launch overhead)."""
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        ev[i][0].record(stream)
        reshape(i)
        ev[i][1].record(stream)
        decode(i)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    res = np.array([e[0].elapsed_time(e[1]) for e in ev])
    dec = np.array([e[1].elapsed_time(e[2]) for e in ev])
    return {"pa_reshape_and_cache": float(np.median(res)), "pa_decode": float(np.median(dec)),
            "pa_decode_p10": float(np.percentile(dec, 10)), "pa_decode_p90": float(np.percentile(dec, 90))}


def check_graph_replays(g, decode, R: int, out) -> None:
    """Replays of the decode graph must equal the eager call bit for bit, with
    eager work in between (the graph ends with replica R-1)."""
    decode(R - 1)
    torch.cuda.synchronize()
    want = out.clone()
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(out.view(torch.int16), want.view(torch.int16)):
            raise RuntimeError("graph replay differs from the eager decode")
        decode(0)
    torch.cuda.synchronize()


def copy_ceiling(dev, nbytes: int = 1 << 30, reps: int = 10) -> float:
    """GB/s of a plain device-to-device copy of nbytes (read + write bytes
    counted), HIP events around `reps` back-to-back copies: the bandwidth this
    box's HBM actually delivers to a simple stream, reported beside the
    nominal peak."""
    src = torch.empty(nbytes // 2, dtype=torch.float16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    end.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (start.elapsed_time(end) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def calibration_copy(pa, dev) -> None:
    """pa_copy_blocks over a known byte count (3 calls of 256 blocks of 128 KiB
    per pool: 64 MiB read and 64 MiB written each), so that counter runs carry
    their own scale for FETCH_SIZE / WRITE_SIZE."""
    k = torch.zeros((512, 32, 16, 128), dtype=torch.float16, device=dev)
    v = torch.zeros_like(k)
    pairs = torch.stack([torch.arange(256), torch.arange(256, 512)], 1).to(torch.int32).to(dev)
    for _ in range(3):
        pa.pa_copy_blocks(k, v, pairs)
    torch.cuda.synchronize()
    del k, v


def _host_threads() -> int:
    return len(os.sched_getaffinity(0))


def _run_rows(fn, rows, threads: int, seconds: float):
    """Run fn(row) over rows, in batches of `threads` rows on that many host
    threads, until the rows are done or `seconds` have passed; returns (rows
    done, elapsed seconds)."""
    from concurrent.futures import ThreadPoolExecutor
    done = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while done < len(rows):
            batch = rows[done:done + threads]
            list(ex.map(fn, batch))
            done += len(batch)
            if time.perf_counter() - t0 >= seconds:
                break
    return done, time.perf_counter() - t0


def cpu_baseline(w_host, step_bytes: int, seconds: float) -> dict:
    """The float64 oracle, as it stands, on the host's cores: the decode of
    the step's (sequence, query head) rows, each row one oracle call on that
    head's slice of the pools (decode_ref; decode_gqa_ref with its K/V head;
    decode_fp8_ref on the 8-bit codes), rows in sequence order.  Run once with
    one host thread per core (BLAS and torch limited to one thread each, rows
    spread over the threads) and once on a single thread, each for about
    `seconds` or until every row is done; the rate is the step's algorithmic
    bytes times the fraction of its context tokens covered, over the time."""
    from threadpoolctl import threadpool_limits
    from oracle import decode_fp8_ref, decode_gqa_ref, decode_ref
    lens, fmt, q = w_host["lens"], w_host["fmt"], w_host["q"]
    S, H = q.shape[0], q.shape[1]
    G = H // w_host["k"].shape[1]
    rows = [(s, h) for s in range(S) for h in range(H)]
    total_tokens = float(lens.astype(np.int64).sum()) * H

    def row(sh):
        s, h = sh
        kv = h // G
        qa, ta, la = q[s:s + 1, h:h + 1], w_host["tables"][s:s + 1], lens[s:s + 1]
        k, v = w_host["k"][:, kv:kv + 1], w_host["v"][:, kv:kv + 1]
        if fmt is not None:
            decode_fp8_ref(qa, k, v, w_host["ks"][:, kv:kv + 1], w_host["vs"][:, kv:kv + 1], ta, la,
                           w_host["scale"], w_host["bs"], fmt)
        elif G > 1:
            decode_gqa_ref(qa, k, v, ta, la, w_host["scale"], w_host["bs"])
        else:
            decode_ref(qa, k, v, ta, la, w_host["scale"], w_host["bs"])

    def rate(n, t):
        toks = float(sum(int(lens[s]) for s, _ in rows[:n]))
        return step_bytes * (toks / total_tokens) / t / 1e9, toks

    cores = _host_threads()
    prev = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        with threadpool_limits(limits=1):
            n_all, t_all = _run_rows(row, rows, cores, seconds)
            n_one, t_one = _run_rows(row, rows, 1, seconds)
    finally:
        torch.set_num_threads(prev)
    v_all, tok_all = rate(n_all, t_all)
    v_one, tok_one = rate(n_one, t_one)
    return {"value": round(v_all, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": (f"float64 numpy oracle over the first {n_all} of the step's {len(rows)} (sequence, head) "
                       f"rows ({tok_all / total_tokens:.1%} of its context tokens) in {t_all:.1f} s on "
                       f"{cores} host threads, one row per oracle call; scaled to the step's bytes"),
            "cores_1": {"value": round(v_one, 4), "unit": "GB/s", "cores": 1,
                        "sample": (f"the first {n_one} rows ({tok_one / total_tokens:.1%} of the context tokens) "
                                   f"in {t_one:.1f} s on one host thread")}}


HOST_LINK_GBS = 64.0           # PCIe 5.0 x16, per direction (published)


def swap_bench(pa, dev, steps: int, warmup: int) -> dict:
    """pa_swap_blocks between the layer-shape device pools and pinned host
    pools: 256 scattered blocks out (device -> host), then back in, 128 KiB
    per block per pool (64 MiB each way).  Beside it, two ways the same bytes
    could move with the DMA engines: one hipMemcpyAsync per block and pool
    (torch copy_), and a single contiguous copy of 64 MiB (the host link's
    practical ceiling for this direction)."""
    from paged_kv_cache_186_amd import workloads as W
    w = W.layer_shape(0, device=dev)
    nblk = 256
    rng = np.random.default_rng(1)
    dev_ids = rng.choice(w.num_blocks, size=nblk, replace=False).astype(np.int32)
    host_ids = rng.permutation(nblk).astype(np.int32)
    shape = (nblk,) + tuple(w.k_pool.shape[1:])
    hk = torch.empty(shape, dtype=w.dtype, pin_memory=True)
    hv = torch.empty(shape, dtype=w.dtype, pin_memory=True)
    out_map = torch.from_numpy(np.stack([dev_ids, host_ids], 1)).to(dev)
    in_map = torch.from_numpy(np.stack([host_ids, dev_ids], 1)).to(dev)
    nbytes = 2 * nblk * w.k_pool[0].numel() * w.k_pool.element_size()
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    res = {}
    res["out_kernel"] = timed(lambda: pa.pa_swap_blocks(hk, hv, w.k_pool, w.v_pool, out_map))
    res["in_kernel"] = timed(lambda: pa.pa_swap_blocks(w.k_pool, w.v_pool, hk, hv, in_map))
    di, hi = dev_ids.tolist(), host_ids.tolist()

    def per_block(out: bool):
        for d, h in zip(di, hi):
            if out:
                hk[h].copy_(w.k_pool[d], non_blocking=True)
                hv[h].copy_(w.v_pool[d], non_blocking=True)
            else:
                w.k_pool[d].copy_(hk[h], non_blocking=True)
                w.v_pool[d].copy_(hv[h], non_blocking=True)
    res["out_memcpy_per_block"] = timed(lambda: per_block(True))
    res["in_memcpy_per_block"] = timed(lambda: per_block(False))
    flat_d = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    flat_h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    res["out_one_memcpy"] = timed(lambda: flat_h.copy_(flat_d, non_blocking=True))
    res["in_one_memcpy"] = timed(lambda: flat_d.copy_(flat_h, non_blocking=True))
    # the kernel's result must equal the oracle's byte copy
    from oracle import swap_blocks_ref
    pa.pa_swap_blocks(hk, hv, w.k_pool, w.v_pool, out_map)
    torch.cuda.synchronize()
    rk, _ = swap_blocks_ref(torch.zeros_like(hk), torch.zeros_like(hv), w.k_pool.cpu(), w.v_pool.cpu(),
                            out_map.cpu().numpy())
    if not torch.equal(hk.view(torch.int16), rk.view(torch.int16)):
        raise RuntimeError("swap out differs from the oracle")
    gbs = {k: round(nbytes / (v * 1e-3) / 1e9, 2) for k, v in res.items()}
    return {
        "metric": "pa_swap_blocks: host-link GB/s swapping 256 scattered KV blocks (K+V, 64 MiB) "
                  "out to pinned host memory and back, 1 MI355X",
        "value": round((gbs["out_kernel"] + gbs["in_kernel"]) / 2, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(res["out_kernel"] + res["in_kernel"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded N(0,1) layer-shape pools)",
        "config": {"workload": "swap of 256 of the 1024 layer-shape blocks (32 heads x 16 x 128 fp16, "
                               "K and V: 128 KiB each per block)", "bytes_each_way": nbytes},
        "gb_per_s": gbs, "ms": {k: round(v, 4) for k, v in res.items()},
        "roofline": {"bound": "host link", "achieved": round((gbs["out_kernel"] + gbs["in_kernel"]) / 2, 2),
                     "peak": HOST_LINK_GBS, "unit": "GB/s",
                     "frac": round((gbs["out_kernel"] + gbs["in_kernel"]) / 2 / HOST_LINK_GBS, 4),
                     "traffic": None},
    }


PEAK_MFMA_16BIT_TFLOPS = 2500.0  # MI355X dense fp16 / bf16 matrix peak (published)

from paged_kv_cache_186_amd.workloads import QUERY_OPS  # noqa: E402


def queries_bench(pa, dev, op: str, steps: int, warmup: int, seed: int, heads: int, cpu: bool,
                  cpu_seconds: float, partition: int = 0) -> dict:
    """One call of pa_prefill / pa_decode_mla per step, cold cache (pool
    replicas rotated), HIP-graph replays timed with HIP events."""
    from paged_kv_cache_186_amd import workloads as W
    calibration_copy(pa, dev)
    qw = W.query_workload(op, seed, dev, heads)
    S, H, Hkv, D, Dv, bs, dtype, tq = qw.S, qw.H, qw.Hkv, qw.D, qw.Dv, qw.bs, qw.dtype, qw.tq
    mla = qw.mla
    lens, tables_np, qs_np, T, width, scale = qw.lens, qw.tables_np, qw.qs_np, qw.T, qw.width, qw.scale
    tables = torch.from_numpy(tables_np).to(dev)
    clens = torch.from_numpy(lens.astype(np.int32)).to(dev)
    qs = torch.from_numpy(qs_np).to(dev)
    base, q = qw.pools, qw.q
    out = torch.empty((T, H, Dv), dtype=dtype, device=dev)
    pool_bytes = sum(t.numel() * t.element_size() for t in base)
    R = max(1, math.ceil(COLD_BYTES / pool_bytes))
    reps = [base] + [tuple(t.clone() for t in base) for _ in range(R - 1)]
    ws_need = (pa.pa_decode_mla_workspace_size(S, H, width, bs, partition) if mla
               else pa.pa_prefill_workspace_size(S, T, H, Hkv, D, width, bs, partition))
    ws = pa.new_workspace(ws_need, dev)
    log(f"{op}: {S} seqs, context {int(lens.min())}..{int(lens.max())} ({int(lens.sum())} tokens), "
        f"{tq} query tokens each, {H} query / {Hkv} K/V heads, D={D}, BS={bs}, {dtype}; "
        f"{R} pool replicas ({R * pool_bytes / 2**30:.2f} GiB)")

    def call(i):
        if mla:
            pa.pa_decode_mla(out, q, reps[i % R][0], tables, clens, scale, bs, partition_size=partition,
                             workspace=ws)
        else:
            kp, vp = reps[i % R]
            pa.pa_prefill(out, q, kp, vp, tables, clens, qs, scale, bs, partition_size=partition, workspace=ws)

    for i in range(max(1, warmup)):
        call(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    graphs = capture_steps(call, R, steps)
    call(R - 1)
    torch.cuda.synchronize()
    want = out.clone()
    graphs[0].replay()
    torch.cuda.synchronize()
    if not torch.equal(out.view(torch.int16), want.view(torch.int16)):
        raise RuntimeError("graph replay differs from the eager call")
    ms = time_steps(graphs, steps, stream)

    # algorithmic work: every (query row, visible key) pair once
    e = 2
    pairs = int(sum(sum(int(L) - tq + i + 1 for i in range(tq)) for L in lens))   # per query head
    flops = pairs * H * 2 * (D + Dv)
    kv_rows = int(lens.sum())
    bytes_ = (kv_rows * Hkv * (D if mla else 2 * D) * e + T * H * (D + Dv) * e
              + 4 * int(sum(-(-int(L) // bs) for L in lens)) + 4 * S + (4 * (S + 1) if not mla else 0))
    t = ms * 1e-3
    tflops = flops / t / 1e12
    gbs = bytes_ / t / 1e9
    mfma_bound = op == "prefill"
    digest = kernel_source_digest(PF_SOURCES)
    tag = op + (f"_h{H}" if heads else "") + (f"_p{partition}" if partition else "")
    # pa_decode_mla takes mla_heads_kernel under the default split for up to
    # 512 sequences
    # pa_prefill takes its row-block kernel with the default split when the
    # 128-row blocks of (sequence, K/V head) rows fill the GPU (the same test
    # the library makes)
    # and the grouped-query decode kernel for at most 64 sequences with at most
    # 16 (32 for groups above 16) query rows per sequence and K/V head on average
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    group = H // Hkv
    tiles = not partition and Hkv * (T * group // 128) >= cus and T * group >= 64 * S
    few = not partition and S <= 64 and T * group <= (32 if group > 16 else 16) * S
    kernel = (("mla_heads_kernel" if not partition and S <= 512 else "mla_split_kernel") if mla
              else "decode_mfma_kernel" if few
              else ("prefill_tile_kernel" if tiles else "prefill_kernel"))
    traffic = traffic_from_profile(digest, os.path.join(PROFILES, f"{kernel}_{tag}_traffic.txt"))
    metric = {"prefill": "chunked prefill over the paged cache (pa_prefill): achieved TFLOP/s, 1 MI355X",
              "verify": "speculative verification over the paged cache (pa_prefill): achieved HBM GB/s, 1 MI355X",
              "verify1": "one-token queries through pa_prefill: achieved HBM GB/s, 1 MI355X",
              "mla": "MLA latent-cache decode (pa_decode_mla): achieved HBM GB/s, 1 MI355X"}[op]
    result = {
        "metric": metric,
        "value": round(tflops if mfma_bound else gbs, 2),
        "unit": "TFLOP/s" if mfma_bound else "GB/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16" if dtype == torch.float16 else "bf16",
        "data": "synthetic (seeded N(0,1) q/K/V, seeded lengths and block layout)",
        "config": {"partition": partition or "library default",
                   "workload": f"{op}: {S} seqs x {tq} query tokens, context {int(lens.min())}..{int(lens.max())}, "
                               f"{H} query / {Hkv} K/V heads, D={D}{' (latent, values 512)' if mla else ''}, "
                               f"BS={bs}",
                   "context_tokens": kv_rows, "query_rows": T,
                   "cache": f"cold: rotates {R} pool replicas", "parallelism": "none (1 GPU)"},
        "us_per_step": round(ms * 1e3, 3),
        "flops_per_step": flops, "bytes_per_step": bytes_,
        "achieved": {"TFLOP/s": round(tflops, 2), "GB/s": round(gbs, 2)},
        "roofline": ({"bound": "mfma", "kernel": kernel, "achieved": round(tflops, 2),
                      "peak": PEAK_MFMA_16BIT_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(tflops / PEAK_MFMA_16BIT_TFLOPS, 4), "traffic": traffic,
                      "kernel_source_sha": digest}
                     if mfma_bound else
                     {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 2),
                      "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                      "traffic": traffic, "kernel_source_sha": digest}),
    }
    if cpu:
        result["cpu_baseline"] = queries_cpu_baseline(op, reps[0], q, tables_np, lens, qs_np, scale, bs, H, Hkv,
                                                      D, Dv, tq, mfma_bound, cpu_seconds)
    return result


def queries_cpu_baseline(op, pools, q, tables_np, lens, qs_np, scale, bs, H, Hkv, D, Dv, tq, mfma_bound,
                         seconds):
    """The float64 oracle on the host's cores, on a bounded sample: units of
    work are (sequence, K/V head) pairs for prefill / verify (the sequence's
    query rows of that K/V head's query heads, one prefill_ref call each) and
    sequences for MLA (one mla_decode_ref call each), in order.  Run once on
    one host thread per core (BLAS and torch limited to one thread each) and
    once on a single thread, each for about `seconds` or until every unit is
    done; the rate is the work of the units done over the time, in the
    metric's unit."""
    from threadpoolctl import threadpool_limits
    from oracle import mla_decode_ref, prefill_ref
    G = H // Hkv
    S = len(lens)
    qh = q.cpu()
    if op == "mla":
        pool = pools[0].cpu()
        units = list(range(S))

        def run(s):
            mla_decode_ref(qh[s:s + 1], pool, tables_np[s:s + 1], lens[s:s + 1], scale, bs, Dv)

        def work(s):
            L = int(lens[s])
            return L * H * 2 * (D + Dv) if mfma_bound else L * D * 2 + H * (D + Dv) * 2
        what = "sequences (one mla_decode_ref call each, all heads)"
    else:
        kp, vp = pools[0].cpu(), pools[1].cpu()
        units = [(s, kvh) for s in range(S) for kvh in range(Hkv)]

        def run(u):
            s, kvh = u
            rows = slice(int(qs_np[s]), int(qs_np[s + 1]))
            n = int(qs_np[s + 1] - qs_np[s])
            prefill_ref(qh[rows, kvh * G:(kvh + 1) * G], kp[:, kvh:kvh + 1], vp[:, kvh:kvh + 1],
                        tables_np[s:s + 1], lens[s:s + 1], np.array([0, n], np.int32), scale, bs)

        def work(u):
            s, _ = u
            L, n = int(lens[s]), int(qs_np[s + 1] - qs_np[s])
            pairs = sum(L - n + i + 1 for i in range(n)) * G
            return pairs * 2 * (D + Dv) if mfma_bound else L * D * 2 * 2 + n * G * D * 2 * 2
        what = "(sequence, K/V head) pairs (one prefill_ref call each over that head's query rows)"
    cores = _host_threads()
    prev = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        with threadpool_limits(limits=1):
            n_all, t_all = _run_rows(run, units, cores, seconds)
            n_one, t_one = _run_rows(run, units, 1, seconds)
    finally:
        torch.set_num_threads(prev)
    div = 1e12 if mfma_bound else 1e9
    unit = "TFLOP/s" if mfma_bound else "GB/s"
    v_all = sum(work(u) for u in units[:n_all]) / t_all / div
    v_one = sum(work(u) for u in units[:n_one]) / t_one / div
    return {"value": round(v_all, 6), "unit": unit, "cores": cores, "kind": "oracle",
            "sample": f"float64 numpy oracle over the first {n_all} of {len(units)} {what}, "
                      f"{t_all:.1f} s on {cores} host threads",
            "cores_1": {"value": round(v_one, 6), "unit": unit, "cores": 1,
                        "sample": f"the first {n_one} units in {t_one:.1f} s on one host thread"}}


def capture_steps(enqueue_step, R: int, K: int):
    """Graphs for exactly K steps: `full` holds steps 0..R-1 (one per pool
    replica) and is replayed K // R times, `rest` holds steps 0..K % R - 1
    (None when K is a multiple of R)."""
    full = capture(lambda: [enqueue_step(i) for i in range(R)])
    r = K % R
    rest = capture(lambda: [enqueue_step(i) for i in range(r)]) if r else None
    return full, K // R, rest


def time_steps(graphs, K: int, stream) -> float:
    """Milliseconds per step over exactly K steps: HIP events on the kernels'
    stream around K // R replays of the R-step graph and one replay of the
    remainder graph."""
    full, n_full, rest = graphs
    full.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(n_full):
        full.replay()
    if rest is not None:
        rest.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / K


# The headline run also measures these decode configurations (same library
# defaults, fewer steps) and reports them under "configs": the pages' layer
# shape, continuous batching, the 128K context at batch 1, and the 4 x 128K
# batch with explicit partitions of 512 tokens.
EXTRA_CONFIGS = [("layer_shape", 0), ("continuous_batching", 0), ("long_context_b1", 0),
                 ("long_context_b4", 512)]
DEFAULT_WORKLOAD = "long_context_b4"


def decode_bench(pa, dev, args, workload: str, partition: int, steps: int, warmup: int,
                 cpu: bool, full: bool = True) -> dict:
    """One decode step (pa_reshape_and_cache of each sequence's current token,
    then pa_decode) on a workload, cold cache, exactly `steps` timed steps."""
    from paged_kv_cache_186_amd import workloads as W
    stream = torch.cuda.current_stream(dev)
    log(f"building workload {workload} (seed {args.seed})")
    w = build_workload(workload, args.seed, dev)
    Hkv = args.kv_heads or w.num_heads
    gqa = Hkv != w.num_heads
    if gqa:
        if w.num_heads % Hkv:
            raise SystemExit(f"--kv-heads {Hkv} does not divide {w.num_heads} query heads")
        w.k_pool = w.k_pool[:, :Hkv].contiguous()
        w.v_pool = w.v_pool[:, :Hkv].contiguous()
        torch.cuda.empty_cache()
    fp8 = args.kv != "native"
    host = None
    if fp8:
        # the 8-bit cache holds the same values, quantized (input generation)
        kc, vc, ks, vs = W.fp8_pools(w, args.kv)
        if cpu:
            host = {"k": kc.cpu().view(torch.uint8).numpy(), "v": vc.cpu().view(torch.uint8).numpy(),
                    "ks": ks.cpu().numpy(), "vs": vs.cpu().numpy()}
        w.k_pool = w.v_pool = None
        torch.cuda.empty_cache()
    elif cpu:
        host = {"k": w.k_pool.cpu(), "v": w.v_pool.cpu()}
    log(describe(w) + (f", KV cache fp8 {args.kv}" if fp8 else "") + (f", {Hkv} K/V heads" if gqa else ""))
    e = w.q.element_size()
    e_kv = 1 if fp8 else e
    S, H, D, bs = w.num_seqs, w.num_heads, w.head_dim, w.block_size
    lens = w.context_lens_np()
    tables = w.block_tables().to(dev)
    clens = w.context_lens().to(dev)

    # the token decoded this step is the last one of each context: its K/V are
    # (re)written into its slot, then attention runs over the whole context
    slots = [w.manager.slot_of(s, int(lens[i]) - 1) for i, s in enumerate(w.seq_ids)]
    q = w.q
    _, k_new, v_new = W.new_token_values(w, 0)
    k_new, v_new = k_new[:, :Hkv].contiguous(), v_new[:, :Hkv].contiguous()
    slot_t = torch.tensor(slots, dtype=torch.int32, device=dev)

    base = (kc, vc, ks, vs) if fp8 else (w.k_pool, w.v_pool)
    pool_bytes = sum(t.numel() * t.element_size() for t in base)
    R = args.replicas or max(1, math.ceil(COLD_BYTES / pool_bytes))
    log(f"pool K+V {pool_bytes / 2**20:.0f} MiB; {R} replica(s) for cold-cache timing")
    reps = [base] + [tuple(t.clone() for t in base) for _ in range(R - 1)]
    out = torch.empty_like(q)
    ws_bytes = (pa.pa_decode_gqa_workspace_size(S, H, Hkv, D, w.table_width, bs, partition, q.dtype,
                                                 base[0].dtype) if gqa
                else pa.pa_decode_workspace_size(S, H, D, w.table_width, bs, partition))
    ws = pa.new_workspace(ws_bytes, dev)

    if full:
        calibration_copy(pa, dev)

    def reshape(i):
        if fp8:
            pa.pa_reshape_and_cache_fp8(*reps[i % R], k_new, v_new, slot_t)
        else:
            pa.pa_reshape_and_cache(*reps[i % R], k_new, v_new, slot_t)

    def decode(i):
        if gqa:
            kp, vp = reps[i % R][:2]
            kss, vss = (reps[i % R][2:] if fp8 else (None, None))
            pa.pa_decode_gqa(out, q, kp, vp, tables, clens, w.scale, bs, k_scales=kss, v_scales=vss,
                             partition_size=partition, workspace=ws)
        elif fp8:
            kp, vp, kss, vss = reps[i % R]
            pa.pa_decode_fp8(out, q, kp, vp, kss, vss, tables, clens, w.scale, bs,
                             partition_size=partition, workspace=ws)
        else:
            kp, vp = reps[i % R]
            pa.pa_decode(out, q, kp, vp, tables, clens, w.scale, bs,
                         partition_size=partition, workspace=ws)

    def step(i):
        reshape(i)
        decode(i)

    # eager warmup, then HIP graphs of the steps (one per replica), replayed,
    # so no host-side launch cost sits inside the timed region
    log(f"warmup {warmup} steps (eager)")
    for i in range(max(1, warmup)):
        step(i)
    torch.cuda.synchronize()
    eager = time_eager(reshape, decode, min(steps, 200), stream) if full else None

    step_graphs = capture_steps(step, R, steps)
    decode_graphs = capture_steps(decode, R, steps)
    check_graph_replays(decode_graphs[0], decode, R, out)

    log(f"timing {steps} cold steps ({decode_graphs[1]} replays of a {R}-step graph"
        + (f" and one of {steps % R} steps)" if steps % R else ")"))
    step_ms = time_steps(step_graphs, steps, stream)
    dec_ms = time_steps(decode_graphs, steps, stream)
    warm_ms = None
    if full and R > 1:
        log(f"timing {steps} warm steps")
        warm_ms = time_steps(capture_steps(lambda i: step(0), R, steps), steps, stream)

    b_dec = decode_bytes(lens, H, D, e, bs, e_kv, Hkv)
    b_res = reshape_bytes(S, Hkv, D, e, e_kv)
    step_s = step_ms * 1e-3
    value = (b_dec + b_res) / step_s / 1e9
    dec_gbs = b_dec / (dec_ms * 1e-3) / 1e9
    digest = kernel_source_digest()
    tag = workload + (f"_p{partition}" if partition else "")
    traffic = traffic_from_profile(digest, profile_path(tag, args.kv, Hkv if gqa else 0))
    split = "balanced (partition_size 0)" if partition == 0 else f"partitions of {partition} tokens"
    cache = (f"cold: rotates {R} pool replicas ({R * pool_bytes / 2**30:.2f} GiB)" if R > 1 else
             f"cold: the {pool_bytes / 2**30:.2f} GiB pool exceeds the 256 MB last-level cache")

    if not full:
        return {"workload": describe(w), "split": split, "steps": steps,
                "us_per_step": round(step_ms * 1e3, 3), "value": round(value, 2), "unit": "GB/s",
                "pct_of_hbm_peak": round(100 * value / PEAK_HBM_GBS, 2),
                "pa_decode_us": round(dec_ms * 1e3, 3), "pa_decode_bytes": b_dec,
                "roofline_frac": round(dec_gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                "cache": cache}

    # the shared-prefix workload's copy-on-write (pa_copy_blocks of the pairs
    # that made the last shared block private), cold, one call per replica
    cow = None
    if getattr(w, "cow_pairs", None) and not fp8 and not gqa:
        pairs = torch.tensor(w.cow_pairs, dtype=torch.int32, device=dev)
        cow_ms = time_steps(capture_steps(lambda i: pa.pa_copy_blocks(*reps[i % R][:2], pairs), R, steps),
                            steps, stream)
        b_cow = 2 * 2 * len(w.cow_pairs) * bs * Hkv * D * e  # K and V, read + write
        cow = {"pairs": len(w.cow_pairs), "bytes_per_call": b_cow, "us_per_call": round(cow_ms * 1e3, 3),
               "GB/s": round(b_cow / (cow_ms * 1e-3) / 1e9, 2),
               "timing": "HIP graph of one call per pool replica, HIP events around the replays"}

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {2: "f16" if w.dtype == torch.float16 else "bf16", 4: "f32"}[e]
                 + (f" (KV cache fp8 {args.kv}, per-block scales)" if fp8 else ""),
        "data": "synthetic (seeded N(0,1) q/K/V, seeded lengths and block layout)",
        "config": {
            "workload": describe(w),
            "seed": args.seed,
            "num_seqs": S, "num_heads": H, "head_dim": D, "block_size": bs,
            "context_tokens": int(lens.sum()),
            "kv_cache": "native" if not fp8 else f"fp8 {args.kv} + fp32 scale per (block, head)",
            "kv_heads": Hkv,
            "split": split,
            "accumulate": "f32",
            "cache": cache,
            "timing": "HIP graph replays of the steps, HIP events around the replays",
            "parallelism": "none (1 GPU)",
        },
        "us_per_step": round(step_ms * 1e3, 3),
        "pct_of_hbm_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "sequence_heads_per_s": round(S * H / step_s, 1),
        "bytes_per_step": {"pa_decode": b_dec, "pa_reshape_and_cache": b_res},
        "kernels_us": {"pa_decode": round(dec_ms * 1e3, 3),
                       "pa_reshape_and_cache_and_gaps": round((step_ms - dec_ms) * 1e3, 3)},
        "eager_us": {k: round(v * 1e3, 3) for k, v in eager.items()},
        "roofline": {"bound": "hbm", "kernel": "pa_decode (one kernel launch per call)",
                     "achieved": round(dec_gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "kernel_source_sha": digest},
    }
    if warm_ms is not None:
        result["warm"] = {"value": round((b_dec + b_res) / (warm_ms * 1e-3) / 1e9, 2),
                          "us_per_step": round(warm_ms * 1e3, 3),
                          "note": "no replica rotation: the working set can sit in the last-level cache"}
    if cow is not None:
        result["copy_blocks"] = cow
    del reps, base, ws
    w.k_pool = w.v_pool = None
    torch.cuda.empty_cache()
    result["roofline"]["achievable_copy_GB/s"] = round(copy_ceiling(dev), 1)
    if cpu:
        log(f"cpu baseline: oracle for ~{args.cpu_seconds:.0f} s on all host cores, then on one thread")
        host.update({"q": q.cpu(), "tables": w.block_tables_np(), "lens": lens, "scale": w.scale,
                     "bs": bs, "fmt": args.kv if fp8 else None})
        result["cpu_baseline"] = cpu_baseline(host, b_dec + b_res, args.cpu_seconds)
        del host
    return result


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    choices=["layer_shape", "continuous_batching", "shared_prefix",
                             "long_context_b1", "long_context_b4", "tiny"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--kv", default="native", choices=["native", "e4m3", "e5m2"],
                    help="KV cache element format: the workload's own dtype, or an 8-bit cache "
                         "(OCP E4M3 / E5M2 with per-block, per-head scales; q and out keep their dtype)")
    ap.add_argument("--partition", type=int, default=0, help="partition tokens (0 = library default)")
    ap.add_argument("--replicas", type=int, default=0, help="KV pool replicas (0 = enough for 2 GiB)")
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="K/V heads (0 = as many as query heads); fewer runs grouped-query decode "
                         "(pa_decode_gqa) over the first kv-heads heads of the pools")
    ap.add_argument("--op", default="decode", choices=["decode", "swap", "prefill", "verify", "verify1", "mla"],
                    help="decode: the decode step (default); swap: pa_swap_blocks over the host link; "
                         "prefill / verify: pa_prefill on a prompt-chunk / drafted-token workload; "
                         "mla: pa_decode_mla")
    ap.add_argument("--heads", type=int, default=0, help="query heads for --op prefill/verify/mla (0 = default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="measure only --workload (the default run also measures the other decode configs)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures a single GPU; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        return 2

    import paged_kv_cache_186_amd as pa
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pa.load_library()

    if args.op == "swap":
        print(json.dumps(swap_bench(pa, dev, min(args.steps, 50), min(args.warmup, 5))), flush=True)
        return 0
    if args.op in QUERY_OPS:
        print(json.dumps(queries_bench(pa, dev, args.op, args.steps, min(args.warmup, 10), args.seed, args.heads,
                                       not args.no_cpu_baseline, args.cpu_seconds, args.partition)), flush=True)
        return 0

    result = decode_bench(pa, dev, args, args.workload, args.partition, args.steps, args.warmup,
                          not args.no_cpu_baseline)
    extras = (not args.no_extra and args.workload == DEFAULT_WORKLOAD and args.partition == 0
              and args.kv == "native" and not args.kv_heads)
    if extras:
        result["configs"] = {}
        for name, part in EXTRA_CONFIGS:
            key = name + (f"_partitions_{part}" if part else "")
            result["configs"][key] = decode_bench(pa, dev, args, name, part, min(args.steps, 200),
                                                  min(args.warmup, 10), False, full=False)
            torch.cuda.empty_cache()
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
