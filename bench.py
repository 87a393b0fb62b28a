#!/usr/bin/env python3
"""Throughput of the copy-on-write paged KV cache on one MI355X.

Default run, one JSON line. The headline is decode attention over the MCTS
tree, the deepest and widest of the workloads: a 4096-token root prompt, a
binary tree of depth 6 grown by fork + append with 32 tokens of K/V per edge,
all 64 leaves decoded at once over all 32 layers (32 query heads / 8 KV
heads, head_dim 128, block_size 16, bf16 K/V and q; root blocks are held by
64 leaves, depth-k edges by 64/2^k). ``value`` = the unique K/V bytes the
call must read (distinct blocks x valid slots x 4096 B x 32 layers =
1,065,353,216 B) divided by the wall time of a call, in GB/s. ``roofline``
prices the call's two attention launches (the wide-row launch over the
shared root and the narrow launch over each leaf's path, which also writes
the outputs) over their summed average durations, measured with HIP events
on the launch stream, and lists each launch's own fraction.
``cpu_baseline`` times the CPU oracle on a sample of layers of the same
inputs, and ``parity`` compares one whole layer of the timed output with
the oracle (the run exits with status 3 if any check fails).

Nested under ``configs``, measured in the same run: the beam search decode
step (fork every beam, append one token with a copy-on-write of the shared
15/16-full tail, attention over 32 layers, free), agent decode (4 requests
sharing 13,312 tokens + 32,768 private each, head_dim 256) and the
draft-tree verify (4 requests x 32,768 context + 48-node tree) with its
commit leg; each with its own roofline and parity check. ``ceiling`` is a
plain device read and copy of 2 GiB, for scale.

``--workload beam|mcts|agent|verify|prompt_cache`` runs one workload alone
(for profiler runs and counters).
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

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak of MI355X
METRIC = "unique-KV HBM GB/s (% of peak) and branch-queries/sec, paged decode attn"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


KERNEL_SOURCES = ("kernels.hip", "tree.hip", "wide_spec.hip", "kernel_common.h", "attn_plan.h", "schedule.hpp",
                  "schedule.cpp", "api.cpp")


def code_only(text: str) -> str:
    """C/C++ source without comments and with whitespace runs collapsed, so
    that a change to comments alone keeps the hash (string literals, which
    hold the inline assembly, are kept as written)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"' or c == "'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(read=None) -> str:
    """sha256 (first 16 hex) of the code (comments dropped) of the kernels,
    the planner that cuts their work and the entry points that set its
    defaults: all of it decides the HBM traffic. read(name) returns a
    file's text (default: the working tree)."""
    if read is None:
        def read(name):
            with open(os.path.join(ROOT, "paged_kv_cache_amd", "csrc", name), encoding="utf-8") as f:
                return f.read()
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update(code_only(read(name)).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed counter runs, if they were
    taken on the current kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))[workload]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("kernel_hash") != kernel_source_hash() or \
            sorted(str(rec.get("kernel")).split("+")) != sorted(kernel.split("+")):
        return None
    return rec.get("bytes_per_launch")


def record_traffic(workload: str, fetch_dir: str, write_dir: str, source: str) -> dict:
    """Turns two rocprofv3 --pmc runs of this bench (FETCH_SIZE, then
    WRITE_SIZE, each with --calibrate-copy) into the per-launch HBM bytes of
    the attention kernels and stores them in profiles/traffic.json under
    the current kernel source hash. The counters are scaled by what they
    read for the calibration copy (1 GiB read, 1 GiB written)."""
    import csv
    import glob

    def rows(d, counter):
        out = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter:
                    out.append((r["Kernel_Name"], float(r["Counter_Value"])))
        if not out:
            raise SystemExit(f"no {counter} rows under {d}")
        return out

    res = {"kernel": None, "kernel_hash": kernel_source_hash(), "source": source}
    total = 0.0
    names = []
    for counter, d, key in (("FETCH_SIZE", fetch_dir, "read"), ("WRITE_SIZE", write_dir, "write")):
        rr = rows(d, counter)
        copy_kib = max(v for n, v in rr if "copyBuffer" in n)
        scale = round((1 << 30) / (copy_kib * 1024) * 4) / 4   # to a quarter: 2.0 / 1.0 here
        per = 0.0
        names = []
        for kname in ("attn_mfma_kernel", "attn_wide_kernel", "attn_tree_kernel"):
            vals = [v for n, v in rr if kname in n]
            if vals:
                names.append(kname)
                per += sum(vals) / len(vals) * 1024 * scale
                res[f"dispatches_{kname}"] = len(vals)
        res[f"{key}_bytes"] = int(per)
        res[f"{'fetch' if key == 'read' else 'write'}_scale"] = scale
        total += per
    res["kernel"] = "+".join(names)
    res["bytes_per_launch"] = int(total)
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        data = {}
    data[workload] = res
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")
    return res


def warm_up(args, step, torch, min_seconds: float = 0.3):
    """W untimed steps, continued until min_seconds have passed: a fresh GPU
    needs a fraction of a second of load before its clocks settle."""
    t0 = time.perf_counter()
    done = 0
    while done < args.warmup or time.perf_counter() - t0 < min_seconds:
        step()
        done += 1
        if done % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def timing_on(c, step, names, torch, n):
    """Switches the pool's kernel timing on, then runs n steps whose readings
    are dropped, n at least the steps of the pass to be measured: launches
    that create the pool's timing events (the first timed launches, one event
    pair each) read long (the MCTS root ~15%: 233 against 203 us), so the
    measured pass reuses events made here."""
    c.set_option("timing", 1)
    for _ in range(n):
        step()
    torch.cuda.synchronize()
    for k in names:
        c.timing_read(k)


def to_dev(t):
    import torch
    if t.dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(t.raw)).cuda()
    return torch.from_numpy(np.ascontiguousarray(t.raw).view(np.int16)).cuda().view(torch.bfloat16)


def unique_tokens(cache, seqs) -> int:
    valid = {}
    for s in seqs:
        n = cache.length(s)
        for j, b in enumerate(cache.table(s)):
            valid[b] = min(cache.BS, n - j * cache.BS)
    return sum(valid.values())


def percentiles(xs):
    """p10, p50, p90 of per-step durations (ms), nearest rank."""
    if not xs:
        return None
    ys = sorted(xs)
    pick = lambda p: ys[min(len(ys) - 1, int(p * (len(ys) - 1) + 0.5))]  # noqa: E731
    return [round(pick(0.1), 5), round(pick(0.5), 5), round(pick(0.9), 5)]


# largest plan the library passes in the kernel launches' own arguments
INLINE_PLAN_BYTES = 12288


def side_bytes(sh, n_layers, n_rows, info):
    """Bytes a decode moves beside the unique K/V, per call: the queries
    (n_layers x n_rows x Hq x D in the K/V dtype), the float32 output, the
    float32 partial states (D values + running max and sum per partial row
    and plane, written by attention and read by the combine) and the plan
    records (in the launch arguments when they fit in 12,288 bytes and the
    combine's lists in 1,024, else copied to the device before the
    launches)."""
    eb = 2 if sh.dtype == "bf16" else 4
    q = n_layers * n_rows * sh.Hq * sh.D * eb
    out = n_layers * n_rows * sh.Hq * sh.D * 4
    part = 2 * info["partial_rows"] * n_layers * sh.Hkv * (sh.D + 2) * 4
    plan = info["plan_bytes"]
    return {"q": q, "out": out, "partials": part, "plan": plan,
            "plan_in_launch_args": plan <= INLINE_PLAN_BYTES}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [d.get("num_threads", 0) for d in threadpool_info() if d.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:
        pass
    return os.cpu_count() or 1


# ------------------------------------------------------------ oracle legs

MAX_ABS, REL_L2 = 2e-3, 1e-2   # the parity bar of the test suite


def oracle_pool(w, inp):
    """The oracle's pool run through the workload's trace (test
    infrastructure: used here for the cpu_baseline and parity legs only,
    outside the timed regions)."""
    from oracle.pool import OraclePool, run_trace
    kv = {i: (k, v) for i, _s, k, v in inp.appends}
    pool = OraclePool(w.num_blocks_bound() + 8, w.shape.BS)
    run_trace(pool, w.ops, lambda i: (kv[i][0].f32(), kv[i][1].f32()))
    return pool


def compare(got, want) -> dict:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    ma = float(np.max(np.abs(got - want)))
    rl = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    ok = bool(np.all(np.isfinite(got)) and ma <= MAX_ABS and rl <= REL_L2)
    return {"max_abs": float(f"{ma:.3e}"), "rel_l2": float(f"{rl:.3e}"), "ok": ok}


def parity_decode(pool, w, inp, got, layer) -> dict:
    """One whole layer of a decode output (every branch and query head)
    against the oracle's float64 result."""
    import oracle
    want = oracle.decode(pool, list(w.query_sids), inp.q.f32(), w.softmax_scale, layers=[layer])[0]
    res = compare(got[layer], want)
    res.update(layer=layer, rows=int(want.shape[0] * want.shape[1]))
    return res


def parity_verify(pool, w, inp, got, req, nodes) -> dict:
    """Some tree nodes of one verify request (every query head) against the
    oracle: node i sees the request's context and its own root path."""
    import oracle
    K, V = pool.kv(w.query_sids[req], layer=0)
    ctx = K.shape[0] - w.n_nodes
    qf = inp.q.f32()
    G = w.shape.G
    gs, ws = [], []
    for i in nodes:
        idx = np.concatenate([np.arange(ctx), ctx + np.asarray(oracle.ancestors(inp.parents[req], i))])
        for g in range(w.shape.Hkv):
            ws.append(oracle.attention._softmax_attend(qf[req, i, g * G:(g + 1) * G], K[idx, g],
                                                        V[idx, g], w.softmax_scale))
            gs.append(got[req, i, g * G:(g + 1) * G])
    res = compare(np.concatenate(gs), np.concatenate(ws))
    res.update(request=req, nodes=list(map(int, nodes)), rows=len(nodes) * w.shape.Hq)
    return res


def cpu_baseline_decode(pool, w, q, uniq_bytes_per_layer: int, budget_s: float) -> dict:
    """The oracle (float64 numpy) timed on the same inputs (q: float32
    [L][B][Hq][D]): whole layers of the decode (every branch and head), one
    after another, until the time budget is used (at least one layer)."""
    import oracle
    sids = list(w.query_sids)
    done = 0
    t0 = time.perf_counter()
    while True:
        oracle.decode(pool, sids, q, w.softmax_scale, layers=[done % w.shape.L])
        done += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or dt / done * (done + 1) > 2 * budget_s:
            break
    return {"value": round(uniq_bytes_per_layer * done / dt / 1e9, 4), "unit": "GB/s",
            "cores": blas_threads(), "kind": "oracle", "cpu": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{done} whole layer(s) of the decode ({len(sids)} branches x {w.shape.Hq} "
                      f"heads each), same inputs, float64 numpy, {dt:.1f} s",
            "branch_queries_per_s": round(len(sids) * done / dt, 1)}


# ------------------------------------------------------------------ beam

def setup_beam(pkv, torch):
    from workloads import generate, get
    w = get("beam")
    sh = w.shape
    inp = generate(w)
    nb = 128 + 8 * 16 + 8 + 16
    c = pkv.PagedKVCache(nb, sh.BS, sh.L, sh.Hkv, sh.Hq, sh.D, dtype=sh.dtype)
    apply_options(c)
    root_k, root_v = inp.appends[0][2], inp.appends[0][3]
    root = c.create()
    c.append([root], [2048], to_dev(root_k), to_dev(root_v))
    beams = [c.fork(root) for _ in range(8)]
    c.free(root)
    step_k, step_v = [], []
    for i, b in enumerate(beams):
        k, v = inp.appends[1 + i][2], inp.appends[1 + i][3]
        kd, vd = to_dev(k), to_dev(v)
        c.append([b], [255], kd[:, :255].contiguous(), vd[:, :255].contiguous())
        step_k.append(kd[:, 255:256])
        step_v.append(vd[:, 255:256])
    step_k = torch.cat(step_k, dim=1).contiguous()     # [L][8][Hkv][D]
    step_v = torch.cat(step_v, dim=1).contiguous()
    q = to_dev(inp.q)
    out = torch.empty((sh.L, 8, sh.Hq, sh.D), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    return w, inp, c, beams, step_k, step_v, q, out


def beam_step(c, beams, step_k, step_v, q, out, scale, keep=False):
    kids = c.fork_many(beams)
    c.append(kids, [1] * len(kids), step_k, step_v)
    c.decode(kids, q, scale=scale, out=out)
    if keep:
        return kids
    c.free_many(kids)
    return None


def plan_host_us(c, seqs, n_layers) -> float:
    """Host time of one decode plan (segments, chunks, items), median of 21:
    the plan cache is keyed by the sequence list, so alternating its order
    forces a rebuild each call (the same work either way)."""
    ts = []
    rev = list(seqs)[::-1]
    for i in range(21):
        t0 = time.perf_counter()
        c.plan_info(rev if i & 1 else seqs, n_layers)
        ts.append(time.perf_counter() - t0)
    c.plan_info(seqs)
    return round(sorted(ts)[len(ts) // 2] * 1e6, 1)


def fork_ns(c, seq, n=4096, reps=5) -> dict:
    """Host cost of fork and of free, per sequence: n forks of one sequence
    in one C call (pkv_seq_fork_many, the argument arrays built beforehand,
    so the library's loop is what is timed), then one pkv_seq_free_many;
    best of reps."""
    from paged_kv_cache_amd import _lib
    parents = (_lib.PkvSeq * n)(*([seq] * n))
    kids = (_lib.PkvSeq * n)()
    best_f = best_d = float("inf")
    for _ in range(reps):
        t0 = time.perf_counter()
        _lib.check(_lib.lib.pkv_seq_fork_many(c.handle, parents, n, kids))
        t1 = time.perf_counter()
        _lib.check(_lib.lib.pkv_seq_free_many(c.handle, kids, n))
        t2 = time.perf_counter()
        best_f, best_d = min(best_f, t1 - t0), min(best_d, t2 - t1)
    return {"table_blocks": len(c.table(seq)), "fork_ns": round(best_f / n * 1e9, 1),
            "free_ns": round(best_d / n * 1e9, 1)}


def per_layer_launches(c, seqs, q, out, scale, n_layers, torch, reps=5) -> dict:
    """The secondary figure: the same decode as n_layers single-layer calls
    (each plans, uploads and launches for its layer). Device time is the
    summed attention + combine launches per pass (HIP events); wall time
    includes the host work of every call."""
    names = ("attention", "attention_wide", "combine")

    def one_pass():
        for l in range(n_layers):
            c.decode(seqs, q[l:l + 1], layer0=l, n_layers=1, scale=scale, out=out[l:l + 1])

    one_pass()
    torch.cuda.synchronize()
    for k in names:
        c.timing_read(k)
    c.set_option("timing", 1)
    t0 = time.perf_counter()
    for _ in range(reps):
        one_pass()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / reps
    c.set_option("timing", 0)
    dev = {k: c.timing_read(k)[0] / reps for k in names}
    return {"launches_per_pass": n_layers,
            "attention_ms": round(dev["attention"] + dev["attention_wide"], 4),
            "combine_ms": round(dev["combine"], 4), "wall_ms": round(wall * 1e3, 4)}


def run_beam(args, pkv, torch, cpu_baseline=True):
    w, inp, c, beams, step_k, step_v, q, out = setup_beam(pkv, torch)
    sh = w.shape
    scale = w.softmax_scale
    # plan facts, from a step kept alive
    kids = beam_step(c, beams, step_k, step_v, q, out, scale, keep=True)
    torch.cuda.synchronize()
    uniq_tok = unique_tokens(c, kids)
    info = c.plan_info(kids)
    assert info["unique_tokens"] == uniq_tok, (info, uniq_tok)
    c.free_many(kids)
    uniq_bytes = uniq_tok * sh.token_kv_bytes * sh.L
    warm_up(args, lambda: beam_step(c, beams, step_k, step_v, q, out, scale), torch)
    # timed region: K steps, no timing events (they add commands to the stream)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        beam_step(c, beams, step_k, step_v, q, out, scale)
    t_host = time.perf_counter() - t0
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    got = out.cpu().numpy()     # the last timed step's output
    # kernel durations: the same K steps again with start/end events on every kernel
    timing_on(c, lambda: beam_step(c, beams, step_k, step_v, q, out, scale),
              ("attention", "combine", "append"), torch, args.steps)
    for _ in range(args.steps):
        beam_step(c, beams, step_k, step_v, q, out, scale)
    torch.cuda.synchronize()
    ktimes = {k: c.timing_read(k) for k in ("attention", "combine", "append")}
    # and once more, read back after each step for the spread of the attention
    # time (the synchronization idles the GPU between steps, so the average
    # above comes from the unsynchronized run)
    per_step = []
    for _ in range(args.steps):
        beam_step(c, beams, step_k, step_v, q, out, scale)
        torch.cuda.synchronize()
        ms, n = c.timing_read("attention")
        per_step.append(ms / max(n, 1))
    c.set_option("timing", 0)
    for kname in ("combine", "append"):
        c.timing_read(kname)
    layered = plan_us = forks = None
    kids = beam_step(c, beams, step_k, step_v, q, out, scale, keep=True)
    torch.cuda.synchronize()
    if args.secondary:
        layered = per_layer_launches(c, kids, q, out, scale, sh.L, torch)
    plan_us = plan_host_us(c, kids, sh.L)
    forks = fork_ns(c, kids[0])
    c.free_many(kids)
    if args.calibrate_copy:
        calibrate_copy(torch)
    ms_step = dt / args.steps * 1e3
    value = uniq_bytes / (dt / args.steps) / 1e9
    attn_ms, attn_n = ktimes["attention"]
    attn_avg_s = attn_ms / max(attn_n, 1) / 1e3
    achieved = uniq_bytes / attn_avg_s / 1e9
    traffic = measured_traffic("beam", "attn_mfma_kernel")
    cow_bytes = 8 * 2 * sh.L * sh.Hkv * 15 * sh.D * 2
    append_ms = ktimes["append"][0] / max(ktimes["append"][1], 1)
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "beam search decode step: 8 beams x (2048 shared + 256 private tokens), "
                               "fork + copy-on-write append + attention over 32 layers + free",
                   "beams": 8, "shared_prompt_tokens": 2048, "private_tokens": 256, "layers": 32,
                   "q_heads": sh.Hq, "kv_heads": sh.Hkv, "head_dim": sh.D, "block_size": sh.BS,
                   "parallelism": "single GPU"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "branch_queries_per_s": round(8 * sh.L / (dt / args.steps), 1),
        "unique_kv_bytes_per_step": uniq_bytes,
        "kernel_ms": {k: round(v[0] / max(v[1], 1), 5) for k, v in ktimes.items()},
        "attention_ms_p10_p50_p90": percentiles(per_step),
        "host_ms_per_step": round(t_host / args.steps * 1e3, 4),
        "plan_host_us": plan_us,
        "per_layer_launches": layered,
        "fork": forks,
        # the step's copy-on-write: 8 partly filled tails (15 of 16 slots) copied
        # for every layer and KV head, K and V (bytes read = bytes written)
        "cow": {"ops": 8, "bytes_read": cow_bytes, "append_ms": round(append_ms, 5),
                "GB_s": round(2 * cow_bytes / (append_ms / 1e3) / 1e9, 1)},
        "plan": info,
        "other_bytes_per_step": side_bytes(sh, sh.L, 8, info),
        "roofline": {"bound": "hbm", "kernel": "attn_mfma_kernel", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
    }
    c.close()
    pool = oracle_pool(w, inp)
    res["parity"] = parity_decode(pool, w, inp, got, layer=sh.L - 1)
    if cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decode(pool, w, inp.q.f32(), uniq_bytes // sh.L,
                                                  args.cpu_budget)
    return res


def calibrate_copy(torch):
    """A plain device copy of known size (1 GiB read + 1 GiB written), for
    scaling the HBM counters. A 1 GiB fill of another buffer in between
    evicts the source from the 256 MB last-level cache."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    flush = torch.empty_like(a)
    a.fill_(1)
    flush.fill_(2)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b, flush


def ceiling(torch, pkv=None, reps=10) -> dict:
    """What plain device streaming reaches on this GPU, for scale beside the
    8 TB/s peak: the library's streaming read of 2 GiB (pkv_stream_read,
    16-byte loads over every CU, non-temporal and ordinary), a 2 GiB bf16
    reduction (reads 2 GiB) and a 2 GiB copy (reads and writes 2 GiB), torch's
    own kernels; HIP events, best of reps. Buffers far larger than the 256 MB
    last-level cache."""
    n = 1 << 30
    a = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best(fn):
        fn()
        t = float("inf")
        for _ in range(reps):
            ev0.record()
            fn()
            ev1.record()
            ev1.synchronize()
            t = min(t, ev0.elapsed_time(ev1) / 1e3)
        return t

    t_read = best(lambda: a.sum(dtype=torch.float32))
    t_copy = best(lambda: b.copy_(a))
    out = {"read_GB_s": round(2 * n / t_read / 1e9, 1), "copy_GB_s": round(4 * n / t_copy / 1e9, 1),
           "bytes": 2 * n, "how": "torch.sum over 2 GiB bf16 (read) and a 2 GiB copy (read + write), "
                                  "best of 10, HIP events"}
    if pkv is not None:
        from paged_kv_cache_amd import binding
        sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
        for key, nt in (("stream_read_nt_GB_s", True), ("stream_read_GB_s", False)):
            t = best(lambda: binding.pkv_stream_read(a, sink, streaming=nt))
            out[key] = round(2 * n / t / 1e9, 1)
        out["how_stream"] = ("pkv_stream_read over the same 2 GiB: 16-byte loads, four in flight per "
                             "lane, 8192 workgroups each reading a contiguous range; non-temporal (as "
                             "the attention kernels read K/V that one wave uses) and ordinary loads")
    del a, b
    return out


# --------------------------------------------------------- other trees

def build_tree(pkv, w, inp, extra_blocks=0):
    sh = w.shape
    c = pkv.PagedKVCache(w.num_blocks_bound() + 8 + extra_blocks, sh.BS, sh.L, sh.Hkv, sh.Hq, sh.D,
                         dtype=sh.dtype)
    apply_options(c)
    kv = {i: (k, v) for i, _s, k, v in inp.appends}
    h = {}
    for i, op in enumerate(w.ops):
        if op.kind == "create":
            h[op.sid] = c.create()
        elif op.kind == "fork":
            h[op.sid] = c.fork(h[op.parent])
        elif op.kind == "append":
            c.append([h[op.sid]], [op.n], to_dev(kv[i][0]), to_dev(kv[i][1]))
        else:
            c.free(h.pop(op.sid))
    return c, h


def run_tree(args, pkv, torch, name, cpu_baseline=False):
    from workloads import generate, get
    w = get(name)
    sh = w.shape
    inp = generate(w)
    # verify: room for the contexts to grow by the committed paths
    extra = len(w.query_sids) * (COMMIT_STEPS * w.n_nodes // sh.BS + 2) if w.kind == "verify" else 0
    c, h = build_tree(pkv, w, inp, extra)
    seqs = [h[s] for s in w.query_sids]
    q = to_dev(inp.q)
    res, got = time_attention(args, c, seqs, q, w, torch, f"{w.name}: {w.note}",
                              inp.parents if w.kind == "verify" else None)
    if w.kind != "verify":
        res["plan_host_us"] = plan_host_us(c, seqs, sh.L)
        res["fork"] = fork_ns(c, seqs[0])
        if sh.L > 1 and args.secondary:
            out = torch.empty((sh.L, len(seqs), sh.Hq, sh.D), dtype=torch.float32, device="cuda")
            res["per_layer_launches"] = per_layer_launches(c, seqs, q, out, w.softmax_scale, sh.L, torch)
    if w.kind == "verify":
        res["commit"] = commit_leg(
            c, seqs, w, inp, lambda: c.verify(seqs, inp.parents, q, scale=w.softmax_scale), torch)
    c.close()
    pool = oracle_pool(w, inp)
    if w.kind == "verify":
        import oracle
        # the first request's deepest node, its root and six more
        depth = [len(oracle.ancestors(inp.parents[0], i)) for i in range(w.n_nodes)]
        nodes = sorted({0, int(np.argmax(depth)), *np.random.default_rng(5).choice(w.n_nodes, 6,
                                                                                   replace=False)})
        res["parity"] = parity_verify(pool, w, inp, got, 0, nodes)
    else:
        res["parity"] = parity_decode(pool, w, inp, got, layer=0)
    if cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decode(pool, w, inp.q.f32(),
                                                  res["unique_kv_bytes_per_step"] // sh.L,
                                                  args.cpu_budget)
    return res


def time_attention(args, c, seqs, q, w, torch, workload: str, parents=None):
    """Times decode (or, with parents, verify) over seqs: wall time per call
    and each kernel's device time from HIP events. Returns the record and
    the output of the last timed call (host copy)."""
    sh = w.shape
    uniq_tok = unique_tokens(c, seqs)
    uniq_bytes = uniq_tok * sh.token_kv_bytes * sh.L
    if parents is not None:
        out = torch.empty((len(seqs), w.n_nodes, sh.Hq, sh.D), dtype=torch.float32, device="cuda")
        fn = lambda: c.verify(seqs, parents, q, scale=w.softmax_scale, out=out)  # noqa: E731
        n_queries = len(seqs) * w.n_nodes
    else:
        out = torch.empty((sh.L, len(seqs), sh.Hq, sh.D), dtype=torch.float32, device="cuda")
        fn = lambda: c.decode(seqs, q, scale=w.softmax_scale, out=out)  # noqa: E731
        n_queries = len(seqs) * sh.L
    warm_up(args, fn, torch)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fn()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    got = out.cpu().numpy()
    names = ("attention", "attention_wide", "attention_tree", "combine")
    timing_on(c, fn, names, torch, args.steps)
    for _ in range(args.steps):
        fn()
    torch.cuda.synchronize()
    # per call: summed device time of each kernel kind (0 if it did not run)
    kt = {k: v[0] / args.steps for k, v in ((k, c.timing_read(k)) for k in names)}
    # the spread, from a run read back after each call
    per_call = []
    for _ in range(args.steps):
        fn()
        torch.cuda.synchronize()
        per_call.append(sum(c.timing_read(k)[0]
                            for k in ("attention", "attention_wide", "attention_tree")))
    c.set_option("timing", 0)
    c.timing_read("combine")
    if args.calibrate_copy:
        calibrate_copy(torch)
    # the attention bytes are split between the narrow and the wide launch:
    # price the pair, over their summed durations, and each launch over its
    # own share of the unique tokens
    parts = [n for k, n in (("attention_tree", "attn_tree_kernel"), ("attention_wide", "attn_wide_kernel"),
                            ("attention", "attn_mfma_kernel")) if kt[k] > 0]
    kernel = "+".join(parts)
    attn_s = (kt["attention"] + kt["attention_wide"] + kt["attention_tree"]) / 1e3
    achieved = uniq_bytes / attn_s / 1e9
    info = c.plan_info(seqs) if parents is None else None
    launches = {}
    if info is not None and kt["attention_tree"] > 0:
        # one launch reads every unique token once; its matrix-core work is
        # 4*D flop per (query row, token of that row's sequence)
        gbs = uniq_bytes / (kt["attention_tree"] / 1e3) / 1e9
        flop = 4 * sh.D * sh.Hq * sh.L * sum(c.length(s) for s in seqs)
        tf = flop / (kt["attention_tree"] / 1e3) / 1e12
        launches["attn_tree_kernel"] = {
            "unique_bytes": int(uniq_bytes), "ms": round(kt["attention_tree"], 5),
            "GB_s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
            "mfma_TFLOP_s": round(tf, 1), "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
    elif info is not None:
        wide_bytes = info["wide_tokens"] * sh.token_kv_bytes * sh.L
        for k, n, b in (("attention_wide", "attn_wide_kernel", wide_bytes),
                        ("attention", "attn_mfma_kernel", uniq_bytes - wide_bytes)):
            if kt[k] > 0:
                gbs = b / (kt[k] / 1e3) / 1e9
                launches[n] = {"unique_bytes": int(b), "ms": round(kt[k], 5), "GB_s": round(gbs, 1),
                               "frac": round(gbs / HBM_PEAK_GBS, 4)}
        if kt["attention_wide"] > 0:
            # matrix-core rate of the wide launch, 4*D flop per (query row, token)
            rows = sum(1 for _ in seqs) * sh.G  # every branch's rows read the wide chunks
            flop = 4 * sh.D * rows * info["wide_tokens"] * sh.Hkv * sh.L
            tf = flop / (kt["attention_wide"] / 1e3) / 1e12
            launches["attn_wide_kernel"]["mfma_TFLOP_s"] = round(tf, 1)
            launches["attn_wide_kernel"]["mfma_frac"] = round(tf / MFMA_BF16_PEAK_TFLOPS, 4)
    rec = {
        "metric": METRIC, "value": round(uniq_bytes / dt / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(dt * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "q_heads": sh.Hq, "kv_heads": sh.Hkv, "head_dim": sh.D,
                   "block_size": sh.BS, "layers": sh.L, "branches": len(seqs),
                   "parallelism": "single GPU"},
        "pct_of_hbm_peak": round(100 * uniq_bytes / dt / 1e9 / HBM_PEAK_GBS, 2),
        "branch_queries_per_s": round(n_queries / dt, 1),
        "unique_kv_bytes_per_step": uniq_bytes,
        "kernel_ms": {k: round(v, 5) for k, v in kt.items()},
        "attention_ms_p10_p50_p90": percentiles(per_call),
        "plan": info,
        "other_bytes_per_step": side_bytes(sh, sh.L, len(seqs), info) if info else None,
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(w.name, kernel), "launches": launches or None},
        "mfma": mfma_rate(c, seqs, w, parents, attn_s) if parents is not None else None,
    }
    return rec, got


def mfma_rate(c, seqs, w, parents, attn_s):
    """Matrix-core rate of a verify launch: 4*D flop per (query row, token
    of its request) by definition (Q.K and P.V; the tree's few masked nodes
    included), and 6*D as issued (P enters P.V as a bf16 pair)."""
    sh = w.shape
    rows = w.n_nodes * sh.G                      # query rows per (request, KV head)
    tokens = sum(c.length(s) for s in seqs)      # the kernel reads every token for every row
    row_tok = rows * tokens * sh.Hkv
    algo = 4 * sh.D * row_tok / attn_s / 1e12
    issued = 6 * sh.D * row_tok / attn_s / 1e12
    return {"unit": "TFLOP/s", "peak": MFMA_BF16_PEAK_TFLOPS, "algorithmic": round(algo, 1),
            "issued": round(issued, 1), "frac_algorithmic": round(algo / MFMA_BF16_PEAK_TFLOPS, 4),
            "frac_issued": round(issued / MFMA_BF16_PEAK_TFLOPS, 4)}


def run_prompt_cache(args, pkv, torch):
    """The agent workload's tree built through the prompt cache instead of
    forks: agent 0 computes the system prompt and snapshots it; agents 1-3
    resume from the longest cached prefix of their own prompt and compute
    only the rest. Reports the cache's host latency and the prompt tokens
    it saves, then times decode over the four agents."""
    from workloads import get
    w = get("agent")
    sh = w.shape
    n_sys, n_agents, n_priv = 13312, 4, 32768
    c = pkv.PagedKVCache(w.num_blocks_bound() + 8, sh.BS, sh.L, sh.Hkv, sh.Hq, sh.D, dtype=sh.dtype)
    apply_options(c)
    rng = np.random.default_rng(3)
    system = rng.integers(0, 32000, size=n_sys).astype(np.int32)
    prompts = [np.concatenate([system, rng.integers(0, 32000, size=n_priv).astype(np.int32)])
               for _ in range(n_agents)]
    kv = torch.randn((sh.L, n_sys + n_priv, sh.Hkv, sh.D), device="cuda").to(torch.bfloat16)
    seqs, computed, match_s, insert_s = [], 0, [], []
    for a in range(n_agents):
        t0 = time.perf_counter()
        s, m = c.cache_match(prompts[a])
        match_s.append(time.perf_counter() - t0)
        n = len(prompts[a]) - m
        c.append([s], [n], kv[:, m:].contiguous(), kv[:, m:].contiguous())
        computed += n
        t0 = time.perf_counter()
        c.cache_insert(s, prompts[a])
        insert_s.append(time.perf_counter() - t0)
        seqs.append(s)
    torch.cuda.synchronize()
    total = sum(len(p) for p in prompts)
    q = torch.randn((sh.L, n_agents, sh.Hq, sh.D), device="cuda").to(torch.bfloat16)
    res, _ = time_attention(args, c, seqs, q, w, torch,
                            f"agents resumed from the prompt cache: {n_agents} x ({n_sys} cached "
                            f"system-prompt tokens + {n_priv} own tokens), block_size {sh.BS}")
    entries, _ = c.cache_info()
    res["prompt_cache"] = {
        "prompt_tokens_computed": computed, "prompt_tokens_total": total,
        "saved_pct": round(100 * (1 - computed / total), 1), "entries": entries,
        "match_us_median": round(1e6 * float(np.median(match_s[1:])), 1),
        "insert_us_median": round(1e6 * float(np.median(insert_s)), 1),
        "blocks_per_prompt": len(prompts[0]) // sh.BS}
    c.close()
    return res


COMMIT_STEPS = 20


def commit_leg(c, seqs, w, inp, verify, torch):
    """Speculative steps after the timed verify calls: every request keeps a
    random root path of its tree (one batch commit for all requests), then a
    new tree of the same shape is appended and verified. Reports the
    commit's wall time per step (host planning included) and its kernels'
    device time."""
    sh = w.shape
    R, N = len(seqs), w.n_nodes
    rng = np.random.default_rng(11)
    kv = torch.randn((sh.L, R * N, sh.Hkv, sh.D), device="cuda").to(torch.bfloat16)
    paths = []
    for _ in range(COMMIT_STEPS):
        step = []
        for r in range(R):
            leaf, path = int(rng.integers(N)), []
            while leaf != -1:
                path.append(leaf)
                leaf = int(inp.parents[r][leaf])
            step.append(path[::-1])
        paths.append(step)
    for k in ("commit_gather", "append"):
        c.timing_read(k)
    c.set_option("timing", 1)
    wall = gather = append = 0.0
    for i in range(COMMIT_STEPS):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        c.commit_batch(seqs, inp.parents, paths[i])
        torch.cuda.synchronize()
        wall += time.perf_counter() - t0
        gather += c.timing_read("commit_gather")[0]
        append += c.timing_read("append")[0]
        c.append(seqs, [N] * R, kv, kv)
        verify()
        c.timing_read("append")
    torch.cuda.synchronize()
    c.set_option("timing", 0)
    kept = sum(len(p) for st in paths for p in st) / COMMIT_STEPS
    return {"steps": COMMIT_STEPS, "requests": R, "kept_tokens_per_step": kept,
            "ms_per_step": round(wall * 1e3 / COMMIT_STEPS, 4),
            "gather_ms": round(gather / COMMIT_STEPS, 5), "append_ms": round(append / COMMIT_STEPS, 5)}


NESTED_KEYS = ("value", "unit", "ms_per_step", "pct_of_hbm_peak", "branch_queries_per_s",
               "unique_kv_bytes_per_step", "kernel_ms", "attention_ms_p10_p50_p90", "roofline",
               "mfma", "parity", "cow", "commit", "fork", "plan_host_us", "host_ms_per_step",
               "per_layer_launches")


def nested(rec) -> dict:
    out = {"workload": rec["config"]["workload"]}
    out.update({k: rec[k] for k in NESTED_KEYS if rec.get(k) is not None})
    return out


def run_all(args, pkv, torch):
    """The headline (MCTS decode) with the other configs nested in the same
    record; every leg checks one layer (or some tree nodes) of its timed
    output against the oracle."""
    def note(msg):
        print(msg, file=sys.stderr, flush=True)

    note("bench: mcts (headline)")
    head = run_tree(args, pkv, torch, "mcts", cpu_baseline=not args.no_cpu_baseline)
    head["config"]["workload"] = (
        "MCTS tree decode: 4096-token root, binary tree of depth 6 (32 tokens per edge), all 64 "
        "leaves decoded at once over 32 layers; 32 q heads / 8 KV heads, head_dim 128, block_size "
        "16, bf16")
    configs = {}
    for name in ("beam_step", "agent", "verify"):
        note(f"bench: {name}")
        rec = run_beam(args, pkv, torch, cpu_baseline=False) if name == "beam_step" \
            else run_tree(args, pkv, torch, name)
        configs[name] = nested(rec)
        torch.cuda.empty_cache()
    head["configs"] = configs
    note("bench: ceiling")
    head["ceiling"] = ceiling(torch, pkv)
    return head


OPTIONS: list = []   # --option key=value, applied to every pool the bench makes


def apply_options(c) -> None:
    """Planner and kernel options given as --option key=value."""
    for kv in OPTIONS:
        k, v = kv.split("=", 1)
        c.set_option(k, int(v))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="all",
                    choices=["all", "beam", "mcts", "agent", "verify", "prompt_cache"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--option", action="append", default=[], metavar="KEY=VALUE",
                    help="a pool option (pkv_pool_set_option) for every pool the bench makes")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--secondary", action="store_true",
                    help="also time the same decode as single-layer launches (its launches "
                         "would mix into a profiler's per-kernel averages)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling HBM counters)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="store the HBM bytes of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) "
                         "of this workload in profiles/traffic.json, then exit (no GPU needed)")
    ap.add_argument("--traffic-source", default="", help="the profile summary to cite")
    args = ap.parse_args()
    OPTIONS.extend(args.option)
    if args.record_traffic:
        print(json.dumps(record_traffic(args.workload, *args.record_traffic, args.traffic_source)))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    import paged_kv_cache_amd as pkv
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.workload == "all":
        res = run_all(args, pkv, torch)
    elif args.workload == "beam":
        res = run_beam(args, pkv, torch, cpu_baseline=not args.no_cpu_baseline)
    elif args.workload == "prompt_cache":
        res = run_prompt_cache(args, pkv, torch)
    else:
        res = run_tree(args, pkv, torch, args.workload, cpu_baseline=not args.no_cpu_baseline)
    print(json.dumps(res), flush=True)
    checks = [res.get("parity")] + [r.get("parity") for r in res.get("configs", {}).values()]
    if any(c is not None and not c["ok"] for c in checks):
        print("bench.py: a timed output does not match the oracle", file=sys.stderr)
        sys.exit(3)


if __name__ == "__main__":
    main()
