#!/usr/bin/env python3
"""Benchmark of batch-invariant paged-KV causal GQA prefill attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints ONE JSON line. A step is one pass of the whole attention path over one batch (the
prefill kernel, plus the merge kernel when rows span several 4096-token splits); the plan and
its work-list upload are made once per batch shape, outside the timed region, as a model
reuses them for every layer (their host / upload times are reported separately).

value     extend KV GB/s: 16 requests, each extending 1-4 tokens behind a 1024-token prefix
          (32 q / 8 kv heads, head_dim 128, bf16, page 16). Every request owns a private copy
          of its prefix pages and 8 such pools are rotated across steps (> 512 MB), so the
          256 MB Infinity Cache cannot serve the KV: logical KV bytes / step time.
prefill   cold 16 x 1028-token causal prefill, same shapes: causal FLOPs / step time.
others    the remaining configurations, each timed and its cached-vs-full bits checked: the
          67-token prompt (full prefill vs 3-token extend, latency), the mixed batch (3,700-token
          prefill + 7 cached tails, causal TFLOP/s), the long fp8 path (24/4/256, 8k and 32k
          prefills and a 1k extend behind 31k cached keys: TFLOP/s and workspace bytes),
          head_dim 512 (16/4/512 prefill and extends) and the cold prefill at page sizes 1, 2,
          12 and 16 (TFLOP/s).
decode    8 one-token decodes over 8k-128k keys each (same shapes, 2-32 KV splits a row, the
          split partials merged): logical KV bytes / step time (1.4 GB of KV, far past the
          Infinity Cache).
roofline  the extend kernel against HBM (8 TB/s), and against a measured ceiling: the
          read-only streaming reference (dpp_stream_kv) gathering the same pages with no
          compute; prefill's own against bf16 MFMA peak.
cpu_baseline  the fp64 CPU oracle on the same extend batch, repeated for ~10 s.
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

HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "extend_16x1-4_behind_1024_counters.json")
KERNEL_SOURCES = ["deterministic_paged_prefill_amd/csrc/prefill.hip",
                  "deterministic_paged_prefill_amd/csrc/dpp_internal.h"]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def causal_flops(batch, hq: int, d: int) -> float:
    """4 * d * Hq * sum over query rows of (p + 1) keys: QK^T and PV, causal work only."""
    total = 0
    for r in batch.requests:
        a = r.kv_len - r.qo_len  # position of the first query row
        # sum_{p=a}^{kv_len-1} (p + 1)
        total += (r.kv_len * (r.kv_len + 1) - a * (a + 1)) // 2
    return 4.0 * d * hq * total


def kv_bytes(batch, hkv: int, d: int, elem: int) -> int:
    """Logical KV bytes: every request's K and V rows read once."""
    return sum(r.kv_len for r in batch.requests) * hkv * d * 2 * elem


class Runner:
    """Pre-resolved dpp_run arguments so the timed loop is one C call per step."""

    def __init__(self, work, batch, replicas: int = 1, cap: int = 256 << 20, adaptive: bool = False):
        import torch

        import deterministic_paged_prefill_amd as dpp
        self.dpp = dpp
        self.lib = dpp.library()
        self.work = work
        self.batch = batch
        t0 = time.perf_counter()
        self.plan = dpp.plan(work.num_qo_heads, work.num_kv_heads, work.head_dim, work.page_size,
                             batch.qo_indptr, batch.kv_indptr, batch.kv_last_page_len,
                             kv_dtype=work.kv_dtype, k_scale=work.k_scale, v_scale=work.v_scale,
                             workspace_cap=cap, adaptive_kv_tile=adaptive)
        self.plan_us = (time.perf_counter() - t0) * 1e6
        dev = torch.device("cuda")
        P = work.num_pages
        # replica i: the whole pool copied to pages [i*P, (i+1)*P), page ids shifted by i*P
        self.k = work.k_pool.to(dev).repeat(replicas, 1, 1, 1).contiguous()
        self.v = work.v_pool.to(dev).repeat(replicas, 1, 1, 1).contiguous()
        base = torch.from_numpy(batch.kv_indices).to(dev)
        self.kvi = [(base + i * P).contiguous() for i in range(replicas)]
        self.q = batch.q.to(dev)
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((self.q.shape[0], work.num_qo_heads), dtype=torch.float32, device=dev)
        self.ws = self.plan.new_workspace(dev)
        self.stream = torch.cuda.current_stream()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        self.plan.upload(self.ws, self.stream)
        torch.cuda.synchronize()
        self.upload_us = (time.perf_counter() - t0) * 1e6
        self.replicas = replicas
        self.args = [(self.plan._h, self.q.data_ptr(), self.q.shape[0], self.k.data_ptr(),
                      self.v.data_ptr(), self.k.shape[0], kvi.data_ptr(), kvi.numel(), self.o.data_ptr(),
                      self.lse.data_ptr(), self.ws.data_ptr(), self.ws.numel(),
                      dpp.RUN_REUSE_UPLOAD, self.stream.cuda_stream) for kvi in self.kvi]

    def step(self, i: int) -> None:
        st = self.lib.dpp_run(*self.args[i % self.replicas])
        if st != 0:
            self.dpp._check(st)

    def timed(self, steps: int, warmup: int):
        import torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record(self.stream)
        for i in range(steps):
            self.step(warmup + i)
        end.record(self.stream)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3
        return start.elapsed_time(end) / steps, wall_ms / steps

    def replan_us(self, n: int = 20) -> tuple:
        """Host cost of a new batch of the same shape, as a serving loop pays it every batch:
        (plan us, upload us) medians over n rounds, each plan destroyed before the next (its
        pinned staging block goes back to the library's pool), into a workspace of its own."""
        import numpy as np
        import torch
        w, b = self.work, self.batch
        ws = self.plan.new_workspace("cuda")
        plan_t, up_t = [], []
        for _ in range(n):
            t0 = time.perf_counter()
            p = self.dpp.plan(w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                              b.qo_indptr, b.kv_indptr, b.kv_last_page_len, kv_dtype=w.kv_dtype,
                              k_scale=w.k_scale, v_scale=w.v_scale)
            t1 = time.perf_counter()
            p.upload(ws, self.stream)
            torch.cuda.synchronize()
            t2 = time.perf_counter()
            p.close()
            plan_t.append(t1 - t0)
            up_t.append(t2 - t1)
        return float(np.median(plan_t) * 1e6), float(np.median(up_t) * 1e6)

    def stream_timed(self, split: int, depth: int, steps: int, warmup: int, head_split: bool = False) -> float:
        """ms per launch of the read-only streaming reference (dpp_stream_kv) over the same pages,
        rotated like the attention steps."""
        import torch
        flags = self.dpp.RUN_REUSE_UPLOAD | (self.dpp.STREAM_HEAD_SPLIT if head_split else 0)
        args = [(self.plan._h, self.k.data_ptr(), self.v.data_ptr(), self.k.shape[0], kvi.data_ptr(),
                 kvi.numel(), self.ws.data_ptr(), self.ws.numel(), split, depth, flags,
                 self.stream.cuda_stream) for kvi in self.kvi]
        for i in range(warmup):
            self.dpp._check(self.lib.dpp_stream_kv(*args[i % self.replicas]))
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(self.stream)
        for i in range(steps):
            self.lib.dpp_stream_kv(*args[(warmup + i) % self.replicas])
        end.record(self.stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    def stream_ceiling(self, steps: int, warmup: int, same_gather: bool = False) -> dict:
        """Best of the streaming reference's grids (1 or 2 workgroups per unit, 4 or 8 loads in
        flight per wave): the measured ceiling of this gather on this GPU."""
        best = None
        for split in (1, 2):
            for depth in (4, 8):
                ms = self.stream_timed(split, depth, steps, warmup)
                if best is None or ms < best[0]:
                    best = (ms, split, depth)
        # the gather of the head_dim-split attention launch itself: two workgroups per unit, each
        # all of K and half of V
        out = dict(ms=best[0], split=best[1], depth=best[2])
        if same_gather:
            same = min((self.stream_timed(2, depth, steps, warmup, head_split=True), depth) for depth in (4, 8))
            out.update(same_gather_ms=same[0], same_gather_depth=same[1])
        return out

    def graph_timed(self, steps_per_graph: int, replays: int):
        """The same steps captured in one HIP graph (torch.cuda.graph over dpp_run, work list
        uploaded beforehand) and replayed: ms per step."""
        import torch
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            for i in range(steps_per_graph):
                args = list(self.args[i % self.replicas])
                args[-1] = side.cuda_stream
                st = self.lib.dpp_run(*args)
                if st != 0:
                    self.dpp._check(st)
        torch.cuda.synchronize()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(replays):
            g.replay()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / (replays * steps_per_graph)

    def outputs(self, replica: int = 0):
        import torch
        self.step(replica)
        torch.cuda.synchronize()
        return self.o.cpu(), self.lse.cpu()


def traffic_from_profile(launch_bytes: float):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel source (else None)."""
    try:
        with open(PROFILE_COUNTERS) as f:
            prof = json.load(f)
    except (OSError, ValueError):
        return None
    if prof.get("kernel_source_sha256_16") != kernel_hash():
        return None
    # each counter scaled by the bytes a plain device copy of known size moves per KiB it reads
    return (prof["fetch_kib_per_dispatch"] * prof["fetch_bytes_per_kib"] +
            prof["write_kib_per_dispatch"] * prof["write_bytes_per_kib"])


def cpu_baseline(work, batch, budget_s: float):
    import oracle
    oracle.build(force=False)
    kw = work.oracle_kwargs(batch)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.paged_prefill(**kw)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    gb = kv_bytes(batch, work.num_kv_heads, work.head_dim, 2) * reps / 1e9
    return {"value": round(gb / el, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"the whole extend batch ({batch.num_q_tokens} query tokens x "
                      f"{work.num_qo_heads} heads over 1025-1028 keys each), fp64 C + OpenMP, "
                      f"{reps} repetitions in {el:.1f} s"}


def row_flops(batch, hq: int, d: int, rows) -> float:
    """Causal FLOPs of the given global query rows: 4 d Hq (p + 1) each."""
    import numpy as np
    pos = np.empty(batch.num_q_tokens, dtype=np.int64)
    for r, req in enumerate(batch.requests):
        a = int(batch.qo_indptr[r])
        pos[a:a + req.qo_len] = np.arange(req.kv_len - req.qo_len, req.kv_len)
    return 4.0 * d * hq * float((pos[np.asarray(rows, dtype=np.int64)] + 1).sum())


def cpu_baseline_configs(budget_s: float) -> dict:
    """The oracle on every other configuration: seeded row samples of each (every stride-th
    query row, stride chosen for about budget_s seconds in all), timed and extrapolated to the
    whole batch by causal FLOPs (the oracle's cost is linear in them)."""
    import numpy as np

    import oracle
    import workloads as wl
    oracle.build(force=False)
    cases = [
        ("single_extend_67 (full prefill)", wl.single_extend, "full"),
        ("cold_prefill_16x1028", wl.cold_prefill, "full"),
        ("mixed_3700_plus_7_tails", wl.mixed_batch, "mixed"),
        ("long_fp8 prefill_8192", wl.long_fp8, "prefill_8192"),
        ("long_fp8 prefill_32768", wl.long_fp8, "prefill_32768"),
        ("long_fp8 extend_1024_behind_31744", wl.long_fp8, "extend"),
        ("decode_8x1_over_8k-128k", lambda: wl.decode_batch(full_prompts=0), "decode"),
    ]
    out = {}
    per_case = budget_s / len(cases)
    works = {}
    for name, build, which in cases:
        if build not in works:
            works[build] = build()
        work = works[build]
        b = work.batches[which]
        n = b.num_q_tokens
        total = causal_flops(b, work.num_qo_heads, work.head_dim)
        # probe one row to size the sample, then time the sample
        probe = np.array([n - 1])
        t0 = time.perf_counter()
        oracle.paged_prefill(**work.oracle_kwargs(b), rows=probe)
        t_probe = max(time.perf_counter() - t0, 1e-4)
        f_probe = row_flops(b, work.num_qo_heads, work.head_dim, probe)
        want = max(1, int(per_case / t_probe * f_probe / (total / n)))
        stride = max(1, n // want)
        rows = np.arange(stride // 2, n, stride, dtype=np.int64)
        t0 = time.perf_counter()
        oracle.paged_prefill(**work.oracle_kwargs(b), rows=rows)
        el = time.perf_counter() - t0
        f_rows = row_flops(b, work.num_qo_heads, work.head_dim, rows)
        full_s = el * total / f_rows
        out[name] = {"sample_rows": int(rows.size), "of_rows": n, "sample_s": round(el, 3),
                     "extrapolated_full_s": round(full_s, 3),
                     "tflops": round(total / full_s / 1e12, 5)}
    del works
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=8, help="rotated KV pools for the extend batch")
    ap.add_argument("--cpu-budget-s", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-others", action="store_true")
    ap.add_argument("--only", choices=["extend", "prefill", "decode", "copy", "stream", "mixed", "fp8_8k"], default=None,
                    help="run one leg only and print its timing (for profiler runs)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark measures one GPU: the attention path is built "
                                   "and measured on a single MI355X (it would shard by request, kv "
                                   "head or KV split without changing a bit); run with --gpus 1"}))
        return 2

    import numpy as np
    import torch

    import workloads as wl
    if not torch.cuda.is_available():
        log("no GPU visible")
        return 1

    if args.only == "copy":
        # calibration for the HBM byte counters: one device copy of exactly 512 MiB
        n = 512 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {n} bytes x3")
        return 0

    hq, hkv, d = 32, 8, 128
    result = {}

    # ---------------------------------------------------------------- extend (value)
    if args.only == "stream":  # profiler run: the streaming reference over the extend pages
        work = wl.extend_batch(layout="distinct")
        run = Runner(work, work.batches["cached"], replicas=args.replicas)
        ms = run.stream_timed(2, 4, args.steps, args.warmup)
        log(f"stream reference: {ms * 1e3:.2f} us/launch")
        return 0
    if args.only in (None, "extend"):
        log("building extend workload (distinct pages)")
        work = wl.extend_batch(layout="distinct")
        cached, full = work.batches["cached"], work.batches["full"]
        run = Runner(work, cached, replicas=args.replicas)
        if args.only == "extend":  # profiler run: only the timed launches
            ms, wall = run.timed(args.steps, args.warmup)
            log(f"extend: {ms * 1e3:.2f} us/step (wall {wall * 1e3:.2f} us)")
            return 0
        # timed before the host-side checks below, whose CPU thread pool would otherwise still
        # be spinning while the launches are issued
        ms, wall = run.timed(args.steps, args.warmup)
        # the metric's bit-exactness clause: cached rows vs the same rows of a full prefill
        o_c, l_c = run.outputs(0)
        fr = Runner(work, full, replicas=1)
        o_f, l_f = fr.outputs(0)
        max_diff = 0.0
        for r in range(cached.batch_size):
            ia, ib = wl.matching_rows(cached, r, full, r)
            max_diff = max(max_diff, float((o_c[ia].float() - o_f[ib].float()).abs().max()),
                           float((l_c[ia] - l_f[ib]).abs().max()))
        assert np.isfinite(o_c.float().numpy()).all()
        del fr
        log(f"cached-vs-full max|diff| = {max_diff}")
        ms_graph = run.graph_timed(40, 10)
        ceiling = run.stream_ceiling(args.steps, args.warmup, same_gather=True)
        replan = run.replan_us()
        nbytes = kv_bytes(cached, hkv, d, 2)
        io_bytes = (2 * cached.num_q_tokens * hq * d * 2 + cached.num_q_tokens * hq * 4
                    + cached.kv_indices.size * 4)
        alg = nbytes + io_bytes
        achieved = alg / (ms * 1e-3) / 1e9
        result["extend"] = dict(ms=ms, wall_ms=wall, graph_ms=ms_graph, kv_bytes=nbytes, alg_bytes=alg, gbps=nbytes / (ms * 1e-3) / 1e9,
                                achieved=achieved, plan_us=run.plan_us, upload_us=run.upload_us, ceiling=ceiling,
                                replan=replan,
                                max_diff=max_diff, work=work, batch=cached,
                                items=run.plan.info.num_prefill_items)
        # radix layout (prefix pages physically shared): logical bytes over a cache-served read
        work_r = wl.extend_batch(layout="radix")
        rr = Runner(work_r, work_r.batches["cached"], replicas=1)
        ms_r, _ = rr.timed(args.steps, args.warmup)
        result["extend"]["radix_logical_gbps"] = kv_bytes(work_r.batches["cached"], hkv, d, 2) / (ms_r * 1e-3) / 1e9
        result["extend"]["radix_ms"] = ms_r
        del rr, run
        # negative control: the same extend batch planned with a batch-dependent KV tile
        ra = Runner(work, cached, replicas=args.replicas, adaptive=True)
        o_a, l_a = ra.outputs(0)
        fa = Runner(work, full, replicas=1, adaptive=True)
        o_fa, l_fa = fa.outputs(0)
        da_o = da_l = 0.0
        for r in range(cached.batch_size):
            ia, ib = wl.matching_rows(cached, r, full, r)
            da_o = max(da_o, float((o_a[ia].float() - o_fa[ib].float()).abs().max()))
            da_l = max(da_l, float((l_a[ia] - l_fa[ib]).abs().max()))
        ms_a, _ = ra.timed(args.steps, args.warmup)
        result["extend"]["adaptive"] = dict(ms=ms_a, block_n=ra.plan.info.block_n,
                                            full_block_n=fa.plan.info.block_n, max_o=da_o, max_l=da_l)
        del ra, fa

    # ---------------------------------------------------------------- cold prefill
    if args.only in (None, "prefill") and not args.no_prefill:
        log("building cold prefill workload")
        work_p = wl.cold_prefill()
        bp = work_p.batches["full"]
        pr = Runner(work_p, bp, replicas=1)
        # A sustained matrix-core load takes ~100 launches (~25 ms) to reach its steady rate
        # on a fresh GPU (the memory-bound extend leg does not move); time after that.
        ms_p, wall_p = pr.timed(max(10, args.steps // 4), max(100, args.warmup))
        if args.only == "prefill":
            log(f"prefill: {ms_p * 1e3:.2f} us/step")
            return 0
        fl = causal_flops(bp, hq, d)
        result["prefill"] = dict(ms=ms_p, flops=fl, tflops=fl / (ms_p * 1e-3) / 1e12,
                                 plan_us=pr.plan_us, items=pr.plan.info.num_prefill_items)
        del pr

    # ---------------------------------------------------------------- long-KV decode
    # ---------------------------------------------------------------- profiler runs of two other legs
    if args.only in ("mixed", "fp8_8k"):  # only the timed launches of that leg
        if args.only == "mixed":
            w_o = wl.mixed_batch()
            b_o = w_o.batches["mixed"]
        else:
            w_o = wl.long_fp8()
            b_o = w_o.batches["prefill_8192"]
        r_o = Runner(w_o, b_o, replicas=1)
        ms_o, _ = r_o.timed(args.steps, args.warmup)
        fl_o = causal_flops(b_o, w_o.num_qo_heads, w_o.head_dim)
        log(f"{args.only}: {ms_o * 1e3:.2f} us/step, {fl_o / (ms_o * 1e-3) / 1e12:.1f} TFLOP/s causal")
        return 0

    if args.only in (None, "decode") and not args.no_decode:
        log("building long-KV decode workload")
        work_d = wl.decode_batch(full_prompts=0)
        bd = work_d.batches["decode"]
        dr = Runner(work_d, bd, replicas=1)
        ms_d, _ = dr.timed(max(10, args.steps // 4), max(5, args.warmup // 4))
        ceil_d = dr.stream_ceiling(max(10, args.steps // 4), 3) if args.only is None else None
        if args.only == "decode":
            log(f"decode: {ms_d * 1e3:.2f} us/step")
            return 0
        nb = kv_bytes(bd, hkv, d, 2)
        result["decode"] = dict(ms=ms_d, kv_bytes=nb, gbps=nb / (ms_d * 1e-3) / 1e9,
                                items=dr.plan.info.num_prefill_items,
                                merges=dr.plan.info.num_merge_items, ceiling=ceil_d,
                                workspace=dr.plan.info.workspace_bytes)
        del dr

    # ---------------------------------------------------------------- remaining configurations
    others = {}
    if args.only is None and not args.no_others:
        def bits_equal(a_batch, oa, la, b_batch, ob, lb, pairs):
            worst = 0.0
            for ra, rb in pairs:
                ia, ib = wl.matching_rows(a_batch, ra, b_batch, rb)
                worst = max(worst, float((oa[ia].float() - ob[ib].float()).abs().max()),
                            float((la[ia] - lb[ib]).abs().max()))
            return worst

        def timed_leg(work, batch, steps, warmup):
            rr = Runner(work, batch, replicas=1)
            o, l = rr.outputs(0)
            # matrix-heavy launches reach their steady clock after ~25 ms of work: warm up for
            # at least 30 ms (one step timed first to size it)
            one, _ = rr.timed(1, 0)
            ms, _ = rr.timed(steps, max(warmup, int(30.0 / max(one, 1e-3)) + 1))
            info = rr.plan.info
            del rr
            return ms, o, l, info

        log("single 67-token prompt")
        w1 = wl.single_extend()
        ms_f, o_f, l_f, _ = timed_leg(w1, w1.batches["full"], 50, 10)
        ms_c, o_c, l_c, _ = timed_leg(w1, w1.batches["cached"], 50, 10)
        others["single_extend_67"] = {
            "workload": "one 67-token prompt, 32/8/128 bf16, page 16: full prefill vs 3-token extend behind 64 cached tokens",
            "full_prefill_us": round(ms_f * 1e3, 2), "extend_us": round(ms_c * 1e3, 2),
            "cached_vs_full_max_abs_diff": bits_equal(w1.batches["cached"], o_c, l_c, w1.batches["full"], o_f, l_f, [(0, 0)])}
        log("mixed batch")
        w4 = wl.mixed_batch()
        mb, fb = w4.batches["mixed"], w4.batches["full"]
        ms_m, o_m, l_m, info_m = timed_leg(w4, mb, 20, 20)
        _, o_mf, l_mf, _ = timed_leg(w4, fb, 1, 1)
        fl_m = causal_flops(mb, hq, d)
        others["mixed_3700_plus_7_tails"] = {
            "workload": "one 3,700-token prefill + 7 requests with 3,700 cached tokens and tails 1/2/4/6/37/64/300, 32/8/128 bf16, page 16",
            "us_per_step": round(ms_m * 1e3, 2), "causal_flops": fl_m,
            "tflops": round(fl_m / (ms_m * 1e-3) / 1e12, 2),
            "cached_vs_full_max_abs_diff": bits_equal(mb, o_m, l_m, fb, o_mf, l_mf, [(i + 1, i) for i in range(7)])}
        log("long fp8 path")
        w5 = wl.long_fp8()
        legs = {}
        outs = {}
        for name in ("prefill_8192", "prefill_32768", "extend"):
            b5 = w5.batches[name]
            ms5, o5, l5, info5 = timed_leg(w5, b5, 5 if name == "prefill_32768" else 10, 3)
            fl5 = causal_flops(b5, w5.num_qo_heads, w5.head_dim)
            legs[name] = {"us_per_step": round(ms5 * 1e3, 2), "causal_flops": fl5,
                          "tflops": round(fl5 / (ms5 * 1e-3) / 1e12, 2),
                          "workspace_bytes": info5.workspace_bytes, "passes": info5.num_passes}
            outs[name] = (o5, l5)
        legs["extend_vs_32k_prefill_max_abs_diff"] = bits_equal(
            w5.batches["extend"], *outs["extend"], w5.batches["prefill_32768"], *outs["prefill_32768"], [(0, 0)])
        others["long_fp8_24x4x256"] = dict(
            workload="24 q / 4 kv heads, head_dim 256, fp8 E4M3 KV (N(0,1) x 32, scale 1/32), page 16: "
                     "prefills of 8,192 and 32,768 tokens, a 1,024-token extend behind 31,744 cached tokens",
            **legs)
        del outs
        log("head_dim 512")
        w6 = wl.random_workload(512, hq=16, hkv=4, d=512, page_size=16, kv_dtype="bf16", specs=[(2048, 4)] * 4)
        b6e, b6f = w6.batches["batch"], w6.batches["full"]
        ms6f, o6f, l6f, _ = timed_leg(w6, b6f, 10, 5)
        ms6e, o6e, l6e, _ = timed_leg(w6, b6e, 50, 10)
        fl6 = causal_flops(b6f, 16, 512)
        others["head_dim_512"] = {
            "workload": "16 q / 4 kv heads, head_dim 512, bf16, page 16: cold prefill of 4 x 2,048 tokens, "
                        "and 4-token extends of the same prompts behind 2,044 cached tokens",
            "prefill_us": round(ms6f * 1e3, 2), "prefill_causal_flops": fl6,
            "prefill_tflops": round(fl6 / (ms6f * 1e-3) / 1e12, 2), "extend_us": round(ms6e * 1e3, 2),
            "cached_vs_full_max_abs_diff": bits_equal(b6e, o6e, l6e, b6f, o6f, l6f, [(i, i) for i in range(4)])}
        log("page sizes")
        pages = {}
        for page in (1, 2, 12, 16):
            w7 = wl.cold_prefill(page_size=page)
            b7 = w7.batches["full"]
            ms7, _, _, _ = timed_leg(w7, b7, 20, 20)
            pages[str(page)] = round(causal_flops(b7, hq, d) / (ms7 * 1e-3) / 1e12, 2)
            del w7
        others["page_sizes"] = {
            "workload": "the cold 16 x 1,028 prefill (32/8/128 bf16) with its KV in pages of 1, 2, 12 and 16 tokens "
                        "(page ids shuffled): causal TFLOP/s per page size",
            "tflops": pages}

    ext = result["extend"]
    traffic = traffic_from_profile(ext["alg_bytes"])
    line = {
        "metric": "prefill attn TFLOP/s + extend KV GB/s (1 GPU); cached-vs-full max|diff|=0",
        "value": round(ext["gbps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ext["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "extend batch: 16 requests x 1-4 new tokens (uniform) behind a "
                               "1024-token prefix, 32 q / 8 kv heads, head_dim 128, bf16, page 16, "
                               f"distinct prefix pages, {args.replicas} rotated pools",
                   "kv_bytes_per_step": ext["kv_bytes"],
                   "query_tokens": int(ext["batch"].num_q_tokens),
                   "parallelism": "single GPU"},
        "cached_vs_full_max_abs_diff": ext["max_diff"],
        "roofline": {"bound": "hbm", "achieved": round(ext["achieved"], 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(ext["achieved"] / HBM_PEAK_GBPS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "measured_ceiling": {
                         "what": "read-only streaming reference (dpp_stream_kv): the same KV pages, "
                                 "rotated pools and work list, gathered into LDS and dropped, no compute",
                         "us_per_launch": round(ext["ceiling"]["ms"] * 1e3, 2),
                         "kv_gbps": round(ext["kv_bytes"] / (ext["ceiling"]["ms"] * 1e-3) / 1e9, 1),
                         "workgroups_per_unit": ext["ceiling"]["split"],
                         "loads_in_flight_per_wave": ext["ceiling"]["depth"],
                         "frac": round(ext["ceiling"]["ms"] / ext["ms"], 4),
                         "same_gather": {
                             "what": "the same reference reading what the attention launch reads: two "
                                     "workgroups per unit, each all of K and one head_dim half of V",
                             "us_per_launch": round(ext["ceiling"]["same_gather_ms"] * 1e3, 2),
                             "loads_in_flight_per_wave": ext["ceiling"]["same_gather_depth"],
                             "frac": round(ext["ceiling"]["same_gather_ms"] / ext["ms"], 4)}}},
        "extend_detail": {"us_per_step": round(ext["ms"] * 1e3, 2),
                          "host_wall_us_per_step": round(ext["wall_ms"] * 1e3, 2),
                          "graph_replay_us_per_step": round(ext["graph_ms"] * 1e3, 2),
                          "algorithmic_bytes_per_launch": ext["alg_bytes"],
                          "work_items": ext["items"], "plan_us": round(ext["plan_us"], 1),
                          "upload_us": round(ext["upload_us"], 1),
                          "next_batch_plan_us": round(ext["replan"][0], 1),
                          "next_batch_upload_us": round(ext["replan"][1], 1),
                          "radix_layout_logical_gbps": round(ext["radix_logical_gbps"], 1),
                          "radix_layout_us_per_step": round(ext["radix_ms"] * 1e3, 2)},
        "adaptive_tile_control": {
            "what": "the same extend batch planned with a KV tile picked from the batch (FlashInfer's "
                    "average-packed-length rule; NOT batch invariant), against its full prefills",
            "block_n": ext["adaptive"]["block_n"], "full_prefill_block_n": ext["adaptive"]["full_block_n"],
            "us_per_step": round(ext["adaptive"]["ms"] * 1e3, 2),
            "cached_vs_full_max_abs_diff_o": ext["adaptive"]["max_o"],
            "cached_vs_full_max_abs_diff_lse": ext["adaptive"]["max_l"],
            "invariance_cost": round(ext["ms"] / ext["adaptive"]["ms"] - 1.0, 4)},
        "kernel_source_sha256_16": kernel_hash(),
    }
    if "prefill" in result:
        p = result["prefill"]
        line["prefill"] = {"workload": "cold causal prefill, 16 x 1028 tokens, 32/8/128 bf16, page 16",
                           "tflops": round(p["tflops"], 2), "ms_per_step": round(p["ms"], 5),
                           "causal_flops": p["flops"], "work_items": p["items"],
                           "roofline": {"bound": "mfma", "achieved": round(p["tflops"], 2),
                                        "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                        "frac": round(p["tflops"] / BF16_MFMA_PEAK_TFLOPS, 4)}}
    if "decode" in result:
        dd = result["decode"]
        line["decode"] = {"workload": "long-KV decode, 8 requests x 1 token over " +
                                      "/".join(str(n) for n in wl.DECODE_KV_LENS) +
                                      " keys, 32/8/128 bf16, page 16",
                          "kv_gbps": round(dd["gbps"], 2), "us_per_step": round(dd["ms"] * 1e3, 2),
                          "kv_bytes_per_step": dd["kv_bytes"], "work_items": dd["items"],
                          "merge_items": dd["merges"], "workspace_bytes": dd["workspace"],
                          "roofline": {"bound": "hbm", "achieved": round(dd["gbps"], 2),
                                       "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                       "frac": round(dd["gbps"] / HBM_PEAK_GBPS, 4),
                                       "measured_ceiling": None if dd["ceiling"] is None else {
                                           "us_per_launch": round(dd["ceiling"]["ms"] * 1e3, 2),
                                           "kv_gbps": round(dd["kv_bytes"] / (dd["ceiling"]["ms"] * 1e-3) / 1e9, 1),
                                           "frac": round(dd["ceiling"]["ms"] / dd["ms"], 4)}}}
    if others:
        line["other_configs"] = others
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(ext["work"], ext["batch"], args.cpu_budget_s)
        log("timing the CPU oracle on the other configurations (row samples)")
        line["cpu_baseline"]["other_configs"] = cpu_baseline_configs(args.cpu_budget_s)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
