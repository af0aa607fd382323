"""Benchmark: one step = one attn_varlen_paged_fwd call (append + planning +
attention + split merge) over a seeded synthetic batch on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--rope]

Default (no --workload): the four full-size workloads in one run, one JSON
line.  The headline (`value`, `roofline`, `cpu_baseline`) is varlen prefill
without a cache (16 sequences, lengths U[256, 2048], 32 query / 8 kv heads,
head_dim 128, bf16, causal): prefill TFLOP/s.  The line also carries
`decode` (paged decode, KV GB/s against HBM), `chunked_prefill` (TFLOP/s) and
`mixed_fp8` (the mixed prefill + decode batch over an fp8 cache: the step,
the prefill rows alone, the decode rows alone, the fused / serial ratio, the
combined roofline fraction, and the same batch through the fp8 QKV-Prob call
against the fp8 MFMA peak), each with its own roofline and CPU baseline.
With --workload NAME only that workload is measured and it is the headline
(names: varlen_prefill, paged_decode, chunked_prefill, mixed_fp8, tiny).

Per workload: W warm-up steps, then untimed steps for --settle seconds (the
GPU's clocks ramp up from idle over hundreds of milliseconds), then an
instrumented pass (the library brackets
every kernel launch with HIP events on its launch stream: per-kernel
durations), then the timed pass of exactly K steps between two
synchronisations (no per-launch events) that gives `value` and `ms_per_step`.
Inputs rotate over several device copies so that the 256 MB MALL cannot
serve a previous step's K/V.

Algorithmic work: prefill FLOPs = 4 * D per visible (query, key) pair per
query head; decode bytes = Lk * Hkv * D * 2 * bytes per cached element per
sequence.  With --rope each step is attn_varlen_paged_rope_fwd (rotary
embedding of q and k_new, rotary_dim = head_dim, half-split pairing) and the
line carries the time of the rotation kernel that turns the rows copied
before attention (the other rows are turned inside the attention kernels and
the fp8 append).
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

METRIC = "prefill attn TFLOP/s + decode KV GB/s (% of MI355X peak), varlen paged"
PEAK_BF16_TFLOPS = 2500.0     # dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # dense fp8 MFMA
PEAK_HBM_GBS = 8000.0         # HBM3E
KERNEL_SOURCES = ["varlen_paged_kv_amd/csrc/kernels/attn_fwd.hip", "varlen_paged_kv_amd/csrc/kernels/append_dev.h",
                  "varlen_paged_kv_amd/csrc/vpk_internal.h"]
SUITE = ["varlen_prefill", "paged_decode", "chunked_prefill", "mixed_fp8"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def visible_pairs(ql, kl, causal):
    """Number of (query, key) pairs that are not masked, per sequence."""
    out = np.zeros(len(ql), np.float64)
    for b, (lq, lk) in enumerate(zip(ql, kl)):
        lq, lk = int(lq), int(lk)
        if not causal:
            out[b] = lq * lk
            continue
        i = np.arange(lq)
        out[b] = np.clip(i + lk - lq + 1, 0, lk).sum()
    return out


def work_of(wl):
    pairs = visible_pairs(wl.q_lens(), wl.kv_lens(), wl.causal)
    flops = pairs * wl.Hq * 4.0 * wl.D
    ebytes = 1 if wl.cache_dtype == "fp8" else 2
    kv_bytes = wl.kv_lens().astype(np.float64) * wl.Hkv * wl.D * 2 * ebytes
    return flops, kv_bytes


def decode_rows(wl):
    """Sequences served by the decode-mode grid (q_len * g <= 32 packed rows)."""
    return wl.q_lens() * (wl.Hq // wl.Hkv) <= 32


def kernel_sha(sources=None):
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(name, sources=None):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the kernel is unchanged."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha256") != kernel_sha(sources):
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(wl, budget_s):
    """Time the oracle (as it stands) on a bounded sample of the same workload."""
    import oracle
    from threadpoolctl import threadpool_info

    threads = 0
    for info in threadpool_info():
        if info.get("user_api") == "blas":
            threads = max(threads, int(info.get("num_threads", 0)))
    threads = threads or (os.cpu_count() or 1)
    flops, kv_bytes = work_of(wl)
    by_bytes = wl.name == "paged_decode"
    # append first (part of the call), then attention sequence by sequence
    t0 = time.perf_counter()
    if wl.k_cache is not None and wl.k_new is not None:
        kc, vc = oracle.append(wl.k_new, wl.v_new, wl.cu_seqlens_knew, wl.k_cache, wl.v_cache,
                               wl.block_table, wl.cache_seqlens, wl.page_size, wl.cache_dtype,
                               wl.kv_scale)
    else:
        kc, vc = wl.k_cache, wl.v_cache
    t_append = time.perf_counter() - t0
    done, work, elapsed = [], 0.0, 0.0
    order = np.argsort(-(kv_bytes if by_bytes else flops + kv_bytes))[::-1]   # smallest first
    passes = 0
    while elapsed < budget_s and passes < 8:   # the whole batch again while under budget
        passes += 1
        for b in order:
            b = int(b)
            s, e = int(wl.cu_seqlens_q[b]), int(wl.cu_seqlens_q[b + 1])
            t0 = time.perf_counter()
            K, V = oracle.sequence_kv(b, k_new=wl.k_new, v_new=wl.v_new, cu_seqlens_knew=wl.cu_seqlens_knew,
                                      k_cache=kc, v_cache=vc, block_table=wl.block_table,
                                      cache_seqlens=wl.cache_seqlens, page_size=wl.page_size,
                                      cache_dtype=wl.cache_dtype, kv_scale=wl.kv_scale)
            if e > s:
                oracle.attend(oracle.bf16_bits_to_f64(wl.q[s:e]), K, V, wl.causal, wl.scale)
            elapsed += time.perf_counter() - t0
            done.append(b)
            work += float(kv_bytes[b] if by_bytes else flops[b])
            if elapsed >= budget_s:
                break
    # the append over the whole batch is charged pro rata to the sample
    frac = len(done) / wl.B
    elapsed += t_append * frac
    if by_bytes:
        value, unit = work / elapsed / 1e9, "GB/s"
    else:
        value, unit = work / elapsed / 1e12, "TFLOP/s"
    return {"value": value, "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{len(done)} sequence passes over the {wl.B} sequences of the {wl.name} batch "
                      f"(smallest first, {passes} pass(es) of the batch at most), all {wl.Hq} query heads, "
                      f"numpy float64, plus the batch's append pro rata; {elapsed:.1f} s"}


class GpuSampler:
    """Clock and power of the GPU sampled every 5 ms on a host thread while the timed pass
    runs (torch.cuda.clock_rate / power_draw, which query amd-smi); best effort: None
    where the query is not available."""

    def __init__(self, torch):
        self.torch, self.samples, self.stop = torch, [], False

    def _run(self):
        while not self.stop:
            try:
                self.samples.append((self.torch.cuda.clock_rate(), self.torch.cuda.power_draw()))
            except Exception:
                return
            time.sleep(0.005)

    def __enter__(self):
        import threading
        self.t = threading.Thread(target=self._run, daemon=True)
        self.t.start()
        return self

    def __exit__(self, *exc):
        self.stop = True
        self.t.join()

    def summary(self):
        if not self.samples:
            return None
        clk = sorted(c for c, _ in self.samples)
        pw = sorted(p for _, p in self.samples)
        return {"samples": len(self.samples), "sclk_mhz_median": clk[len(clk) // 2], "sclk_mhz_min": clk[0],
                "power_median": pw[len(pw) // 2], "power_max": pw[-1],
                "note": "torch.cuda.clock_rate (MHz) and torch.cuda.power_draw (as the driver reports it)"}


class Runner:
    """Device copies of one workload's inputs and the timing passes over them."""

    def __init__(self, wl, dev, rotate, rope=False, mode="direct", qp_scale=None):
        import torch
        import varlen_paged_kv_amd as vpk
        self.torch, self.vpk, self.wl = torch, vpk, wl
        self.fp8 = wl.cache_dtype == "fp8"
        self.mode = mode
        # (q_scale, p_scale): each step is the fp8 QKV-Prob call (direct calls only)
        self.qp_scale = qp_scale

        def bf16(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

        def i32(a):
            return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)

        self.copies = []
        for _ in range(max(1, rotate)):
            c = dict(q=bf16(wl.q), cu_q=i32(wl.cu_seqlens_q))
            c["k_new"] = bf16(wl.k_new) if wl.k_new is not None else None
            c["v_new"] = bf16(wl.v_new) if wl.v_new is not None else None
            c["cu_kn"] = i32(wl.cu_seqlens_knew) if wl.cu_seqlens_knew is not None else None
            if wl.k_cache is not None:
                mk = (lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)) if self.fp8 else bf16
                c["kc"], c["vc"] = mk(wl.k_cache), mk(wl.v_cache)
                c["bt"], c["cl"] = i32(wl.block_table), i32(wl.cache_seqlens)
            else:
                c["kc"] = c["vc"] = c["bt"] = c["cl"] = None
            c["out"] = torch.empty_like(c["q"])
            c["lse"] = torch.empty((wl.Hq, wl.Tq), dtype=torch.float32, device=dev)
            self.copies.append(c)
        self.host = dict(cu_seqlens_q=wl.cu_seqlens_q, cu_seqlens_knew=wl.cu_seqlens_knew,
                         cache_seqlens=wl.cache_seqlens, block_table=wl.block_table)
        self.plan = None
        self.graphs = []
        if mode in ("prepared", "graph"):
            # one plan for the lengths (all copies share them); a graph of one run per copy
            has_cache = wl.k_cache is not None
            self.plan = vpk.Plan(wl.cu_seqlens_q, wl.Hq, wl.Hkv, wl.D, cu_seqlens_knew=wl.cu_seqlens_knew,
                                 cache_seqlens=wl.cache_seqlens if has_cache else None,
                                 block_table=wl.block_table if has_cache else None,
                                 page_size=wl.page_size if has_cache else 0, num_pages=wl.num_pages,
                                 max_pages_per_seq=wl.block_table.shape[1] if has_cache else 0,
                                 cache_dtype=wl.cache_dtype or "bf16", causal=wl.causal)
        if mode == "graph":
            import gc
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                for i in range(len(self.copies)):
                    self._plan_run(i)
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            gc.collect()
            for i in range(len(self.copies)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    self._plan_run(i)
                self.graphs.append(g)
            torch.cuda.synchronize()
        self.rope_kw = None
        if rope:
            from synth import rope_tables
            cos, sin = rope_tables(int(wl.kv_lens().max()), wl.D)
            self.rope_kw = dict(rope_cos=torch.from_numpy(cos).to(dev), rope_sin=torch.from_numpy(sin).to(dev),
                                rotary_dim=wl.D, interleaved=False)

    def _plan_run(self, i):
        wl, c = self.wl, self.copies[i % len(self.copies)]
        self.plan.run(c["q"], c["k_new"], c["v_new"], c["kc"], c["vc"], c["bt"], scale=wl.scale,
                      kv_scale=wl.kv_scale if self.fp8 else None, out=c["out"], lse=c["lse"])

    def step(self, i):
        if self.mode == "graph":
            self.graphs[i % len(self.graphs)].replay()
            return
        if self.mode == "prepared":
            self._plan_run(i)
            return
        wl, c = self.wl, self.copies[i % len(self.copies)]
        args = (c["q"], c["cu_q"], c["k_new"], c["v_new"], c["cu_kn"], c["kc"], c["vc"], c["bt"], c["cl"],
                wl.page_size, wl.causal, wl.scale, wl.kv_scale if self.fp8 else None)
        if self.qp_scale is not None:
            self.vpk.attn_varlen_paged_qkv_prob_fwd(*args, q_scale=self.qp_scale[0], p_scale=self.qp_scale[1],
                                                    out=c["out"], lse=c["lse"], host_index=self.host,
                                                    **(self.rope_kw or {}))
        elif self.rope_kw is None:
            self.vpk.attn_varlen_paged_fwd(*args, out=c["out"], lse=c["lse"], host_index=self.host)
        else:
            self.vpk.attn_varlen_paged_rope_fwd(*args, **self.rope_kw, out=c["out"], lse=c["lse"],
                                                host_index=self.host)

    def timed(self, steps, instrumented):
        """`steps` steps between two synchronisations; with `instrumented`, the library also
        brackets every kernel launch with HIP events on its launch stream."""
        torch, vpk = self.torch, self.vpk
        vpk.timing_reset()
        vpk.timing_enable(instrumented)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        for i in range(steps):
            self.step(i)
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        vpk.timing_enable(False)
        return start.elapsed_time(end), wall

    def measure(self, steps, warmup, settle_s):
        """Warm-up, clock settling, instrumented pass (per-kernel averages, us), timed pass (ms per step)."""
        vpk = self.vpk
        for i in range(warmup):
            self.step(i)
        self.torch.cuda.synchronize()
        # keep the GPU busy until its clocks have settled (an idle GPU ramps up over
        # hundreds of milliseconds; a short warm-up alone would time the ramp)
        t0, n = time.perf_counter(), 0
        while time.perf_counter() - t0 < settle_s:
            for _ in range(8):
                self.step(n)
                n += 1
            self.torch.cuda.synchronize()
        self.settle_steps = n
        inst_ms, _ = self.timed(steps, True)
        kern = {}
        for key, kid in (("prefill_grid", vpk.KERNEL_ATTENTION), ("decode_grid", vpk.KERNEL_ATTENTION_DECODE),
                         ("mixed_grid", vpk.KERNEL_ATTENTION_MIXED), ("append", vpk.KERNEL_APPEND),
                         ("merge", vpk.KERNEL_MERGE), ("rope", vpk.KERNEL_ROPE),
                         ("prob8_grid", vpk.KERNEL_ATTENTION_PROB8)):
            ms, n = vpk.timing_read(kid)
            kern[key] = (ms * 1e3 / n if n else 0.0, n)
        with GpuSampler(self.torch) as gs:
            gpu_ms, wall = self.timed(steps, False)
        return dict(ms_per_step=gpu_ms / steps, host_us_per_step=wall * 1e6 / steps,
                    inst_us_per_step=inst_ms * 1e3 / steps, kernels=kern, settle_steps=self.settle_steps,
                    gpu=gs.summary())


def kernel_note(m, steps):
    return ("HIP events recorded by the library around each launch on its launch stream, over an "
            f"instrumented pass of {steps} steps before the timed pass "
            f"({m['inst_us_per_step']:.1f} us/step with the events)")


def summary(name, m):
    k = m["kernels"]
    parts = ", ".join(f"{key} {us:.1f} us x{n}" for key, (us, n) in k.items() if n)
    return (f"{name}: {m['ms_per_step'] * 1e3:.1f} us/step after {m['settle_steps']} settling steps "
            f"(host {m['host_us_per_step']:.1f} us/step; "
            f"instrumented pass {m['inst_us_per_step']:.1f} us/step); {parts}")


def mfma_roof(flops, us, traffic, note):
    ach = flops / (us / 1e6) / 1e12 if us > 0 else 0.0
    return {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": ach / PEAK_BF16_TFLOPS, "traffic": traffic, "kernel": "attention (prefill-mode grid)",
            "kernel_avg_us": us, "kernel_timing": note}


def hbm_roof(nbytes, us, traffic, note, kernel="attention (decode-mode grid)"):
    ach = nbytes / (us / 1e6) / 1e9 if us > 0 else 0.0
    return {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": ach / PEAK_HBM_GBS, "traffic": traffic, "kernel": kernel,
            "kernel_avg_us": us, "kernel_timing": note}


def config_of(wl, flops, kv_bytes, rope):
    return {"workload": wl.name, "batch": wl.B, "total_q": wl.Tq, "total_new": wl.Tn, "q_heads": wl.Hq,
            "kv_heads": wl.Hkv, "head_dim": wl.D, "page_size": wl.page_size, "causal": wl.causal,
            "kv_cache": wl.cache_dtype or "none", "pages": wl.num_pages, "flops_per_step": flops,
            "kv_bytes_per_step": kv_bytes, "parallelism": "single GPU",
            **({"rope": "rotary_dim=head_dim, half-split"} if rope else {})}


def measure_workload(name, args, dev, cpu_budget):
    """One workload's object: throughput of the whole step, roofline of its dominant kernel,
    CPU baseline; the mixed batch also times its prefill and decode rows alone."""
    from synth import make_workload, subset
    t0 = time.perf_counter()
    wl = make_workload(name)
    flops, kv_bytes = work_of(wl)
    step_flops, step_bytes = float(flops.sum()), float(kv_bytes.sum())
    dec = decode_rows(wl)
    pre_flops, dec_bytes = float(flops[~dec].sum()), float(kv_bytes[dec].sum())
    log(f"{name}: Tq={wl.Tq} Tn={wl.Tn} pages={wl.num_pages} flops/step={step_flops:.3e} "
        f"kv bytes/step={step_bytes:.3e} (inputs drawn in {time.perf_counter() - t0:.1f} s)")
    r = Runner(wl, dev, args.rotate, rope=args.rope, mode=args.mode)
    m = r.measure(args.steps, args.warmup, args.settle)
    log(summary(name, m))
    k = m["kernels"]
    note = kernel_note(m, args.steps)
    elapsed = m["ms_per_step"] / 1e3
    obj = {"workload": name, "ms_per_step": m["ms_per_step"], "config": config_of(wl, step_flops, step_bytes,
                                                                                      args.rope),
           "gpu_during_timed_pass": m.get("gpu")}
    if name == "paged_decode":
        obj.update(value=step_bytes / elapsed / 1e9, unit="GB/s")
        obj["pct_of_peak"] = 100.0 * obj["value"] / PEAK_HBM_GBS
        obj["roofline"] = hbm_roof(dec_bytes, k["decode_grid"][0], load_traffic(name), note)
        obj["roofline"]["merge_avg_us"] = k["merge"][0]
        # the same kernel against a read bandwidth measured on this GPU in this run
        ceil = read_ceiling(dev)
        if ceil:
            obj["read_ceiling"] = dict(ceil, kernel_frac=obj["roofline"]["achieved"] / ceil["value"])
    elif name == "mixed_fp8":
        obj.update(value=step_flops / elapsed / 1e12, unit="TFLOP/s")
        obj["pct_of_peak"] = 100.0 * obj["value"] / PEAK_BF16_TFLOPS
        if k["mixed_grid"][1]:
            # one launch for both kinds of items: its prefill FLOPs and decode bytes over its time
            mus = k["mixed_grid"][0]
            roof = mfma_roof(pre_flops, mus, load_traffic(name), note)
            roof["kernel"] = "attention (mixed grid: prefill-mode tiles and decode-mode splits in one launch)"
            roof["decode_part"] = hbm_roof(dec_bytes, mus, None, note, kernel="the same launch's decode-mode items")
            roof["combined_frac_kernel"] = (pre_flops / (PEAK_BF16_TFLOPS * 1e12) +
                                            dec_bytes / (PEAK_HBM_GBS * 1e9)) / (mus / 1e6)
        else:
            roof = mfma_roof(pre_flops, k["prefill_grid"][0], load_traffic(name), note)
            roof["decode_grid"] = hbm_roof(dec_bytes, k["decode_grid"][0], None, note)
        # the whole step against both roofs at once: prefill FLOPs at the bf16 peak plus
        # decode KV bytes at the HBM peak, over the step time
        roof["combined_frac"] = (pre_flops / (PEAK_BF16_TFLOPS * 1e12) + dec_bytes / (PEAK_HBM_GBS * 1e9)) / elapsed
        obj["roofline"] = roof
        del r
        if not args.no_qkv_prob:
            obj["qkv_prob"] = measure_qkv_prob(wl, args, dev, pre_flops, dec_bytes, step_flops)
        if args.no_parts:
            obj["cpu_baseline"] = cpu_baseline(wl, cpu_budget) if cpu_budget > 0 else None
            return obj
        parts = {}
        for label, seqs in (("prefill_rows", np.nonzero(~dec)[0]), ("decode_rows", np.nonzero(dec)[0])):
            sub = subset(wl, seqs)
            rs = Runner(sub, dev, args.rotate, mode=args.mode)
            ms = rs.measure(args.steps, args.warmup, args.settle)
            log(summary(f"{name} {label} alone", ms))
            parts[label] = ms["ms_per_step"]
            del rs
        obj["parts_alone_ms"] = parts
        obj["fused_over_serial"] = m["ms_per_step"] / (parts["prefill_rows"] + parts["decode_rows"])
    else:
        obj.update(value=step_flops / elapsed / 1e12, unit="TFLOP/s")
        obj["pct_of_peak"] = 100.0 * obj["value"] / PEAK_BF16_TFLOPS
        obj["roofline"] = mfma_roof(pre_flops, k["prefill_grid"][0], load_traffic(name), note)
    if args.rope:
        # the rotation kernel turns only the rows the other kernels do not turn as they
        # read them (decode-mode query rows, the new keys of a bf16 cache or of a call
        # without a cache); its time is reported, the rest is inside the grids above
        rus, rn = k["rope"]
        obj["rope_kernel"] = {"kernel": "rotary embedding of the rows copied before attention",
                              "rotary_dim": wl.D, "interleaved": False, "kernel_avg_us": rus, "launches": rn}
    obj["cpu_baseline"] = None
    if cpu_budget > 0:
        log(f"{name}: timing the CPU oracle on a bounded sample")
        obj["cpu_baseline"] = cpu_baseline(wl, cpu_budget)
    return obj


def measure_qkv_prob(wl, args, dev, pre_flops, dec_bytes, step_flops):
    """The same batch through the fp8 QKV-Prob call (query rows and P in e4m3 too, both products
    on the fp8 MFMA; q_scale = amax(q) / 448, p_scale = 1 / 448): step throughput and the roofline
    of its one attention grid against the fp8 MFMA peak."""
    q32 = (wl.q.astype(np.uint32) << 16).view(np.float32)
    qp = (float(np.float32(np.abs(q32).max() / 448.0)), 1.0 / 448.0)
    r = Runner(wl, dev, args.rotate, rope=args.rope, qp_scale=qp)
    m = r.measure(args.steps, args.warmup, args.settle)
    log(summary(f"{wl.name} QKV-Prob", m))
    del r
    us = m["kernels"]["prob8_grid"][0]
    elapsed = m["ms_per_step"] / 1e3
    ach = pre_flops / (us / 1e6) / 1e12 if us > 0 else 0.0
    roof = {"bound": "mfma", "achieved": ach, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
            "frac": ach / PEAK_FP8_TFLOPS, "traffic": load_traffic(f"{wl.name}_qkv_prob"),
            "kernel": "attention (fp8 QKV-Prob grid: every item of the batch in one launch)",
            "kernel_avg_us": us, "kernel_timing": kernel_note(m, args.steps),
            "note": "achieved counts the algorithmic 4 * D FLOPs per visible (query, key) pair of the "
                    "prefill rows; the kernel also computes every score twice (a first pass for the "
                    "row maximum and sum), 6 * D executed FLOPs per pair",
            "decode_part": {"bytes": dec_bytes, "gbs_over_kernel": dec_bytes / (us / 1e6) / 1e9 if us > 0 else 0.0},
            "combined_frac_kernel": (pre_flops / (PEAK_FP8_TFLOPS * 1e12) + dec_bytes / (PEAK_HBM_GBS * 1e9))
            / (us / 1e6) if us > 0 else 0.0}
    res = {"call": "attn_varlen_paged_qkv_prob_fwd", "dtype": "fp8 e4m3 (Q, K, V and P)",
           "q_scale": qp[0], "p_scale": qp[1], "ms_per_step": m["ms_per_step"],
           "value": step_flops / elapsed / 1e12, "unit": "TFLOP/s", "roofline": roof}
    if not args.no_parts:
        from synth import subset
        dec = decode_rows(wl)
        parts = {}
        for label, seqs in (("prefill_rows", np.nonzero(~dec)[0]), ("decode_rows", np.nonzero(dec)[0])):
            rs = Runner(subset(wl, seqs), dev, args.rotate, rope=args.rope, qp_scale=qp)
            ms = rs.measure(args.steps, args.warmup, args.settle)
            log(summary(f"{wl.name} QKV-Prob {label} alone", ms))
            parts[label] = {"ms_per_step": ms["ms_per_step"], "grid_us": ms["kernels"]["prob8_grid"][0]}
            del rs
        res["parts_alone"] = parts
        pus = parts["prefill_rows"]["grid_us"]
        if pus > 0:
            res["prefill_rows_grid_frac_fp8"] = pre_flops / (pus / 1e6) / 1e12 / PEAK_FP8_TFLOPS
    return res


def read_ceiling(dev, gib=4.0, reps=5):
    """A read bandwidth measured on this GPU in this run, for the decode figure: a streaming
    read of a contiguous `gib` GiB buffer (16 times the 256 MB MALL) by the helper library
    libvpk_measure.so, over several launch shapes, best of `reps` passes each; GB/s of bytes
    read.  None when the helper is not built."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "varlen_paged_kv_amd", "lib", "libvpk_measure.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.vpk_measure_stream_read.restype = ctypes.c_int
    lib.vpk_measure_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_void_p, ctypes.c_void_p]
    nbytes = int(gib * (1 << 30))
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    shapes = [(2048, 1), (4096, 4), (8192, 4), (16384, 8)]
    out = torch.empty(max(g for g, _ in shapes) * 256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    best, best_shape = 0.0, None
    for grid, unroll in shapes:
        for rep in range(reps + 1):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            rc = lib.vpk_measure_stream_read(buf.data_ptr(), nbytes, grid, unroll, out.data_ptr(), stream)
            b.record()
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"stream read launch failed ({rc})")
            gbs = nbytes / (a.elapsed_time(b) / 1e3) / 1e9
            if rep > 0 and gbs > best:
                best, best_shape = gbs, (grid, unroll)
    del buf, out
    torch.cuda.empty_cache()
    return {"value": best, "unit": "GB/s",
            "how": f"streaming read of a contiguous {gib:g} GiB buffer, 16-byte loads in a grid-stride "
                   f"loop; best launch shape {best_shape[0]} x 256 threads, {best_shape[1]} loads in flight "
                   f"per thread, best of {reps}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=None,
                    choices=["varlen_prefill", "paged_decode", "chunked_prefill", "mixed_fp8", "tiny"],
                    help="measure this workload alone (default: the four full-size workloads)")
    ap.add_argument("--rotate", type=int, default=3, help="input copies cycled through (defeats the MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parts", action="store_true", help="mixed batch: do not time its parts alone")
    ap.add_argument("--cpu-budget", type=float, default=6.0, help="seconds of oracle time per workload")
    ap.add_argument("--settle", type=float, default=1.0,
                    help="seconds of untimed steps after the warm-up, before the passes (clock ramp)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB device copy first (reference kernel for HBM counters)")
    ap.add_argument("--persistent", type=int, default=-1)
    ap.add_argument("--mode", default="direct", choices=["direct", "prepared", "graph"],
                    help="each step a direct call, a prepared-plan run (vpk_plan_run), or a graph replay of one")
    ap.add_argument("--plan-upload", type=int, default=0, help="library option plan_upload (0 or 1)")
    ap.add_argument("--mixed-grid", type=int, default=-2, help="library option mixed_grid (-1, 0 or 1; default: the library's)")
    ap.add_argument("--mixed-dec-parts", type=int, default=0, help="library option mixed_dec_parts (0: the library's)")
    ap.add_argument("--force-splits", type=int, default=0,
                    help="library option force_splits: every tile's key range in this many parts (0: the planner's)")
    ap.add_argument("--keep-scores", type=int, default=1,
                    help="library option keep_scores for the QKV-Prob call (0 or 1)")
    ap.add_argument("--rope", action="store_true", help="rotary embedding of q and k_new in every step")
    ap.add_argument("--no-qkv-prob", action="store_true",
                    help="mixed batch: do not also time it through the fp8 QKV-Prob call")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import varlen_paged_kv_amd as vpk

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    vpk.set_option("persistent", args.persistent)
    vpk.set_option("plan_upload", args.plan_upload)
    if args.mixed_grid >= -1:
        vpk.set_option("mixed_grid", args.mixed_grid)
    if args.mixed_dec_parts > 0:
        vpk.set_option("mixed_dec_parts", args.mixed_dec_parts)
    vpk.set_option("keep_scores", args.keep_scores)
    vpk.set_option("force_splits", args.force_splits)

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    names = [args.workload] if args.workload else SUITE
    budget = 0.0 if args.no_cpu_baseline else args.cpu_budget
    objs = {}
    for name in names:
        objs[name] = measure_workload(name, args, dev, budget)
        torch.cuda.empty_cache()
    head = objs[names[0]]
    line = {
        "metric": METRIC, "value": head["value"], "unit": head["unit"], "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) values, lengths and page tables drawn per the workload recipe)",
        "config": head["config"], "pct_of_peak": head["pct_of_peak"], "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
    }
    for key in ("rope_kernel", "qkv_prob", "parts_alone_ms", "fused_over_serial", "read_ceiling",
                "gpu_during_timed_pass"):
        if key in head:
            line[key] = head[key]
    for name in names[1:]:
        line["decode" if name == "paged_decode" else name] = objs[name]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
