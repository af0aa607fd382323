"""Benchmark: one step = one attn_varlen_paged_fwd call (append + plan upload +
attention + split merge) over a seeded synthetic batch on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--rope]

Default workload: varlen prefill without a cache (16 sequences, lengths
U[256, 2048], 32 query / 8 kv heads, head_dim 128, bf16, causal).  Other names:
paged_decode, chunked_prefill, mixed_fp8, tiny.

Prints ONE JSON line.  `value` is the algorithmic throughput of the whole step
(inputs resident in HBM): prefill TFLOP/s (4 * D flops per visible (query, key)
pair per query head) or, for pure decode, KV-cache GB/s (Lk * Hkv * D * 2 *
bytes per element per sequence).  `roofline` is the attention kernel alone,
timed with HIP events recorded by the library on the launch stream.
With --rope each step is attn_varlen_paged_rope_fwd (rotary embedding of q
and k_new first, rotary_dim = head_dim, half-split pairing) and the line also
carries the rotation kernel's own time and bandwidth.
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
PEAK_HBM_GBS = 8000.0         # HBM3E
KERNEL_SOURCES = ["varlen_paged_kv_amd/csrc/kernels/attn_fwd.hip", "varlen_paged_kv_amd/csrc/kernels/append_dev.h",
                  "varlen_paged_kv_amd/csrc/vpk_internal.h"]


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


ROPE_SOURCES = ["varlen_paged_kv_amd/csrc/kernels/rope.hip", "varlen_paged_kv_amd/csrc/vpk_internal.h"]


def kernel_sha(sources=None):
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(workload, sources=None):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the kernel is unchanged."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
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


def cpu_baseline(wl, budget_s=12.0):
    """Time the oracle (as it stands) on a bounded sample of the same workload."""
    import oracle
    from threadpoolctl import threadpool_info

    threads = 0
    for info in threadpool_info():
        if info.get("user_api") == "blas":
            threads = max(threads, int(info.get("num_threads", 0)))
    threads = threads or (os.cpu_count() or 1)
    flops, kv_bytes = work_of(wl)
    decode = wl.name == "paged_decode"
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
    order = np.argsort(-(flops if not decode else kv_bytes))[::-1]   # smallest first
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
            work += float(kv_bytes[b] if decode else flops[b])
            if elapsed >= budget_s:
                break
    # the append over the whole batch is charged pro rata to the sample
    frac = len(done) / wl.B
    elapsed += t_append * frac
    if decode:
        value, unit = work / elapsed / 1e9, "GB/s"
    else:
        value, unit = work / elapsed / 1e12, "TFLOP/s"
    return {"value": value, "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{len(done)} sequence passes over the {wl.B} sequences of the {wl.name} batch "
                      f"(smallest first, {passes} pass(es) of the batch at most), all {wl.Hq} query heads, "
                      f"numpy float64, plus the batch's append pro rata; {elapsed:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="varlen_prefill",
                    choices=["varlen_prefill", "paged_decode", "chunked_prefill", "mixed_fp8", "tiny"])
    ap.add_argument("--rotate", type=int, default=3, help="input copies cycled through (defeats the MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB device copy first (reference kernel for HBM counters)")
    ap.add_argument("--persistent", type=int, default=-1)
    ap.add_argument("--rope", action="store_true", help="rotary embedding of q and k_new in every step")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import varlen_paged_kv_amd as vpk
    from synth import make_workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    wl = make_workload(args.workload)
    flops, kv_bytes = work_of(wl)
    step_flops, step_bytes = float(flops.sum()), float(kv_bytes.sum())
    decode = args.workload == "paged_decode"

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)

    fp8 = wl.cache_dtype == "fp8"
    copies = []
    for _ in range(max(1, args.rotate)):
        c = dict(q=bf16(wl.q), cu_q=i32(wl.cu_seqlens_q))
        c["k_new"] = bf16(wl.k_new) if wl.k_new is not None else None
        c["v_new"] = bf16(wl.v_new) if wl.v_new is not None else None
        c["cu_kn"] = i32(wl.cu_seqlens_knew) if wl.cu_seqlens_knew is not None else None
        if wl.k_cache is not None:
            mk = (lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)) if fp8 else bf16
            c["kc"], c["vc"] = mk(wl.k_cache), mk(wl.v_cache)
            c["bt"], c["cl"] = i32(wl.block_table), i32(wl.cache_seqlens)
        else:
            c["kc"] = c["vc"] = c["bt"] = c["cl"] = None
        c["out"] = torch.empty_like(c["q"])
        c["lse"] = torch.empty((wl.Hq, wl.Tq), dtype=torch.float32, device=dev)
        copies.append(c)
    host = dict(cu_seqlens_q=wl.cu_seqlens_q, cu_seqlens_knew=wl.cu_seqlens_knew,
                cache_seqlens=wl.cache_seqlens, block_table=wl.block_table)
    vpk.set_option("persistent", args.persistent)
    rope_kw = None
    if args.rope:
        from synth import rope_tables
        cos, sin = rope_tables(int(wl.kv_lens().max()), wl.D)
        rope_kw = dict(rope_cos=torch.from_numpy(cos).to(dev), rope_sin=torch.from_numpy(sin).to(dev),
                       rotary_dim=wl.D, interleaved=False)

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(i):
        c = copies[i % len(copies)]
        args_ = (c["q"], c["cu_q"], c["k_new"], c["v_new"], c["cu_kn"], c["kc"], c["vc"], c["bt"], c["cl"],
                 wl.page_size, wl.causal, wl.scale, wl.kv_scale if fp8 else None)
        if rope_kw is None:
            vpk.attn_varlen_paged_fwd(*args_, out=c["out"], lse=c["lse"], host_index=host)
        else:
            vpk.attn_varlen_paged_rope_fwd(*args_, **rope_kw, out=c["out"], lse=c["lse"], host_index=host)

    print(f"[bench] {args.workload}: Tq={wl.Tq} Tn={wl.Tn} pages={wl.num_pages} "
          f"flops/step={step_flops:.3e} kv bytes/step={step_bytes:.3e}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    def timed(instrumented):
        """K steps between two synchronisations; with `instrumented`, the
        library also brackets every kernel launch with HIP events on its
        launch stream (per-kernel durations; the extra events cost a few us
        per launch, so the throughput figure comes from the plain pass)."""
        vpk.timing_reset()
        vpk.timing_enable(instrumented)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        for i in range(args.steps):
            step(i)
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        vpk.timing_enable(False)
        return start.elapsed_time(end), wall

    gpu_ms, wall = timed(False)                 # the timed region of the throughput figure
    inst_ms, _ = timed(True)                    # the same steps again, per-kernel events on
    pre_ms, pre_n = vpk.timing_read(vpk.KERNEL_ATTENTION)
    dec_ms, dec_n = vpk.timing_read(vpk.KERNEL_ATTENTION_DECODE)
    app_ms, app_n = vpk.timing_read(vpk.KERNEL_APPEND)
    mrg_ms, mrg_n = vpk.timing_read(vpk.KERNEL_MERGE)
    rot_ms, rot_n = vpk.timing_read(vpk.KERNEL_ROPE)
    elapsed = max(gpu_ms / 1e3, 1e-9)
    ms_per_step = gpu_ms / args.steps
    avg = lambda ms, n: ms / max(n, 1)
    print(f"[bench] timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step (host {wall * 1e6 / args.steps:.1f} us/step; "
          f"instrumented pass {inst_ms * 1e3 / args.steps:.1f} us/step); "
          f"attention prefill-mode {avg(pre_ms, pre_n) * 1e3:.1f} us x{pre_n}, decode-mode "
          f"{avg(dec_ms, dec_n) * 1e3:.1f} us x{dec_n}, standalone append {avg(app_ms, app_n) * 1e3:.1f} us x{app_n}, "
          f"merge {avg(mrg_ms, mrg_n) * 1e3:.1f} us x{mrg_n}, rotary {avg(rot_ms, rot_n) * 1e3:.1f} us x{rot_n}",
          file=sys.stderr, flush=True)

    # work of the sequences each grid serves (decode-mode: q_len * g <= 32 rows)
    dec_seq = wl.q_lens() * (wl.Hq // wl.Hkv) <= 32
    pre_flops = float(flops[~dec_seq].sum())
    dec_bytes = float(kv_bytes[dec_seq].sum())
    if decode:
        value, unit = step_bytes * args.steps / elapsed / 1e9, "GB/s"
        kus = avg(dec_ms, dec_n) * 1e3
        achieved = step_bytes / (kus / 1e6) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "kernel": "attention (decode-mode grid)"}
    else:
        value, unit = step_flops * args.steps / elapsed / 1e12, "TFLOP/s"
        kus = avg(pre_ms, pre_n) * 1e3
        achieved = pre_flops / (kus / 1e6) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "kernel": "attention (prefill-mode grid)"}
        if dec_n:
            dus = avg(dec_ms, dec_n) * 1e3
            roof["decode_grid"] = {"bound": "hbm", "achieved": dec_bytes / (dus / 1e6) / 1e9,
                                   "peak": PEAK_HBM_GBS, "unit": "GB/s", "kernel_avg_us": dus}
    roof["traffic"] = load_traffic(args.workload)
    roof["kernel_avg_us"] = kus
    roof["kernel_timing"] = ("HIP events recorded by the library around each launch on its launch stream, "
                             f"over a second pass of the same {args.steps} steps "
                             f"({inst_ms * 1e3 / args.steps:.1f} us/step with the events)")

    rope_line = None
    if args.rope:
        # algorithmic bytes: q and k_new read once and written once (bf16); the
        # angle tables (max_pos x D/2 x 8 bytes) are re-read through the caches
        rbytes = 2.0 * 2.0 * wl.D * (wl.Tq * wl.Hq + wl.Tn * wl.Hkv)
        rus = avg(rot_ms, rot_n) * 1e3
        rope_line = {"kernel": "rotary embedding of q and k_new", "rotary_dim": wl.D, "interleaved": False,
                     "kernel_avg_us": rus, "bytes": rbytes, "bound": "hbm",
                     "achieved": rbytes / max(rus, 1e-9) * 1e-3, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": rbytes / max(rus, 1e-9) * 1e-3 / PEAK_HBM_GBS,
                     "traffic": load_traffic("rope_" + args.workload, ROPE_SOURCES)}

    cpu = None
    if not args.no_cpu_baseline and not args.rope:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl)

    line = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) values, lengths and page tables drawn per the workload recipe)",
        "config": {"workload": args.workload, "batch": wl.B, "total_q": wl.Tq, "total_new": wl.Tn,
                   "q_heads": wl.Hq, "kv_heads": wl.Hkv, "head_dim": wl.D,
                   "page_size": wl.page_size, "causal": wl.causal,
                   "kv_cache": wl.cache_dtype or "none", "pages": wl.num_pages,
                   "flops_per_step": step_flops, "kv_bytes_per_step": step_bytes,
                   "parallelism": "single GPU", **({"rope": "rotary_dim=head_dim, half-split"}
                                                   if args.rope else {})},
        "pct_of_peak": 100.0 * value / (PEAK_HBM_GBS if decode else PEAK_BF16_TFLOPS),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if rope_line is not None:
        line["rope_kernel"] = rope_line
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
