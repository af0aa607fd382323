"""Helpers for the GPU parity tests: move a synthetic workload to the device,
call the library through the binding, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import varlen_paged_kv_amd as vpk

# tolerances: bf16 workloads, and the fp8-KV workload (max-abs only relaxed)
TOL = {"bf16": dict(max_abs=2e-2, mean_abs=2e-3, lse=1e-3),
       "fp8": dict(max_abs=3e-2, mean_abs=2e-3, lse=1e-3)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_u8(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes)).cuda()


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


class DeviceCall:
    """Device copies of a workload's inputs, ready for repeated calls."""

    def __init__(self, wl, with_new=True):
        self.wl = wl
        self.q = dev_bf16(wl.q)
        self.cu_q = dev_i32(wl.cu_seqlens_q)
        self.with_new = with_new and wl.k_new is not None
        self.k_new = dev_bf16(wl.k_new) if self.with_new else None
        self.v_new = dev_bf16(wl.v_new) if self.with_new else None
        self.cu_kn = dev_i32(wl.cu_seqlens_knew) if self.with_new else None
        self.fp8 = wl.cache_dtype == "fp8"
        if wl.k_cache is not None:
            mk = dev_u8 if self.fp8 else dev_bf16
            self.k_cache = mk(wl.k_cache)
            self.v_cache = mk(wl.v_cache)
            self.bt = dev_i32(wl.block_table)
            self.cl = dev_i32(wl.cache_seqlens)
        else:
            self.k_cache = self.v_cache = self.bt = self.cl = None
        self.host = dict(cu_seqlens_q=wl.cu_seqlens_q,
                         cu_seqlens_knew=wl.cu_seqlens_knew if self.with_new else None,
                         cache_seqlens=wl.cache_seqlens, block_table=wl.block_table)

    def run(self, stream=None, out=None, lse=None):
        wl = self.wl
        return vpk.attn_varlen_paged_fwd(
            self.q, self.cu_q, self.k_new, self.v_new, self.cu_kn, self.k_cache, self.v_cache,
            self.bt, self.cl, wl.page_size, wl.causal, wl.scale,
            wl.kv_scale if self.fp8 else None, out=out, lse=lse, host_index=self.host,
            stream=stream)

    def cache_host(self):
        if self.k_cache is None:
            return None, None
        if self.fp8:
            return self.k_cache.cpu().numpy(), self.v_cache.cpu().numpy()
        return (self.k_cache.view(torch.int16).cpu().numpy().view(np.uint16),
                self.v_cache.view(torch.int16).cpu().numpy().view(np.uint16))


def oracle_full(wl, with_new=True):
    return oracle.run_call(q=wl.q, cu_seqlens_q=wl.cu_seqlens_q,
                           k_new=wl.k_new if with_new else None,
                           v_new=wl.v_new if with_new else None,
                           cu_seqlens_knew=wl.cu_seqlens_knew if with_new else None,
                           k_cache=wl.k_cache, v_cache=wl.v_cache, block_table=wl.block_table,
                           cache_seqlens=wl.cache_seqlens, page_size=wl.page_size,
                           causal=wl.causal, scale=wl.scale, kv_scale=wl.kv_scale,
                           cache_dtype=wl.cache_dtype)


def to_np_out(out: torch.Tensor) -> np.ndarray:
    return out.float().cpu().numpy().astype(np.float64)


def check_attention(out_np, lse_np, ref_out, ref_lse, kind="bf16", rows=None, label=""):
    """Compare GPU out [R, Hq, D] / lse [Hq, R] with the oracle's float64 values."""
    tol = TOL[kind]
    dead = np.isneginf(ref_lse)                      # [Hq, R]: rows that see no key
    assert np.array_equal(np.isneginf(lse_np), dead), f"{label}: -inf rows differ"
    dead_rows = dead.T                               # [R, Hq]
    assert np.all(out_np[dead_rows] == 0), f"{label}: rows with no key must be 0"
    live = ~dead_rows
    err = np.abs(out_np - ref_out)[live]
    assert np.all(np.isfinite(out_np)), f"{label}: non-finite output"
    if err.size:
        mx, mean = float(err.max()), float(err.mean())
        assert mx <= tol["max_abs"], f"{label}: max-abs {mx:.3e} > {tol['max_abs']}"
        assert mean <= tol["mean_abs"], f"{label}: mean-abs {mean:.3e} > {tol['mean_abs']}"
        le = float(np.abs(lse_np[~dead] - ref_lse[~dead]).max())
        assert le <= tol["lse"], f"{label}: lse max-abs {le:.3e} > {tol['lse']}"
        return mx, mean, le
    return 0.0, 0.0, 0.0


def run_and_check(wl, label, with_new=True):
    """One direct call on the device against the oracle's whole call: attention within tolerance,
    appended cache bytes bit for bit."""
    say(f"[case] {label}: B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} D={wl.D} S={wl.page_size} "
        f"causal={wl.causal} cache={wl.cache_dtype} seed={wl.seed}")
    dc = DeviceCall(wl, with_new=with_new)
    out, lse = dc.run()
    torch.cuda.synchronize()
    ref = oracle_full(wl, with_new=with_new)
    kind = "fp8" if wl.cache_dtype == "fp8" else "bf16"
    errs = check_attention(to_np_out(out), lse.cpu().numpy().astype(np.float64), ref["out"],
                           ref["lse"], kind, label=label)
    kc, vc = dc.cache_host()
    if kc is not None:
        assert np.array_equal(kc, ref["k_cache"]), f"{label}: k_cache bytes differ"
        assert np.array_equal(vc, ref["v_cache"]), f"{label}: v_cache bytes differ"
    say(f"[ok] {label}: max {errs[0]:.2e} mean {errs[1]:.2e} lse {errs[2]:.2e}")
    return dc, out, lse

