"""Shared set-up for the GPU tests: the same seeded workload is placed in GPU
pools through the HIP path and in CPU pools through the oracle, and the two
are compared.  The oracle never sees a value produced on the GPU."""
from __future__ import annotations

import concurrent.futures as cf
import os
import sys

import numpy as np
import torch

import oracle
import paged_kv_attention_mapped_amd as P
import workloads as W

# Tolerance for bf16 outputs with fp32 accumulation, against the float64 oracle.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def dev_bits(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def as_f64(bits) -> np.ndarray:
    return W.bf16_to_f32(bits).astype(np.float64)


def check_close(gpu_bits, ref, what="", max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    g = as_f64(gpu_bits)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref)
    mx, mn = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    rms = float(np.sqrt(np.mean((g - ref) ** 2)) / max(1e-30, np.sqrt(np.mean(ref ** 2)))) if err.size else 0.0
    say(f"  {what}: max_abs={mx:.3e} mean_abs={mn:.3e} rms_rel={rms:.3e}")
    assert mx <= max_abs and mn <= mean_abs, (what, mx, mn)


class GpuPools:
    """Poisoned GPU pools of a workload, filled through pkv_slot_mapping + pkv_append
    (or through pkv_append_mapped when ``fused``)."""

    def __init__(self, wl: W.Workload):
        self.wl = wl
        shape = (wl.num_kv_heads, wl.num_slots, wl.head_dim)
        self.k = torch.full(shape, int(W.BF16_NAN), dtype=torch.int16, device="cuda")
        self.v = torch.full(shape, int(W.BF16_NAN), dtype=torch.int16, device="cuda")
        self.bt = dev_i32(wl.block_tables)

    def write(self, part: str, seqs=None, chunk=64, fused=False, slots_log=None, keep_new=None):
        """Append the ``part`` tokens of ``seqs`` (default all), a few sequences at a time.

        With ``slots_log`` (a list) the fused path also returns every chunk's
        slot array, as ``(seqs, cu_q, cu_k, slots)`` tuples.  With ``keep_new``
        (a list) every chunk's ``packed_tokens("new")`` is kept there, so that
        the step's new rows need not be drawn again."""
        wl = self.wl
        seqs = np.arange(wl.num_seqs) if seqs is None else np.asarray(seqs)
        for i in range(0, len(seqs), chunk):
            sub = seqs[i:i + chunk]
            wl.cache_all_kv(sub)
            k, v, lq, lk = wl.packed_tokens(part, sub)
            if keep_new is not None:
                keep_new.append(wl.packed_tokens("new", sub))
            for s in sub:
                wl._kv_cache.pop(int(s), None)
            if k.shape[0] == 0:
                continue
            if fused:
                out = None if slots_log is None else torch.full(
                    (k.shape[0],), -7, dtype=torch.int32, device="cuda")
                P.append_mapped(dev_bits(k), dev_bits(v), dev_i32(wl.block_tables[sub]),
                                dev_i32(wl.cu_lens(lq)), dev_i32(wl.cu_lens(lk)), self.k, self.v,
                                page_size=wl.page_size, max_seqlen_q=int(lq.max()),
                                slot_mapping_out=out)
                if slots_log is not None:
                    slots_log.append((sub, wl.cu_lens(lq), wl.cu_lens(lk), out))
                continue
            slots = P.slot_mapping(dev_i32(wl.block_tables[sub]), dev_i32(wl.cu_lens(lq)),
                                   dev_i32(wl.cu_lens(lk)), page_size=wl.page_size,
                                   num_pages=wl.num_pages, total_tokens=k.shape[0])
            P.append(dev_bits(k), dev_bits(v), slots, self.k, self.v)
        torch.cuda.synchronize()


class OraclePools:
    """CPU pools of the same workload, filled through the oracle (only ``seqs``)."""

    def __init__(self, wl: W.Workload, seqs=None, parts=("prefix", "new")):
        self.wl = wl
        shape = (wl.num_kv_heads, wl.num_slots, wl.head_dim)
        self.k = np.full(shape, W.BF16_NAN, np.uint16)
        self.v = np.full(shape, W.BF16_NAN, np.uint16)
        seqs = np.arange(wl.num_seqs) if seqs is None else np.asarray(seqs)
        for part in parts:
            k, v, lq, lk = wl.packed_tokens(part, seqs)
            slots = oracle.slot_mapping(wl.block_tables[seqs], wl.cu_lens(lq), wl.cu_lens(lk),
                                        wl.page_size)
            self.k, self.v = oracle.append(self.k, self.v, k, v, slots)


def host_workers() -> int:
    """Worker threads for oracle work on the host (at most 16: the GPU machine's CPU share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def thread_map(fn, items):
    """``fn`` over ``items`` in host threads, one BLAS thread each, results in order."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1), cf.ThreadPoolExecutor(host_workers()) as ex:
        return list(ex.map(fn, items))


def compact_oracle_pools(wl: W.Workload, seqs, parts=("prefix", "new")):
    """Oracle pools holding only the pages of ``seqs``, renumbered in
    increasing physical order, filled through the oracle's slot mapping and
    append.  Returns ``(k, v, tables into them, the physical page of each
    compact page)``: compact page ``c`` stands for physical page
    ``phys[c]``, so the GPU pool rows of those pages must equal ``k``/``v``."""
    ps = wl.page_size
    seqs = np.asarray(seqs)
    npg = [-(-int(wl.total_lens[s]) // ps) for s in seqs]
    phys = np.sort(np.concatenate([wl.block_tables[s, :n] for s, n in zip(seqs, npg)]))
    assert np.unique(phys).size == phys.size, "sequences share a page"
    rank = {int(p): i for i, p in enumerate(phys)}
    bt = np.zeros((len(seqs), max(npg)), np.int32)
    for i, (s, n) in enumerate(zip(seqs, npg)):
        bt[i, :n] = [rank[int(p)] for p in wl.block_tables[s, :n]]
    shape = (wl.num_kv_heads, len(phys) * ps, wl.head_dim)
    k = np.full(shape, W.BF16_NAN, np.uint16)
    v = np.full(shape, W.BF16_NAN, np.uint16)
    for part in parts:
        kk, vv, lq, lk = wl.packed_tokens(part, seqs)
        if kk.shape[0]:
            slots = oracle.slot_mapping(bt, wl.cu_lens(lq), wl.cu_lens(lk), ps)
            k, v = oracle.append(k, v, kk, vv, slots)
    return k, v, bt, phys


def page_rows(phys, page_size) -> np.ndarray:
    """Pool rows of the given physical pages, page by page."""
    return (np.asarray(phys, np.int64)[:, None] * page_size + np.arange(page_size)).ravel()


def summarize(errs, what):
    """Apply the parity bar to all elements of a workload: ``errs`` is a list
    of (sum of |err|, count, max |err|) per piece."""
    tot = sum(e[0] for e in errs)
    cnt = sum(e[1] for e in errs)
    mx = max(e[2] for e in errs)
    say(f"  {what}: max_abs={mx:.3e} mean_abs={tot / cnt:.3e} over {cnt} elements")
    assert mx <= MAX_ABS and tot / cnt <= MEAN_ABS, (what, mx, tot / cnt)


def err_stats(gpu_bits, ref):
    g = as_f64(gpu_bits)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), "non-finite output"
    e = np.abs(g - ref)
    return float(e.sum()), int(e.size), float(e.max())
