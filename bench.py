#!/usr/bin/env python3
"""Benchmark of the paged KV-cache attention step on one MI355X.

A step is one pass of the whole hot path over one batch:
fused slot addressing + append of the step's new K/V rows -> decode attention
(stream-K partition of the batch's pages + merge of the cut segments, or
split-K partials + combine with --num-splits) and/or varlen prefill, per
layer.  The default workload is the bandwidth-bound decode: 256 sequences
with context U[1024, 8192], 32 query / 8 KV heads, head_dim 128, page 32,
random page order.  Inputs (pools, tables, queries, new rows) are resident
in HBM before the timed region starts.

Prints ONE JSON line.  ``value`` is the step's algorithmic HBM traffic
divided by the measured step time (GB/s); ``roofline`` reports the
dominant kernel (the decode kernel; the prefill kernel for the prefill-only
workload) against its peak, timed with HIP events on the stream it runs on.
``cpu_baseline`` times the CPU oracle on a bounded sample of the same
workload.  Steps whose K/V fit in the last-level caches are timed after a
cache scrub (see --scrub).  The step is also captured once as a step graph
and replayed (see --graph), as the rollout engine replays its decode step;
the JSON then reports the replay time, with the eager time beside it.
Every launch of the step takes lengths and tables from device memory and
sizes its grid from host bounds only, so prefill launches are captured too
(one graph per set of host bounds).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA

DESCRIPTIONS = {
    "tiny_decode": "4 decode seqs, ctx {5,17,32,63}, Hq/Hkv/D 2/1/64, page 16, 32-page pool",
    "qwen3_decode": "32 decode seqs, ctx U[128,1024], Hq/Hkv/D 32/8/128, page 32",
    "mixed_step": "8 prompts U[64,256] + 56 decoders ctx U[256,2048], 32/8/128, page 32",
    "large_decode": "256 decode seqs, ctx U[1024,8192], Hq/Hkv/D 32/8/128, page 32, random page order",
    "window_shared": "64 decoders ctx U[512,4096] + 4 chunks of 128 after U[512,4096], "
                     "8/1/256, page 32, window 512, 2 layers sharing the pool",
    "long_prefill": "16 prompts U[1024,4096], 32/8/128, page 32 (prefill only)",
    "full512_decode": "64 decode seqs, ctx U[512,4096], Hq/Hkv/D 8/1/512, page 32 (full attention)",
    "full512_prefill": "8 prompts U[1024,4096], 8/1/512, page 32 (full attention, prefill only)",
}

# key splits of the single varlen launch per workload (pkv_prefill_varlen_split);
# workloads not listed use one (pkv_prefill_varlen)
PREFILL_SPLITS = {"window_shared": 4}


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def _src_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_kv_attention_mapped_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# algorithmic work
# ---------------------------------------------------------------------------
def decode_key_lens(wl):
    L = wl.total_lens[:wl.n_decode].astype(np.int64)
    return np.minimum(L, wl.window) if wl.window > 0 else L


def decode_kernel_bytes(wl) -> int:
    """K/V rows attended + q + table entries + lengths (the split kernel's inputs)."""
    le = decode_key_lens(wl)
    kv = int(le.sum()) * wl.num_kv_heads * wl.head_dim * 2 * 2
    q = wl.n_decode * wl.num_q_heads * wl.head_dim * 2
    # pages holding allowed keys (window start page to the last page)
    L = wl.total_lens[:wl.n_decode].astype(np.int64)
    first = np.maximum(0, L - wl.window) if wl.window > 0 else np.zeros_like(L)
    pages = -(-L // wl.page_size) - first // wl.page_size
    return kv + q + 4 * int(pages.sum()) + 4 * wl.n_decode


def fused_append_bytes(wl) -> int:
    """The decode step's append done inside the decode launch: each new K/V
    row read from k_new/v_new and written to the pool (the table entry is
    already counted by the decode)."""
    return 2 * 2 * wl.n_decode * wl.num_kv_heads * wl.head_dim * 2


def decode_bytes(wl) -> int:
    return decode_kernel_bytes(wl) + wl.n_decode * wl.num_q_heads * wl.head_dim * 2  # + out


def append_bytes(wl) -> int:
    T = int(wl.new_lens.sum())
    return 2 * 2 * T * wl.num_kv_heads * wl.head_dim * 2 + 4 * T  # rows r+w, table entries


def prefill_flops(wl) -> int:
    """4 * D * Hq * (number of (row, key) pairs the masks allow)."""
    pairs = 0
    for s in wl.prefill_ids():
        lq, lk = int(wl.new_lens[s]), int(wl.total_lens[s])
        pos = np.arange(lk - lq, lk)
        cnt = pos + 1
        if wl.window > 0:
            cnt = np.minimum(cnt, wl.window)
        pairs += int(cnt.sum())
    return 4 * wl.head_dim * wl.num_q_heads * pairs


def prefill_bytes(wl) -> int:
    s = wl.prefill_ids()
    tq = int(wl.new_lens[s].sum())
    kv = int(wl.total_lens[s].sum()) * wl.num_kv_heads * wl.head_dim * 2 * 2
    return kv + 2 * tq * wl.num_q_heads * wl.head_dim * 2


# ---------------------------------------------------------------------------
# the step on the GPU
# ---------------------------------------------------------------------------
class Step:
    def __init__(self, wl, torch, P, num_splits=0, mixed="single", prefill_splits=1,
                 append="fused"):
        self.wl, self.torch, self.P = wl, torch, P
        dev = torch.device("cuda")
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)  # noqa: E731
        bits = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).to(dev)  # noqa: E731
        shape = (wl.num_kv_heads, wl.num_slots, wl.head_dim)
        self.k_pool = torch.full(shape, 0x7FC0, dtype=torch.int16, device=dev)
        self.v_pool = torch.full(shape, 0x7FC0, dtype=torch.int16, device=dev)
        self.bt = i32(wl.block_tables)
        # cached context, written once (not timed)
        for i in range(0, wl.num_seqs, 32):
            sub = np.arange(i, min(wl.num_seqs, i + 32))
            wl.cache_all_kv(sub)
            k, v, lq, lk = wl.packed_tokens("prefix", sub)
            nk, nv, _, _ = wl.packed_tokens("new", sub)
            self._keep_new = getattr(self, "_keep_new", []) + [(nk, nv)]
            for s in sub:
                wl._kv_cache.pop(int(s), None)
            if k.shape[0]:
                slots = P.slot_mapping(i32(wl.block_tables[sub]), i32(wl.cu_lens(lq)),
                                       i32(wl.cu_lens(lk)), page_size=wl.page_size,
                                       num_pages=wl.num_pages, total_tokens=k.shape[0])
                P.append(bits(k), bits(v), slots, self.k_pool, self.v_pool)
        torch.cuda.synchronize()
        nk = np.concatenate([a for a, _ in self._keep_new])
        nv = np.concatenate([b for _, b in self._keep_new])
        del self._keep_new
        # this step's new rows and their addressing inputs
        self.k_new, self.v_new = bits(nk), bits(nv)
        self.T = nk.shape[0]
        self.max_new = int(wl.new_lens.max())
        self.cu_new_q = i32(wl.cu_lens(wl.new_lens))
        self.cu_new_k = i32(wl.cu_lens(wl.total_lens))
        # decode
        self.B = wl.n_decode
        if self.B:
            lens = wl.decode_seq_lens()
            self.seq_lens = i32(lens)
            self.max_len = int(lens.max())
            self.bt_dec = i32(wl.block_tables[:self.B])
            hq, d = wl.num_q_heads, wl.head_dim
            self.out_dec = torch.empty((self.B, hq, d), dtype=torch.bfloat16, device=dev)
            self.S, self.pps, self.nw = 0, 0, 0
            # the decomposition the library picks for these arguments
            self.method, cnt = P.decode_method(self.B, hq, wl.num_kv_heads, d, wl.page_size,
                                               self.max_len, wl.window, num_splits)
            if self.method == "stream":
                # stream-K: persistent waves over the flattened page list + merge
                self.nw = cnt
                need = P.lib().pkv_decode_stream_workspace_bytes(self.nw, hq, wl.num_kv_heads, d)
                self.ws = torch.empty(need, dtype=torch.uint8, device=dev)
            elif self.method == "direct":
                self.S, self.pps = 1, 0
            else:
                self.S, self.pps = P.decode_plan(self.B, wl.num_kv_heads, wl.page_size,
                                                 self.max_len, wl.window, num_splits)
                self.part = (torch.empty((self.B, hq, self.S), dtype=torch.float32, device=dev),
                             torch.empty((self.B, hq, self.S), dtype=torch.float32, device=dev),
                             torch.empty((self.B, hq, self.S, d), dtype=torch.float32, device=dev))
        # prefill
        self.N = wl.n_prefill
        if self.N:
            seqs = wl.prefill_ids()
            self.bt_pre = i32(wl.block_tables[seqs])
            self.cu_q = i32(wl.prefill_cu_q())
            self.cu_k = i32(wl.prefill_cu_k())
            self.max_q = int(wl.new_lens[seqs].max())
            self.max_k = int(wl.total_lens[seqs].max())
            self.out_pre = torch.empty((wl.total_q(), wl.num_q_heads, wl.head_dim),
                                       dtype=torch.bfloat16, device=dev)
            self.psplits = max(1, int(prefill_splits))
            nb = P.prefill_split_workspace_bytes(wl.total_q(), wl.num_q_heads, wl.head_dim,
                                                 self.psplits)
            self.pws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
        self.q = []
        for layer in range(wl.num_layers):
            qd, qp = wl.queries(layer)
            self.q.append((bits(qd), bits(qp)))
        # a decode-only step appends its new rows inside the decode launch
        # (pkv_decode_append); the workspace is whatever the decomposition needs
        self.fused = append == "fused" and self.B > 0 and self.N == 0
        if self.fused:
            need = P.decode_workspace_bytes(self.B, wl.num_q_heads, wl.head_dim, wl.num_kv_heads,
                                            wl.page_size, self.max_len, wl.window, num_splits)
            self.fws = torch.empty(max(1, need), dtype=torch.uint8, device=dev)
            self.num_splits = num_splits
        # mixed steps in one varlen launch: decode rows are one-row sequences
        self.single = mixed == "single" and self.B > 0 and self.N > 0
        if self.single:
            self.q_all = [bits(np.concatenate(wl.queries(layer))) for layer in range(wl.num_layers)]
            self.out_all = torch.empty((self.B + wl.total_q(), wl.num_q_heads, wl.head_dim),
                                       dtype=torch.bfloat16, device=dev)
            self.max_k_all = int(wl.total_lens.max())
            # key splits of the single launch (pkv_prefill_varlen_split) and their workspace
            self.psplits = max(1, int(prefill_splits))
            nb = P.prefill_split_workspace_bytes(self.B + wl.total_q(), wl.num_q_heads,
                                                 wl.head_dim, self.psplits)
            self.pws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None

    def run(self, ev=None, pev=None):
        """One step.  ``ev`` / ``pev`` = (before, after) events bracketing the layer-0 decode
        kernel / prefill kernel."""
        P, wl = self.P, self.wl
        if self.fused:
            for layer in range(wl.num_layers):
                qd, _ = self.q[layer]
                if ev is not None and layer == 0:
                    ev[0].record()
                if layer == 0:   # later layers share the pool: no second append
                    P.decode_append(qd, self.k_new, self.v_new, self.k_pool, self.v_pool,
                                    self.bt_dec, self.seq_lens, self.max_len,
                                    page_size=wl.page_size, scale=wl.scale, window=wl.window,
                                    num_splits=self.num_splits, workspace=self.fws,
                                    out=self.out_dec)
                else:
                    P.decode(qd, self.k_pool, self.v_pool, self.bt_dec, self.seq_lens,
                             self.max_len, page_size=wl.page_size, scale=wl.scale,
                             window=wl.window, num_splits=self.num_splits, workspace=self.fws,
                             out=self.out_dec)
                if ev is not None and layer == 0:
                    ev[1].record()
            return
        P.append_mapped(self.k_new, self.v_new, self.bt, self.cu_new_q, self.cu_new_k,
                        self.k_pool, self.v_pool, page_size=wl.page_size,
                        max_seqlen_q=self.max_new)
        if self.single:
            for layer in range(wl.num_layers):
                if ev is not None and layer == 0:
                    ev[0].record()
                if self.psplits > 1:
                    P.prefill_varlen_split(self.q_all[layer], self.k_pool, self.v_pool, self.bt,
                                           self.cu_new_q, self.cu_new_k, self.max_new,
                                           self.max_k_all, page_size=wl.page_size,
                                           num_splits=self.psplits, scale=wl.scale,
                                           window=wl.window, out=self.out_all,
                                           workspace=self.pws)
                else:
                    P.prefill_varlen(self.q_all[layer], self.k_pool, self.v_pool, self.bt,
                                     self.cu_new_q, self.cu_new_k, self.max_new, self.max_k_all,
                                     page_size=wl.page_size, scale=wl.scale, window=wl.window,
                                     out=self.out_all)
                if ev is not None and layer == 0:
                    ev[1].record()
            return
        for layer in range(wl.num_layers):
            qd, qp = self.q[layer]
            if self.B:
                if ev is not None and layer == 0:
                    ev[0].record()
                if self.nw:
                    P.decode_stream(qd, self.k_pool, self.v_pool, self.bt_dec, self.seq_lens,
                                    page_size=wl.page_size, num_waves=self.nw, scale=wl.scale,
                                    window=wl.window, workspace=self.ws, out=self.out_dec)
                    if ev is not None and layer == 0:
                        ev[1].record()
                    P.decode_stream_merge(self.ws, self.out_dec, num_waves=self.nw,
                                          num_kv_heads=wl.num_kv_heads)
                elif self.S > 1:
                    P.decode_split(qd, self.k_pool, self.v_pool, self.bt_dec, self.seq_lens,
                                   self.max_len, page_size=wl.page_size, num_splits=self.S,
                                   pages_per_split=self.pps, scale=wl.scale, window=wl.window,
                                   out=self.part)
                    if ev is not None and layer == 0:
                        ev[1].record()
                    P.decode_combine(*self.part, out=self.out_dec)
                else:
                    P.decode(qd, self.k_pool, self.v_pool, self.bt_dec, self.seq_lens,
                             self.max_len, page_size=wl.page_size, scale=wl.scale,
                             window=wl.window, num_splits=1, out=self.out_dec)
                    if ev is not None and layer == 0:
                        ev[1].record()
            if self.N:
                if pev is not None and layer == 0:
                    pev[0].record()
                if self.psplits > 1:
                    P.prefill_varlen_split(qp, self.k_pool, self.v_pool, self.bt_pre, self.cu_q,
                                           self.cu_k, self.max_q, self.max_k,
                                           page_size=wl.page_size, num_splits=self.psplits,
                                           scale=wl.scale, window=wl.window, out=self.out_pre,
                                           workspace=self.pws)
                else:
                    P.prefill_varlen(qp, self.k_pool, self.v_pool, self.bt_pre, self.cu_q,
                                     self.cu_k, self.max_q, self.max_k, page_size=wl.page_size,
                                     scale=wl.scale, window=wl.window, out=self.out_pre)
                if pev is not None and layer == 0:
                    pev[1].record()

    def run_prefill(self):
        wl = self.wl
        self.P.prefill_varlen(self.q[0][1], self.k_pool, self.v_pool, self.bt_pre, self.cu_q,
                              self.cu_k, self.max_q, self.max_k, page_size=wl.page_size,
                              scale=wl.scale, window=wl.window, out=self.out_pre)


SCRUB_BYTES = 1 << 30


def copy_ceiling(torch, nbytes=1 << 31, reps=5):
    """Read+write GB/s of a plain 2 GiB device copy: the device's practical HBM
    ceiling, context for the roofline (whose peak stays at 8 TB/s)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return round(gbs, 1)


def step_bytes(wl) -> int:
    b = append_bytes(wl)
    if wl.n_decode:
        b += wl.num_layers * decode_bytes(wl)
    if wl.n_prefill:
        b += wl.num_layers * prefill_bytes(wl)
    return b


# ---------------------------------------------------------------------------
# CPU oracle baseline (bounded sample)
# ---------------------------------------------------------------------------
def cpu_baseline(wl, budget_s: float, max_seqs: int, prefill_rows: int = 128):
    """Time the oracle on whole sequences of the workload until ``budget_s``.

    Each sampled sequence gets a pool of its own holding just its pages (the
    pages keep their relative order), filled with its cached context outside
    the timed region; the timed part is that sequence's share of the step:
    slot mapping + append of its new rows + the float64 oracle attention of
    its rows for every layer.  A decode row is attended whole; a prompt or
    chunk is attended on ``prefill_rows`` evenly spaced rows and its time is
    scaled by the share of its (row, key) pairs those rows hold (the
    oracle's cost is proportional to the pairs).  The throughput is the
    sampled sequences' share of the step's algorithmic bytes over the
    estimated oracle time.
    """
    import oracle

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    cores = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(7)
    order = rng.permutation(wl.num_seqs)[:max_seqs]
    qs = [wl.queries(layer) for layer in range(wl.num_layers)]
    cq = wl.cu_lens(wl.new_lens)
    done, t_meas, t_est, sampled_rows = [], 0.0, 0.0, 0
    for i, s in enumerate(order):
        s = int(s)
        if i % 32 == 0:  # generate the next sequences' K/V (untimed) in threads, 32 at a time
            wl.drop_kv()
            wl.cache_all_kv(order[i:i + 32])
        npg = -(-int(wl.total_lens[s]) // wl.page_size)
        phys = wl.block_tables[s, :npg]
        bt = np.argsort(np.argsort(phys)).astype(np.int32)[None, :]
        shape = (wl.num_kv_heads, npg * wl.page_size, wl.head_dim)
        kp = np.full(shape, 0x7FC0, np.uint16)
        vp = kp.copy()
        k, v, lq, lk = wl.packed_tokens("prefix", [s])
        if k.shape[0]:
            kp, vp = oracle.append(kp, vp, k, v, oracle.slot_mapping(
                bt, wl.cu_lens(lq), wl.cu_lens(lk), wl.page_size))
        nk, nv, lq, lk = wl.packed_tokens("new", [s])
        Lq, Lk = int(lq[0]), int(lk[0])
        t0 = time.perf_counter()
        slots = oracle.slot_mapping(bt, wl.cu_lens(lq), wl.cu_lens(lk), wl.page_size)
        kp, vp = oracle.append(kp, vp, nk, nv, slots)
        t_app = time.perf_counter() - t0
        t_att, frac = 0.0, 1.0
        if s < wl.n_decode:
            for qd, _ in qs:
                t1 = time.perf_counter()
                oracle.decode(qd[[s]], kp, vp, bt, wl.total_lens[[s]], wl.page_size, wl.scale,
                              wl.window)
                t_att += time.perf_counter() - t1
        elif Lq > 0:
            pos = np.arange(Lk - Lq, Lk)
            pairs = pos + 1 if wl.window <= 0 else np.minimum(pos + 1, wl.window)
            rows = np.unique(np.linspace(0, Lq - 1, min(Lq, prefill_rows)).round().astype(int))
            frac = float(pairs[rows].sum() / pairs.sum())
            j = s - wl.n_decode
            for _, qp in qs:
                t1 = time.perf_counter()
                K = oracle.gather(kp, bt[0], Lk, wl.page_size)
                V = oracle.gather(vp, bt[0], Lk, wl.page_size)
                oracle.attend_rows(oracle.bf16_to_f64(qp[cq[s] - cq[wl.n_decode] + rows]), K, V,
                                   pos[rows], wl.scale, wl.window)
                t_att += time.perf_counter() - t1
            sampled_rows += len(rows)
        t_meas += t_app + t_att
        t_est += t_app + t_att / frac
        done.append(s)
        if t_meas > budget_s:
            break
    wl.drop_kv()
    sub = _subset(wl, done)
    bytes_done = step_bytes(sub)
    n_dec = int(sum(1 for s in done if s < wl.n_decode))
    what = [f"{len(done)} of {wl.num_seqs} sequences of {wl.name} ({n_dec} decode rows"]
    if len(done) > n_dec:
        what.append(f", {len(done) - n_dec} prompts/chunks attended on {sampled_rows} evenly "
                    f"spaced rows and scaled by their share of the (row, key) pairs")
    return {
        "value": round(bytes_done / t_est / 1e9, 6),
        "unit": "GB/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": ("".join(what) + "), each timed for its share of the step (slot mapping + "
                   f"append + float64 attention, {wl.num_layers} layer(s)); {t_meas:.1f} s of "
                   f"oracle work, {t_est:.1f} s estimated for the sampled sequences' full share; "
                   f"{cores} host cores available, BLAS threads {blas_threads}"),
        "seconds": round(t_meas, 3),
        "estimated_seconds": round(t_est, 3),
        "tokens_per_s": round(len(done) / t_est, 4) if n_dec == len(done) else None,
    }


def _subset(wl, seqs):
    import copy
    sub = copy.copy(wl)
    seqs = np.asarray(sorted(seqs))
    dec = seqs[seqs < wl.n_decode]
    pre = seqs[seqs >= wl.n_decode]
    keep = np.concatenate([dec, pre])
    sub.prefix_lens = wl.prefix_lens[keep]
    sub.new_lens = wl.new_lens[keep]
    sub.block_tables = wl.block_tables[keep]
    sub.n_decode, sub.n_prefill = len(dec), len(pre)
    return sub


# ---------------------------------------------------------------------------
# measured traffic (rocprofv3 counters, recorded under profiles/)
# ---------------------------------------------------------------------------
def recorded_traffic(config: str, src_hash: str, fused: bool = False):
    path = os.path.join(ROOT, "profiles",
                        f"{config}_decode{'_append' if fused else ''}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != src_hash:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
def prefill_measure(torch, P, iters=20, warmup=40):
    """The long prefill's MFMA fraction: each launch timed by its own event
    pair, back to back on resident K/V, and the same kernel inside the
    long-prefill step (its prompts' rows appended just before it); medians
    over the launches.  The warm-up is long enough for the clock to settle:
    the first few dozen launches of a burst run up to ~10% faster than the
    steady state that follows, with or without an append between them."""
    import workloads as W
    wl = W.make("long_prefill")
    st = Step(wl, torch, P)
    for _ in range(warmup):
        st.run_prefill()
    torch.cuda.synchronize()

    def evpair():
        return (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    evs = [evpair() for _ in range(iters)]
    for a, b in evs:
        a.record()
        st.run_prefill()
        b.record()
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    sevs = [evpair() for _ in range(iters)]
    for pe in sevs:
        st.run(None, pe)
    torch.cuda.synchronize()
    sms = np.array([a.elapsed_time(b) for a, b in sevs])
    fl = prefill_flops(wl)
    med, smed = float(np.median(ms)), float(np.median(sms))
    tf, stf = fl / (med * 1e-3) / 1e12, fl / (smed * 1e-3) / 1e12
    del st
    torch.cuda.empty_cache()
    return {"workload": "long_prefill: " + DESCRIPTIONS["long_prefill"],
            "ms_per_call": round(med, 4), "mean_ms": round(float(ms.mean()), 4),
            "min_ms": round(float(ms.min()), 4), "tflops": round(tf, 2),
            "peak_tflops": BF16_PEAK_TFLOPS, "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "flops_per_call": fl,
            "timing": f"median of {iters} launches back to back, each between its own events, "
                      f"after {warmup} untimed launches (steady clock)",
            "in_step": {"ms_per_call": round(smed, 4), "tflops": round(stf, 2),
                        "mfma_frac": round(stf / BF16_PEAK_TFLOPS, 4),
                        "timing": "median of the prefill launch inside the long-prefill step "
                                  "(the prompts' rows appended first), its own events"}}


def read_ceiling(torch, P, nbytes=4 << 30, reps=5):
    """A plain streaming read of 4 GiB (pkv_stream_read): the device's
    practical HBM read ceiling (context; the roofline's peak stays 8 TB/s).
    The best workgroup count of a short sweep; median of ``reps`` reads."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(3)
    cus, _ = P.device_info()
    best = None
    for per_cu in (1, 2, 4, 8, 16):
        wg = cus * per_cu
        sink = torch.empty(4 * wg, dtype=torch.int32, device="cuda")
        for _ in range(2):
            P.stream_read(buf, wg, sink)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for a, b in evs:
            a.record()
            P.stream_read(buf, wg, sink)
            b.record()
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
        gbs = nbytes / (ms * 1e-3) / 1e9
        if best is None or gbs > best["gbs"]:
            best = {"gbs": round(gbs, 1), "bytes": nbytes, "workgroups": wg, "ms": round(ms, 4)}
    del buf
    torch.cuda.empty_cache()
    best["frac_of_peak"] = round(best["gbs"] / HBM_PEAK_GBS, 4)
    best["kernel"] = "stream_read_kernel (pkv_stream_read): 16-byte nontemporal loads, 8 in flight"
    return best


def alloc_measure(torch, P, num_seqs=256, iters=200):
    """Device page allocator: 256 fresh sequences of 1..128 tokens take their
    pages (1..4 of 32 tokens each) from a 32768-page stack and release them
    again; ``iters`` alloc + release pairs run back to back inside step
    graphs between two HIP events."""
    dev = "cuda"
    ps, width, num_pages = 32, 256, 32768
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)  # noqa: E731
    rng = np.random.default_rng(11)
    lens = rng.integers(1, 4 * ps, num_seqs, endpoint=True)
    cu = i32(np.concatenate([[0], np.cumsum(lens)]))
    d_lens, rel = i32(lens), i32(np.ones(num_seqs, np.int32))
    d_bt = i32(np.full((num_seqs, width), -1, np.int32))
    d_free = i32(rng.permutation(num_pages))
    d_count, d_status = i32([num_pages]), i32([0])

    def pair():
        P.page_alloc(cu, cu, d_bt, d_free, d_count, page_size=ps, status=d_status)
        P.page_free(d_lens, rel, d_bt, d_free, d_count, page_size=ps, status=d_status)
    for _ in range(5):
        pair()
    # 20 pairs captured in one step graph and replayed, so the figure is the
    # GPU's (kernels and the gaps between them), not the Python loop's
    per_graph = 20
    gs = torch.cuda.Stream()
    gs.wait_stream(torch.cuda.current_stream())
    graph = P.capture_graph(lambda: [pair() for _ in range(per_graph)], gs)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(gs):
        graph.launch(gs)
        a.record()
        for _ in range(iters // per_graph):
            graph.launch(gs)
        b.record()
    torch.cuda.synchronize()
    graph.destroy()
    iters = (iters // per_graph) * per_graph
    ok = int(d_status.item()) == 0 and int(d_count.item()) == num_pages
    return {"num_seqs": num_seqs, "pages_per_alloc": int(np.sum(-(-lens // ps))),
            "alloc_plus_free_us": round(a.elapsed_time(b) * 1e3 / iters, 2),
            "state_ok": bool(ok),
            "note": "one workgroup each; latency-bound (a scan over the batch, a few KB moved)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="large_decode", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--num-splits", type=int, default=0,
                    help="0: automatic decomposition (stream-K); >= 1: split-K with that many splits")
    ap.add_argument("--mixed", choices=["single", "separate"], default="single",
                    help="a step with decode rows and prefill rows: one varlen launch per layer "
                         "(decode rows as one-row sequences) or decode + prefill launches")
    ap.add_argument("--append", choices=["fused", "separate"], default="fused",
                    help="a decode-only step: new rows written inside the decode launch "
                         "(pkv_decode_append) or by a separate append launch first")
    ap.add_argument("--prefill-splits", type=int, default=0,
                    help="key splits of the single varlen launch (pkv_prefill_varlen_split); "
                         "0: the workload's default")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the page-allocator timing and the copy / read ceilings")
    ap.add_argument("--no-prefill", action="store_true", help="skip the long-prefill MFMA measurement")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--scrub", choices=["auto", "on", "off"], default="auto",
                    help="1 GiB cache scrub before each timed step (auto: when the step's "
                         "algorithmic bytes are under 1 GiB)")
    ap.add_argument("--graph", choices=["on", "off"], default="on",
                    help="also time the step as a replayed step graph")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if world != 1:
        print(json.dumps({"error": "single-GPU build: launch without a multi-rank launcher"}), flush=True)
        sys.exit(2)

    import torch

    import paged_kv_attention_mapped_amd as P
    import workloads as W

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)
    P.lib()
    torch.cuda.set_device(0)

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n, "launches": 3}), flush=True)
        return

    wl = W.make(args.config)
    _log(f"[bench] setting up {args.config}: {DESCRIPTIONS[args.config]}")
    t0 = time.perf_counter()
    psplits = args.prefill_splits if args.prefill_splits > 0 else PREFILL_SPLITS.get(args.config, 1)
    st = Step(wl, torch, P, args.num_splits, args.mixed, psplits, args.append)
    _log(f"[bench] set-up done in {time.perf_counter() - t0:.1f} s; warmup {args.warmup}, steps {args.steps}")

    for _ in range(args.warmup):
        st.run()
    torch.cuda.synchronize()

    # A step whose K/V fit in the last-level caches (256 MB Infinity Cache +
    # L2) is timed after a 1 GiB scratch write, outside its events, so that
    # its K/V come from HBM as in a real model step; larger steps need none.
    scrub = args.scrub == "on" or (args.scrub == "auto" and step_bytes(wl) < SCRUB_BYTES)
    scratch = torch.empty(SCRUB_BYTES, dtype=torch.uint8, device="cuda") if scrub else None

    def evpair():
        return (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    evs = [evpair() for _ in range(args.steps)]      # decode kernel
    pevs = [evpair() for _ in range(args.steps)]     # prefill kernel
    sevs = [evpair() for _ in range(args.steps)]     # whole step
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if scrub:
            scratch.fill_(i & 0xff)
        sevs[i][0].record()
        st.run(evs[i] if st.B else None, pevs[i] if st.N and not st.single else None)
        sevs[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = np.array([a.elapsed_time(b) for a, b in sevs])
    # with scrubbing the scratch writes sit between the steps: time the steps by their events
    ms_step = float(step_ms.mean()) if scrub else wall / args.steps * 1e3
    _log(f"[bench] timed {args.steps} steps: {ms_step:.4f} ms/step"
         f"{' (cache scrubbed before each step)' if scrub else ''}")
    eager = {"ms_per_step": round(ms_step, 5),
             "median_ms_per_step": round(float(np.median(step_ms)), 5),
             "min_ms_per_step": round(float(step_ms.min()), 5)}

    graph_info = None
    if args.graph == "on":
        # the same step captured once on a side stream and replayed; the new
        # rows go to the same slots every step, so every replay's output must
        # equal the eager step's bit for bit
        outs = [st.out_all] if st.single else (
            ([st.out_dec] if st.B else []) + ([st.out_pre] if st.N else []))
        refs = [t.clone() for t in outs]
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        graph = P.capture_graph(st.run, gs)
        gsevs = [evpair() for _ in range(args.steps)]
        with torch.cuda.stream(gs):
            for _ in range(max(1, args.warmup)):
                graph.launch(gs)
            gs.synchronize()
            t0 = time.perf_counter()
            for i in range(args.steps):
                if scrub:
                    scratch.fill_(i & 0xff)
                gsevs[i][0].record()
                graph.launch(gs)
                gsevs[i][1].record()
            gs.synchronize()
        gwall = time.perf_counter() - t0
        g_ms = np.array([a.elapsed_time(b) for a, b in gsevs])
        g_step = float(g_ms.mean()) if scrub else gwall / args.steps * 1e3
        same = all(bool(torch.equal(t, r)) for t, r in zip(outs, refs))
        kn, on = graph.nodes()
        graph.destroy()
        _log(f"[bench] graph replay: {g_step:.4f} ms/step (eager {ms_step:.4f}); "
             f"matches eager: {same}")
        graph_info = {"used": True, "kernel_nodes": kn, "other_nodes": on,
                      "matches_eager": same, "ms_per_step": round(g_step, 5),
                      "median_ms_per_step": round(float(np.median(g_ms)), 5),
                      "min_ms_per_step": round(float(g_ms.min()), 5)}
        if same is False:
            raise SystemExit("graph replay differs from the eager step")
        ms_step, step_ms = g_step, g_ms

    sb = step_bytes(wl)
    value = sb / (ms_step * 1e-3) / 1e9
    out = {
        "metric": "paged-decode achieved HBM GB/s (% of peak) + decode tokens/s; prefill MFMA %",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: {DESCRIPTIONS[args.config]}",
                   "seed": wl.seed, "step_bytes": sb},
        "hbm_frac_step": round(value / HBM_PEAK_GBS, 4),
        "median_ms_per_step": round(float(np.median(step_ms)), 5),
        "min_ms_per_step": round(float(step_ms.min()), 5),
        "cache_scrub": bool(scrub),
        "step_graph": graph_info or {"used": False},
        "eager": eager,
    }
    if st.single:
        # one varlen launch per layer carries the decode rows and the prompts
        kern_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
        kb = decode_kernel_bytes(wl) + prefill_bytes(wl)
        fl = prefill_flops(wl)
        ach = kb / (kern_ms * 1e-3) / 1e9
        out["decode_tokens_per_s"] = round(st.B / (ms_step * 1e-3), 1)
        out["decode_plan"] = {"method": "single varlen launch (decode rows as one-row sequences)",
                              "prefill_key_splits": st.psplits}
        out["roofline"] = {
            "kernel": ("prefill_kernel (decode rows + prefill rows in one launch)" if st.psplits == 1
                       else f"prefill_kernel with up to {st.psplits} key runs per block + "
                            "split_merge_kernel (decode rows + prefill rows)"),
            "bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
            "avg_kernel_ms": round(kern_ms, 5), "algorithmic_bytes_per_launch": kb,
            "prefill_tflops": round(fl / (kern_ms * 1e-3) / 1e12, 2),
        }
    elif st.B:
        k_ms = np.array([a.elapsed_time(b) for a, b in evs])
        kern_ms = float(k_ms.mean())
        kb = decode_kernel_bytes(wl) + (fused_append_bytes(wl) if st.fused else 0)
        ach = kb / (kern_ms * 1e-3) / 1e9
        src_hash = _src_hash("decode.hip", "decode_core.h", "common.h")
        traffic = recorded_traffic(args.config, src_hash, st.fused)
        out["decode_tokens_per_s"] = round(st.B / (ms_step * 1e-3), 1)
        out["decode_plan"] = ({"method": "stream", "stream_k_waves": st.nw} if st.nw else
                              {"method": "direct"} if st.S == 1 else
                              {"method": "split", "num_splits": st.S,
                               "pages_per_split": st.pps})
        out["decode_plan"]["append"] = ("fused into the decode launch (pkv_decode_append)"
                                        if st.fused else "separate launch (pkv_append_mapped)")
        kname = ("decode_stream_kernel (stream-K)" if st.nw else
                 "decode_kernel (split-K partials)" if st.S > 1 else "decode_kernel (direct)")
        if wl.head_dim == 512:
            kname = ("attn512_stream_kernel (stream-K over workgroups)" if st.nw else
                     "attn512_kernel (head-dim split, " +
                     ("split-K partials)" if st.S > 1 else "direct)"))
        if st.fused:
            own = wl.head_dim == 512 and not st.nw  # head_dim 512 splits: append launch first
            kname = ("pkv_decode_append: " + ("append_last_kernel + " if own else "") + kname +
                     (" + stream_merge_kernel" if st.nw else " + combine_kernel" if st.S > 1 else "") +
                     (", the step's new rows appended by their own launch first" if own else
                      ", the step's new rows appended inside the decode launch"))
        out["roofline"] = {
            "kernel": kname,
            "bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
            "avg_kernel_ms": round(kern_ms, 5), "median_kernel_ms": round(float(np.median(k_ms)), 5),
            "algorithmic_bytes_per_launch": kb,
            "kernel_source_sha256_16": src_hash,
        }
        if not scrub:
            # the same decode call with the last-level caches scrubbed before
            # each launch (1 GiB write outside the events): shows whether the
            # back-to-back figure leans on data left in the 256 MB MALL
            sc = torch.empty(SCRUB_BYTES, dtype=torch.uint8, device="cuda")
            sev = [evpair() for _ in range(args.steps)]
            for i in range(args.steps):
                sc.fill_(i & 0xff)
                st.run(sev[i])
            torch.cuda.synchronize()
            s_ms = np.array([a.elapsed_time(b) for a, b in sev])
            del sc
            torch.cuda.empty_cache()
            sach = kb / (float(np.median(s_ms)) * 1e-3) / 1e9
            out["roofline_scrubbed"] = {
                "achieved": round(sach, 2), "frac": round(sach / HBM_PEAK_GBS, 4),
                "median_kernel_ms": round(float(np.median(s_ms)), 5),
                "note": "the decode call of the same step, each launch preceded by a 1 GiB "
                        "cache scrub (outside its events); median over the launches"}
    if st.N and not st.single:
        pk_ms = float(np.mean([a.elapsed_time(b) for a, b in pevs]))
        fl = prefill_flops(wl)
        tf = fl / (pk_ms * 1e-3) / 1e12
        pre = {"kernel": ("prefill_kernel (head_dim 512: one MFMA stream per key tile) + "
                          "attn512_kernel for the one-row sequences (none here)"
                          if wl.head_dim == 512 else "prefill_kernel"),
               "bound": "mfma", "achieved": round(tf, 3),
               "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
               "traffic": None, "avg_kernel_ms": round(pk_ms, 5), "algorithmic_flops_per_launch": fl}
        if st.B:
            # the step's prefill is a few GFLOP: launch-bound, reported as it is
            out["step_prefill"] = dict(pre, note="launch-bound at this size")
        else:
            out["roofline"] = pre
    del st
    torch.cuda.empty_cache()

    if not args.no_prefill and args.config != "long_prefill":
        _log("[bench] long-prefill MFMA measurement")
        out["prefill"] = prefill_measure(torch, P)
    if scratch is not None:
        del scratch
        torch.cuda.empty_cache()
    if not args.no_extras:
        out["page_allocator"] = alloc_measure(torch, P)
        out["hbm_copy_ceiling_gbs"] = copy_ceiling(torch)
        out["hbm_read_ceiling"] = read_ceiling(torch, P)
    if not args.no_cpu_baseline:
        _log(f"[bench] CPU oracle baseline (~{args.cpu_budget:.0f} s)")
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget, 256)
    cus, khz = P.device_info()
    out["gpu"] = torch.cuda.get_device_name(0)
    out["device"] = {"compute_units": cus, "max_sclk_mhz": khz // 1000,
                     "arch": torch.cuda.get_device_properties(0).gcnArchName}
    out["host"] = platform.node()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
