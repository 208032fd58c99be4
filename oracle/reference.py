"""Oracle for paged KV-cache attention, in float64 on the CPU.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library and imports nothing from it.

Everything here is the plain definition of what the paged path computes:

* Pool layout.  One tensor per K and per V holding, for each KV head, all
  pages back to back: ``[Hkv, num_pages * page_size, D]``; a page is
  ``page_size`` consecutive token rows of one head.  (Benchmarks commit log
  1847125, flex_attention paged-KV engine entry, "Why this works" item 1:
  the cache is one contiguous ``[1, H, num_pages*page_size, D]`` tensor and
  a page table maps (logical batch, logical block) to a physical page.)
* Slot write.  New token rows land at a physical row address of the pool
  (same entry, "Files": the in-kernel ``k_cache[addr] = k_val`` write).
* Varlen packing.  Rows of several sequences are packed and delimited by
  ``cu_seq_lens_q`` / ``cu_seq_lens_k`` (CB sync-driver commit 5f3e1c9,
  "qwen3_grpo_unified.py fixes"; benchmarks README, "Flash Attention 4 on
  Blackwell (sm_100)" item 2, ``max_seqlen_q/k``).
* Masks.  Full attention is pure causal; sliding attention is causal and
  ``q_pos - kv_pos < window`` with a strict less-than (benchmarks commit
  log, per-regime sliding-window mask entry).

Readings taken where the pages are silent (each one is listed with its
reason in the design notes):

* query head ``h`` reads KV head ``h // (Hq // Hkv)`` (contiguous groups);
* a query row ``r`` of a sequence with ``Lq`` new and ``Lk`` total tokens
  sits at position ``Lk - Lq + r`` (bottom-right causal alignment; a decode
  row is the last position ``L - 1``);
* softmax attention with no bias, soft-cap or sink; ``window <= 0`` = off;
* a sequence with no allowed key yields a zero row.
"""
from __future__ import annotations

import math

import numpy as np

LOG2E = 1.0 / math.log(2.0)


# ---------------------------------------------------------------------------
# values
# ---------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (a bf16 is the top half of a float32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# addressing and the slot write
# ---------------------------------------------------------------------------
def slot_mapping(block_tables, cu_seq_lens_q, cu_seq_lens_k, page_size) -> np.ndarray:
    """Physical pool row of every new token.

    Token ``r`` of sequence ``j`` (``Lq_j`` new tokens, ``Lk_j`` tokens once
    they are cached) is logical position ``Lk_j - Lq_j + r``; logical page
    ``pos // page_size`` of the sequence maps through its block-table row to
    a physical page, and the row address is ``page * page_size + pos % page_size``.
    """
    bt = np.asarray(block_tables)
    cq = np.asarray(cu_seq_lens_q, dtype=np.int64)
    ck = np.asarray(cu_seq_lens_k, dtype=np.int64)
    out = np.empty(int(cq[-1]), dtype=np.int64)
    for j in range(len(cq) - 1):
        lq = cq[j + 1] - cq[j]
        lk = ck[j + 1] - ck[j]
        for r in range(lq):
            pos = lk - lq + r
            out[cq[j] + r] = int(bt[j, pos // page_size]) * page_size + pos % page_size
    return out


def append(k_pool, v_pool, k_new, v_new, slots):
    """Copy each new token's K and V rows (all KV heads) into its pool row.

    Pools are ``[Hkv, num_slots, D]`` bf16 bit patterns, new rows
    ``[T, Hkv, D]``; a negative slot means the token is skipped.  Returns
    new pools; the inputs are not modified.  The copy is bit-exact.
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    for t, s in enumerate(np.asarray(slots)):
        if s < 0:
            continue
        k_out[:, s, :] = k_new[t, :, :]
        v_out[:, s, :] = v_new[t, :, :]
    return k_out, v_out


def gather(pool, block_table_row, length, page_size) -> np.ndarray:
    """Logical ``[Hkv, length, D]`` view of one sequence, read page by page (float64)."""
    rows = []
    for i in range(int(length)):
        page = int(block_table_row[i // page_size])
        rows.append(page * page_size + i % page_size)
    rows = np.asarray(rows, dtype=np.int64)
    return bf16_to_f64(pool[:, rows, :])


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def allowed_keys(pos: int, window: int) -> np.ndarray:
    """Key positions a query at ``pos`` may attend: ``i <= pos`` and, with a
    window, ``pos - i < window``."""
    lo = 0 if window <= 0 else max(0, pos - window + 1)
    return np.arange(lo, pos + 1, dtype=np.int64)


def attend_rows(q_rows, K, V, positions, scale, window) -> np.ndarray:
    """Textbook softmax attention of query rows against one sequence's keys.

    ``q_rows`` ``[R, Hq, D]`` float64, ``K``/``V`` ``[Hkv, L, D]`` float64,
    ``positions[r]`` = the row's position.  For query head ``h`` the KV head
    is ``h // (Hq // Hkv)``; scores are ``scale * (k . q)`` over the allowed
    keys; ``out = sum_i softmax_i v_i`` with the max subtracted first.
    """
    R, Hq, D = q_rows.shape
    Hkv = K.shape[0]
    g = Hq // Hkv
    out = np.zeros((R, Hq, D), dtype=np.float64)
    for r in range(R):
        keys = allowed_keys(int(positions[r]), window)
        if keys.size == 0:
            continue
        for h in range(Hq):
            kh = h // g
            s = (K[kh, keys, :] @ q_rows[r, h, :]) * scale
            e = np.exp(s - s.max())
            out[r, h, :] = (e @ V[kh, keys, :]) / e.sum()
    return out


def attend_rows_matrix(q_rows, K, V, positions, scale, window, block=512) -> np.ndarray:
    """``attend_rows`` evaluated for many rows of a query head at once.

    The same definition as ``attend_rows`` -- scores ``scale * (k . q)``
    over the allowed keys of each row, the row maximum subtracted, the
    exponentials normalised by their sum, KV head ``h // (Hq // Hkv)`` --
    written with matrix products over a block of rows (``block`` rows at a
    time bound the ``[rows, keys]`` score matrix); a key outside a row's
    allowed set gets score ``-inf`` and so weight 0.  A row with no allowed
    key is zero.  Used where a per-row loop would take too long (prompts of
    thousands of rows).
    """
    R, Hq, D = q_rows.shape
    Hkv = K.shape[0]
    g = Hq // Hkv
    pos = np.asarray(positions, dtype=np.int64)
    out = np.zeros((R, Hq, D), dtype=np.float64)
    for r0 in range(0, R, block):
        p = pos[r0:r0 + block]
        hi = int(min(K.shape[1], p.max() + 1)) if p.size else 0
        if hi <= 0:
            continue
        keys = np.arange(hi, dtype=np.int64)
        allowed = keys[None, :] <= p[:, None]
        if window > 0:
            allowed &= (p[:, None] - keys[None, :]) < window
        has = allowed.any(axis=1)
        for h in range(Hq):
            kh = h // g
            s = (q_rows[r0:r0 + block, h, :] @ K[kh, :hi, :].T) * scale
            s = np.where(allowed, s, -np.inf)
            m = np.where(has, s.max(axis=1), 0.0)
            e = np.exp(s - m[:, None])
            tot = e.sum(axis=1)
            o = (e @ V[kh, :hi, :]) / np.where(has, tot, 1.0)[:, None]
            out[r0:r0 + block, h, :] = np.where(has[:, None], o, 0.0)
    return out


def decode(q, k_pool, v_pool, block_tables, seq_lens, page_size, scale, window=0) -> np.ndarray:
    """One decode row per sequence: ``q [B, Hq, D]`` attends its ``seq_lens[b]``
    cached tokens (the new token included) at position ``seq_lens[b] - 1``."""
    q = bf16_to_f64(q)
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        K = gather(k_pool, block_tables[b], L, page_size)
        V = gather(v_pool, block_tables[b], L, page_size)
        out[b] = attend_rows(q[b:b + 1], K, V, [L - 1], scale, window)[0]
    return out


def prefill_varlen(q, k_pool, v_pool, block_tables, cu_seq_lens_q, cu_seq_lens_k,
                   page_size, scale, window=0) -> np.ndarray:
    """Packed causal prefill: rows ``cu_q[j]..cu_q[j+1]`` of ``q [Tq, Hq, D]``
    belong to sequence ``j``; row ``r`` sits at position ``Lk_j - Lq_j + r``."""
    q = bf16_to_f64(q)
    out = np.zeros(q.shape, dtype=np.float64)
    cq = np.asarray(cu_seq_lens_q, dtype=np.int64)
    ck = np.asarray(cu_seq_lens_k, dtype=np.int64)
    for j in range(len(cq) - 1):
        lq = int(cq[j + 1] - cq[j])
        lk = int(ck[j + 1] - ck[j])
        if lq == 0:
            continue
        K = gather(k_pool, block_tables[j], lk, page_size)
        V = gather(v_pool, block_tables[j], lk, page_size)
        pos = np.arange(lk - lq, lk)
        out[cq[j]:cq[j + 1]] = attend_rows(q[cq[j]:cq[j + 1]], K, V, pos, scale, window)
    return out


# ---------------------------------------------------------------------------
# split-K (flash-decoding) partial results and their merge
# ---------------------------------------------------------------------------
def split_page_range(seq_len: int, page_size: int, window: int, pages_per_split: int, split: int):
    """Logical pages ``[first, end)`` that split ``split`` of a decode row covers.

    The row's keys live on logical pages ``p0 .. ceil(L/ps)-1`` where ``p0``
    is the page of its first allowed key (0 without a window); splits take
    ``pages_per_split`` consecutive pages each, starting at ``p0``.
    """
    L = int(seq_len)
    if L <= 0:
        return 0, 0
    first_key = 0 if window <= 0 else max(0, L - window)
    p0 = first_key // page_size
    pend = -(-L // page_size)
    a = min(pend, p0 + split * pages_per_split)
    b = min(pend, a + pages_per_split) if a < pend else a
    return a, b


def decode_partials(q, k_pool, v_pool, block_tables, seq_lens, page_size, scale, window,
                    pages_per_split, num_splits):
    """Per-split partial state of each decode row.

    For split ``s`` with allowed keys ``I_s`` (the keys of its pages that
    the row may attend) and scores ``x_i = scale * k_i . q``:
    ``m2 = log2(e) * max x_i``, ``l = sum exp(x_i - max)`` and
    ``acc = sum exp(x_i - max) v_i`` (not normalised).  An empty split has
    ``m2 = -inf``, ``l = 0``, ``acc = 0``.
    Returns ``m2, l [B, Hq, S]`` and ``acc [B, Hq, S, D]``.
    """
    qf = bf16_to_f64(q)
    B, Hq, D = qf.shape
    Hkv = k_pool.shape[0]
    g = Hq // Hkv
    S = int(num_splits)
    m2 = np.full((B, Hq, S), -np.inf)
    l = np.zeros((B, Hq, S))
    acc = np.zeros((B, Hq, S, D))
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        K = gather(k_pool, block_tables[b], L, page_size)
        V = gather(v_pool, block_tables[b], L, page_size)
        allowed = set(allowed_keys(L - 1, window).tolist())
        for s in range(S):
            a, e = split_page_range(L, page_size, window, pages_per_split, s)
            keys = [i for i in range(a * page_size, min(L, e * page_size)) if i in allowed]
            if not keys:
                continue
            keys = np.asarray(keys)
            for h in range(Hq):
                x = (K[h // g, keys, :] @ qf[b, h, :]) * scale
                mx = x.max()
                w = np.exp(x - mx)
                m2[b, h, s] = mx * LOG2E
                l[b, h, s] = w.sum()
                acc[b, h, s, :] = w @ V[h // g, keys, :]
    return m2, l, acc


def combine_partials(m2, l, acc) -> np.ndarray:
    """Merge split partials: with ``M = max_s m2_s`` (log2 units),
    ``out = sum_s 2^(m2_s - M) acc_s / sum_s 2^(m2_s - M) l_s``; rows whose
    splits are all empty give zeros."""
    m2 = np.asarray(m2, dtype=np.float64)
    B, Hq, S = m2.shape
    out = np.zeros(acc.shape[:2] + acc.shape[3:], dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            M = m2[b, h].max()
            if not np.isfinite(M):
                continue
            w = np.exp2(m2[b, h] - M)
            out[b, h] = (w @ acc[b, h]) / (w @ l[b, h])
    return out
