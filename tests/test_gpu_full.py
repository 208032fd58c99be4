"""Every row of the three full-size workloads against the oracle.

* The 256-sequence decode (context U[1024, 8192], 32/8/128, page 32): the
  step's append fused into the decode launch (what the benchmark runs), the
  same decode after a separate append, and split-K with combine.  Every
  sequence's pool pages are compared bit for bit with the oracle's, every
  pool row no sequence owns must still hold its poison, and all 256 x 32
  output rows are compared with the oracle.
* The 16-prompt long prefill (U[1024, 4096] rows each, 32/8/128): every
  sequence's pages bit for bit, and every one of its ~42 000 query rows
  against the oracle's attention over the keys it gathers from its pool.
* The 8-prompt head_dim-512 prefill (U[1024, 4096], 8/1/512), the same
  way: the launch the full512_prefill benchmark times (grouped dense grid).

The parity bar (max-abs 2e-2, mean-abs 2e-3) applies to all elements of a
workload.  Oracle work runs in host threads, one BLAS thread each."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from gpu_harness import (GpuPools, compact_oracle_pools, dev_bits, dev_i32, err_stats,  # noqa: E402
                         host_bits, page_rows, say, summarize, thread_map)


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import paged_kv_attention_mapped_amd as P
    P.lib()
    return P


def _poison_outside(wl, g):
    """Every pool row that no sequence owns (positions >= its length, unused pages) is poison."""
    written = (g.k != int(W.BF16_NAN)).any(dim=-1).cpu().numpy()    # [Hkv, slots]
    written |= (g.v != int(W.BF16_NAN)).any(dim=-1).cpu().numpy()
    cu = wl.cu_lens(wl.total_lens)
    used = np.zeros(wl.num_slots, bool)
    used[oracle.slot_mapping(wl.block_tables, cu, cu, wl.page_size)] = True
    assert np.array_equal(written, np.broadcast_to(used, written.shape))


def test_large_decode_every_row(P):
    wl = W.make("large_decode")
    B, ps = wl.n_decode, wl.page_size
    say(f"[full] large_decode: {B} seqs, {int(wl.total_lens.sum())} tokens, {wl.num_pages} pages")
    g = GpuPools(wl)
    kept = []
    g.write("prefix", chunk=32, keep_new=kept)
    kn = np.concatenate([k for k, _, _, _ in kept])
    vn = np.concatenate([v for _, v, _, _ in kept])
    assert kn.shape == (B, wl.num_kv_heads, wl.head_dim)
    qd, _ = wl.queries(0)
    lens = wl.decode_seq_lens()
    maxlen = int(lens.max())
    d_q, d_bt, d_lens = dev_bits(qd), dev_i32(wl.block_tables), dev_i32(lens)
    say("[full] large_decode: fused append + decode (automatic decomposition)")
    out_f = P.decode_append(d_q, dev_bits(kn), dev_bits(vn), g.k, g.v, d_bt, d_lens, maxlen,
                            page_size=ps, scale=wl.scale)
    torch.cuda.synchronize()
    say("[full] large_decode: decode after the append, and split-K + combine")
    out_d = P.decode(d_q, g.k, g.v, d_bt, d_lens, maxlen, page_size=ps, scale=wl.scale)
    S, _ = P.decode_plan(B, wl.num_kv_heads, ps, maxlen, 0)
    out_s = P.decode(d_q, g.k, g.v, d_bt, d_lens, maxlen, page_size=ps, scale=wl.scale,
                     num_splits=S)
    torch.cuda.synchronize()
    got_f, got_d, got_s = host_bits(out_f), host_bits(out_d), host_bits(out_s)
    # reading the new row from k_new instead of the pool changes no bit
    assert np.array_equal(got_f, got_d)
    _poison_outside(wl, g)
    hk, hv = host_bits(g.k), host_bits(g.v)

    def check(seqs):
        k, v, bt, phys = compact_oracle_pools(wl, seqs)
        rows = page_rows(phys, ps)
        same = np.array_equal(hk[:, rows], k) and np.array_equal(hv[:, rows], v)
        ref = oracle.decode(qd[seqs], k, v, bt, lens[seqs], ps, wl.scale)
        return same, err_stats(got_f[seqs], ref), err_stats(got_s[seqs], ref)

    chunks = [np.arange(i, min(B, i + 16)) for i in range(0, B, 16)]
    say(f"[full] large_decode: oracle pools and decode of all {B} sequences")
    res = thread_map(check, chunks)
    bad = [int(c[0]) for c, r in zip(chunks, res) if not r[0]]
    assert not bad, f"pool pages differ from the oracle's in the chunks starting at {bad}"
    summarize([r[1] for r in res], "large_decode every row, fused append + stream-K")
    summarize([r[2] for r in res], f"large_decode every row, split-K {S} splits")


def test_long_prefill_every_row(P):
    wl = W.make("long_prefill")
    ps = wl.page_size
    say(f"[full] long_prefill: {wl.n_prefill} prompts, {wl.total_q()} rows")
    g = GpuPools(wl)
    g.write("prefix", chunk=16)
    g.write("new", chunk=16)
    _, qp = wl.queries(0)
    seqs = wl.prefill_ids()
    cq, ck = wl.prefill_cu_q(), wl.prefill_cu_k()
    out = P.prefill_varlen(dev_bits(qp), g.k, g.v, dev_i32(wl.block_tables[seqs]), dev_i32(cq),
                           dev_i32(ck), int(wl.new_lens[seqs].max()),
                           int(wl.total_lens[seqs].max()), page_size=ps, scale=wl.scale)
    torch.cuda.synchronize()
    got = host_bits(out)
    _poison_outside(wl, g)
    hk, hv = host_bits(g.k), host_bits(g.v)

    def check(j):
        s = int(seqs[j])
        k, v, bt, phys = compact_oracle_pools(wl, [s])
        rows = page_rows(phys, ps)
        same = np.array_equal(hk[:, rows], k) and np.array_equal(hv[:, rows], v)
        Lq, Lk = int(wl.new_lens[s]), int(wl.total_lens[s])
        K = oracle.gather(k, bt[0], Lk, ps)
        V = oracle.gather(v, bt[0], Lk, ps)
        ref = oracle.attend_rows_matrix(oracle.bf16_to_f64(qp[cq[j]:cq[j + 1]]), K, V,
                                        np.arange(Lk - Lq, Lk), wl.scale, 0)
        return same, err_stats(got[cq[j]:cq[j + 1]], ref)

    say("[full] long_prefill: oracle attention of every row")
    res = thread_map(check, range(wl.n_prefill))
    bad = [j for j, r in enumerate(res) if not r[0]]
    assert not bad, f"pool pages differ from the oracle's for prompts {bad}"
    summarize([r[1] for r in res], "long_prefill every row")



def test_full512_prefill_every_row(P):
    wl = W.make("full512_prefill")
    ps = wl.page_size
    say(f"[full] full512_prefill: {wl.n_prefill} prompts, {wl.total_q()} rows")
    g = GpuPools(wl)
    g.write("prefix", chunk=16)
    g.write("new", chunk=16)
    _, qp = wl.queries(0)
    seqs = wl.prefill_ids()
    cq, ck = wl.prefill_cu_q(), wl.prefill_cu_k()
    out = P.prefill_varlen(dev_bits(qp), g.k, g.v, dev_i32(wl.block_tables[seqs]), dev_i32(cq),
                           dev_i32(ck), int(wl.new_lens[seqs].max()),
                           int(wl.total_lens[seqs].max()), page_size=ps, scale=wl.scale)
    torch.cuda.synchronize()
    got = host_bits(out)
    _poison_outside(wl, g)
    hk, hv = host_bits(g.k), host_bits(g.v)

    def check(j):
        s = int(seqs[j])
        k, v, bt, phys = compact_oracle_pools(wl, [s])
        rows = page_rows(phys, ps)
        same = np.array_equal(hk[:, rows], k) and np.array_equal(hv[:, rows], v)
        Lq, Lk = int(wl.new_lens[s]), int(wl.total_lens[s])
        K = oracle.gather(k, bt[0], Lk, ps)
        V = oracle.gather(v, bt[0], Lk, ps)
        ref = oracle.attend_rows_matrix(oracle.bf16_to_f64(qp[cq[j]:cq[j + 1]]), K, V,
                                        np.arange(Lk - Lq, Lk), wl.scale, 0)
        return same, err_stats(got[cq[j]:cq[j + 1]], ref)

    say("[full] full512_prefill: oracle attention of every row")
    res = thread_map(check, range(wl.n_prefill))
    bad = [j for j, r in enumerate(res) if not r[0]]
    assert not bad, f"pool pages differ from the oracle's for prompts {bad}"
    summarize([r[1] for r in res], "full512_prefill every row")
