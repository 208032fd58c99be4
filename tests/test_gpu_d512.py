"""head_dim 512 (the full-attention layers of the dual-regime model) against
the oracle: append bit-exact, decode (the automatic workgroup-level
stream-K with any workgroup count, explicit splits + combine, one split,
decode rows through the varlen entry), varlen prefill with
fresh prompts, chunks after a cached prefix and mixed batches, for groups 1,
2, 3, 4 and 8, pages 16 and 32, with and without a window; prompts long
enough for the grouped dense grid of the prefill launch."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from gpu_harness import (GpuPools, OraclePools, check_close, dev_bits, dev_i32,  # noqa: E402
                         host_bits, say)

SHAPES = [  # name, Hq, Hkv, page, window
    ("g8_p32", 8, 1, 32, 0),
    ("g4_p16_win", 8, 2, 16, 300),
    ("g3_p32", 3, 1, 32, 0),
    ("g1_p16", 2, 2, 16, 0),
    ("g2_p32", 4, 2, 32, 0),
]


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import paged_kv_attention_mapped_amd as P
    P.lib()
    return P


def build(name, hq, hkv, ps, win, **kw):
    cfg = W.Config("d512_" + name, 20261205, hq, hkv, 512, ps, window=win, **kw)
    wl = W.build(cfg)
    g = GpuPools(wl)
    g.write("prefix")
    g.write("new")
    return wl, g, OraclePools(wl)


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_d512_decode(P, shape):
    name, hq, hkv, ps, win = shape
    wl, g, o = build(name, hq, hkv, ps, win,
                     decode_ctx=("fixed", (1, 15, 16, 17, 33, 64, 300, 777, 1500)))
    assert np.array_equal(host_bits(g.k), o.k) and np.array_equal(host_bits(g.v), o.v)
    qd, _ = wl.queries(0)
    lens = wl.decode_seq_lens()
    bt = dev_i32(wl.block_tables[:wl.n_decode])
    ref = oracle.decode(qd, o.k, o.v, wl.block_tables[:wl.n_decode], lens, ps, wl.scale, win)
    assert P.decode_method(wl.n_decode, hq, hkv, 512, ps, int(lens.max()), win)[0] == "stream"
    for splits in (0, 1, 3):
        say(f"[d512 decode] {name} num_splits={splits}")
        out = P.decode(dev_bits(qd), g.k, g.v, bt, dev_i32(lens), int(lens.max()), page_size=ps,
                       scale=wl.scale, window=win, num_splits=splits)
        torch.cuda.synchronize()
        check_close(host_bits(out), ref, f"d512 {name} decode, splits {splits}")
    # the same rows as one-row sequences of a varlen batch
    one = np.ones(wl.n_decode, np.int32)
    out = P.prefill_varlen(dev_bits(qd), g.k, g.v, bt, dev_i32(wl.cu_lens(one)),
                           dev_i32(wl.cu_lens(lens)), 1, int(lens.max()), page_size=ps,
                           scale=wl.scale, window=win)
    torch.cuda.synchronize()
    check_close(host_bits(out), ref, f"d512 {name} decode rows through the varlen entry")


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_d512_prefill(P, shape):
    name, hq, hkv, ps, win = shape
    wl, g, o = build(name, hq, hkv, ps, win, decode_ctx=("fixed", (40, 500)),
                     prefill_new=("fixed", (1, 31, 33, 64, 0, 130)),
                     chunk=("uniform", 2, 100, 700, 50))
    qd, qp = wl.queries(0)
    seqs = wl.prefill_ids()
    say(f"[d512 prefill] {name}: N={len(seqs)} Tq={qp.shape[0]}")
    out = P.prefill_varlen(dev_bits(qp), g.k, g.v, dev_i32(wl.block_tables[seqs]),
                           dev_i32(wl.prefill_cu_q()), dev_i32(wl.prefill_cu_k()),
                           int(wl.new_lens[seqs].max()), int(wl.total_lens[seqs].max()),
                           page_size=ps, scale=wl.scale, window=win)
    torch.cuda.synchronize()
    ref = oracle.prefill_varlen(qp, o.k, o.v, wl.block_tables[seqs], wl.prefill_cu_q(),
                                wl.prefill_cu_k(), ps, wl.scale, win)
    check_close(host_bits(out), ref, f"d512 {name} prefill")
    # decoders and prompts in one launch
    q = np.concatenate([qd, qp])
    cq, ck = wl.cu_lens(wl.new_lens), wl.cu_lens(wl.total_lens)
    out = P.prefill_varlen(dev_bits(q), g.k, g.v, dev_i32(wl.block_tables), dev_i32(cq),
                           dev_i32(ck), int(wl.new_lens.max()), int(wl.total_lens.max()),
                           page_size=ps, scale=wl.scale, window=win)
    torch.cuda.synchronize()
    ref = oracle.prefill_varlen(q, o.k, o.v, wl.block_tables, cq, ck, ps, wl.scale, win)
    check_close(host_bits(out), ref, f"d512 {name} mixed single launch")


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_d512_stream_any_partition(P, shape):
    """The workgroup-level stream-K at head_dim 512 with many workgroup
    counts, so that ranges are cut inside rows, at row and KV-head
    boundaries and across several workgroups; an empty row and page-edge
    lengths; each count run twice, bit-identical."""
    name, hq, hkv, ps, win = shape
    wl, g, o = build(name, hq, hkv, ps, win,
                     decode_ctx=("fixed", (0, 31, 32, 33, 95, 300, 1, 1200, 64)))
    qd, _ = wl.queries(0)
    lens = wl.decode_seq_lens().copy()
    lens[0] = 0                                       # an empty row
    bt = dev_i32(wl.block_tables[:wl.n_decode])
    ref = oracle.decode(qd, o.k, o.v, wl.block_tables[:wl.n_decode], lens, ps, wl.scale, win)
    auto = P.decode_stream_waves(wl.n_decode, hq, hkv, 512, ps, int(lens.max()), win)
    for nw in sorted({1, 2, 3, 5, 13, 64, auto}):
        say(f"[d512 stream] {name} workgroups={nw}")
        outs = []
        for _ in range(2):
            out, ws = P.decode_stream(dev_bits(qd), g.k, g.v, bt, dev_i32(lens), page_size=ps,
                                      num_waves=nw, scale=wl.scale, window=win)
            P.decode_stream_merge(ws, out, num_waves=nw, num_kv_heads=hkv)
            torch.cuda.synchronize()
            outs.append(host_bits(out))
        assert np.array_equal(outs[0], outs[1]), "stream-K decode is not deterministic"
        check_close(outs[0], ref, f"d512 {name} stream, {nw} workgroups")
        assert np.all(outs[0][0] == 0)                # the empty row


DENSE = [  # name, Hq, Hkv, page, window: four, two and one head per workgroup
    ("g8_p32", 8, 1, 32, 0),
    ("g4_p16_win", 8, 2, 16, 300),
    ("g2_p32", 4, 2, 32, 0),
    ("g3_p16", 3, 1, 16, 0),
]


@pytest.mark.parametrize("shape", DENSE, ids=[s[0] for s in DENSE])
def test_d512_prefill_grouped_grid(P, shape):
    """Prompts of 520-1030 rows and 600-row chunks after a cached prefix: at
    least 16 query blocks, so the launch takes the grouped dense grid (the
    shorter cases above walk the compact work list); every row against the
    oracle, rows of short and long sequences in one launch."""
    name, hq, hkv, ps, win = shape
    wl, g, o = build(name, hq, hkv, ps, win, decode_ctx=("fixed", (40,)),
                     prefill_new=("fixed", (520, 1030, 777)),
                     chunk=("uniform", 2, 300, 900, 600))
    qd, qp = wl.queries(0)
    seqs = wl.prefill_ids()
    say(f"[d512 grouped grid] {name}: N={len(seqs)} Tq={qp.shape[0]} max_q={int(wl.new_lens[seqs].max())}")
    assert int(wl.new_lens[seqs].max()) >= 16 * 32
    out = P.prefill_varlen(dev_bits(qp), g.k, g.v, dev_i32(wl.block_tables[seqs]),
                           dev_i32(wl.prefill_cu_q()), dev_i32(wl.prefill_cu_k()),
                           int(wl.new_lens[seqs].max()), int(wl.total_lens[seqs].max()),
                           page_size=ps, scale=wl.scale, window=win)
    torch.cuda.synchronize()
    ref = oracle.prefill_varlen(qp, o.k, o.v, wl.block_tables[seqs], wl.prefill_cu_q(),
                                wl.prefill_cu_k(), ps, wl.scale, win)
    check_close(host_bits(out), ref, f"d512 {name} grouped-grid prefill")


def test_d512_prefill_stays_inside_total_q(P):
    """cu_seq_lens_q running past total_q (a caller error) at head_dim 512:
    q rows past total_q (NaN) are never read, out rows past it keep their
    canaries, and the sequences before the bad one match the oracle.  A
    mixed batch, so both launches (prompts, one-row sequences) see it."""
    canary = 0x5A5A
    wl, g, o = build("g8_p32", 8, 1, 32, 0, decode_ctx=("fixed", (40, 500, 77)),
                     prefill_new=("fixed", (33, 130)), chunk=("uniform", 1, 100, 300, 60))
    qd, qp = wl.queries(0)
    q = np.concatenate([qd, qp])
    cq, ck = wl.cu_lens(wl.new_lens).copy(), wl.cu_lens(wl.total_lens)
    T = int(cq[-1])
    bad = cq.copy()
    bad[-1] += 40                       # the last sequence claims 40 rows past total_q
    q_full = torch.full((T + 64, wl.num_q_heads, 512), int(W.BF16_NAN), dtype=torch.int16,
                        device="cuda")
    q_full[:T] = dev_bits(q)
    out_full = torch.full((T + 64, wl.num_q_heads, 512), canary, dtype=torch.int16, device="cuda")
    say(f"[d512 canary] prefill past total_q: T={T}")
    P.prefill_varlen(q_full[:T], g.k, g.v, dev_i32(wl.block_tables), dev_i32(bad), dev_i32(ck),
                     int(wl.new_lens.max()) + 40, int(wl.total_lens.max()), page_size=32,
                     scale=wl.scale, out=out_full[:T])
    torch.cuda.synchronize()
    assert torch.all(out_full[T:] == canary)
    got = host_bits(out_full[:T])
    assert np.all(np.isfinite(W.bf16_to_f32(got)))
    n = wl.num_seqs - 1
    ref = oracle.prefill_varlen(q[:cq[n]], o.k, o.v, wl.block_tables[:n], cq[:n + 1], ck[:n + 1],
                                32, wl.scale, 0)
    check_close(got[:cq[n]], ref, "d512 rows before the bad sequence")
