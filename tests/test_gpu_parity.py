"""Parity of the HIP path with the CPU oracle, through the C ABI, on the
seeded workloads.  Append and addressing must be bit-exact; attention must be
within max-abs 2e-2 and mean-abs 2e-3 of the float64 oracle."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from gpu_harness import (GpuPools, OraclePools, check_close, dev_bits, dev_i32,  # noqa: E402
                         host_bits, say)

SMALL = ["tiny_decode", "qwen3_decode", "mixed_step", "window_shared"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import paged_kv_attention_mapped_amd as P
    P.lib()  # raises if the library was not built


@pytest.fixture(scope="module")
def P():
    import paged_kv_attention_mapped_amd as P
    return P


_states = {}


def state(name):
    """GPU pools (prefix + this step's tokens appended through the HIP path)."""
    if name not in _states:
        wl = W.make(name)
        say(f"[setup] {name}: seqs={wl.num_seqs} pages={wl.num_pages} tokens={int(wl.total_lens.sum())}")
        g = GpuPools(wl)
        g.write("prefix")
        g.write("new")
        _states[name] = g
    return _states[name]


def run_decode(P, g, q_bits, seqs=None, **kw):
    wl = g.wl
    seqs = wl.decode_ids() if seqs is None else seqs
    lens = wl.total_lens[seqs].astype(np.int32)
    out = P.decode(dev_bits(q_bits), g.k, g.v, dev_i32(wl.block_tables[seqs]), dev_i32(lens),
                   int(lens.max()), page_size=wl.page_size, scale=wl.scale, window=wl.window, **kw)
    torch.cuda.synchronize()
    return host_bits(out)


def run_prefill(P, g, q_bits, seqs=None):
    wl = g.wl
    seqs = wl.prefill_ids() if seqs is None else np.asarray(seqs)
    lq = wl.new_lens[seqs]
    lk = wl.total_lens[seqs]
    out = P.prefill_varlen(dev_bits(q_bits), g.k, g.v, dev_i32(wl.block_tables[seqs]),
                           dev_i32(wl.cu_lens(lq)), dev_i32(wl.cu_lens(lk)), int(lq.max()),
                           int(lk.max()), page_size=wl.page_size, scale=wl.scale,
                           window=wl.window)
    torch.cuda.synchronize()
    return host_bits(out)


# ---------------------------------------------------------------------------
# addressing and append: bit-exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", SMALL + ["large_decode", "long_prefill"])
def test_slot_mapping_bit_exact(P, name):
    wl = W.make(name)
    say(f"[slot_mapping] {name}")
    for part in ("prefix", "new"):
        lq = wl.new_lens if part == "new" else wl.prefix_lens
        lk = wl.total_lens if part == "new" else wl.prefix_lens
        cq, ck = wl.cu_lens(lq), wl.cu_lens(lk)
        got = P.slot_mapping(dev_i32(wl.block_tables), dev_i32(cq), dev_i32(ck),
                             page_size=wl.page_size, num_pages=wl.num_pages,
                             total_tokens=int(cq[-1]))
        ref = oracle.slot_mapping(wl.block_tables, cq, ck, wl.page_size)
        assert np.array_equal(got.cpu().numpy().astype(np.int64), ref)


@pytest.mark.parametrize("name", SMALL)
def test_append_whole_pool_bit_exact(name):
    g = state(name)
    say(f"[append] {name}")
    o = OraclePools(g.wl)
    assert np.array_equal(host_bits(g.k), o.k)
    assert np.array_equal(host_bits(g.v), o.v)


@pytest.mark.parametrize("name", SMALL)
def test_append_mapped_bit_exact(P, name):
    """The fused addressing + append writes the oracle's pools and slots."""
    wl = W.make(name)
    say(f"[append_mapped] {name}")
    g = GpuPools(wl)
    log = []
    g.write("prefix", fused=True, slots_log=log)
    g.write("new", fused=True, slots_log=log, chunk=3)
    o = OraclePools(wl)
    assert np.array_equal(host_bits(g.k), o.k)
    assert np.array_equal(host_bits(g.v), o.v)
    for sub, cq, ck, got in log:
        ref = oracle.slot_mapping(wl.block_tables[sub], cq, ck, wl.page_size)
        assert np.array_equal(got.cpu().numpy().astype(np.int64), ref)


def test_append_mapped_edge_cases(P):
    """Sequences with no new tokens, unmapped table entries (-1, past the pool)
    and positions past the table: those tokens get slot -1 and leave the pool
    untouched; empty steps enqueue nothing."""
    hkv, d, ps, npg = 2, 64, 16, 6
    rng = np.random.default_rng(5)
    bt = np.array([[3, -1, 0], [5, 1, 9], [2, 4, 0], [0, 0, 0]], np.int32)
    lq = np.array([20, 20, 5, 0], np.int32)    # seq 3: no new tokens
    lk = np.array([20, 40, 60, 5], np.int32)   # seq 2 runs past its 3-page table
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    T = int(cq[-1])
    kn = rng.integers(0, 1 << 16, (T, hkv, d), dtype=np.uint16)
    vn = rng.integers(0, 1 << 16, (T, hkv, d), dtype=np.uint16)
    # expected slots: the oracle's address over a table padded with -1, and
    # -1 wherever the physical page is not in [0, npg)
    bt_pad = np.concatenate([bt, np.full((4, 1), -1, np.int32)], axis=1)
    slots = oracle.slot_mapping(bt_pad, cq, ck, ps)
    slots = np.where((slots >= 0) & (slots < npg * ps), slots, -1)
    assert (slots >= 0).sum() == 16 + 12      # seq 0 page 0, seq 1 page 1
    pool0 = np.full((hkv, npg * ps, d), W.BF16_NAN, np.uint16)
    ok, ov = oracle.append(pool0, pool0, kn, vn, slots)
    gk, gv = dev_bits(pool0), dev_bits(pool0)
    out = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    P.append_mapped(dev_bits(kn), dev_bits(vn), dev_i32(bt), dev_i32(cq), dev_i32(ck), gk, gv,
                    page_size=ps, max_seqlen_q=20, slot_mapping_out=out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.int64), slots)
    assert np.array_equal(host_bits(gk), ok) and np.array_equal(host_bits(gv), ov)
    # a host bound below a sequence's row count: only its first rows are written
    rows = np.concatenate([np.arange(n) < 7 for n in lq])
    k7, v7 = oracle.append(pool0, pool0, kn, vn, np.where(rows, slots, -1))
    hk, hv = dev_bits(pool0), dev_bits(pool0)
    out.fill_(-7)
    P.append_mapped(dev_bits(kn), dev_bits(vn), dev_i32(bt), dev_i32(cq), dev_i32(ck), hk, hv,
                    page_size=ps, max_seqlen_q=7, slot_mapping_out=out)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(hk), k7) and np.array_equal(host_bits(hv), v7)
    assert np.array_equal(out.cpu().numpy()[rows].astype(np.int64), slots[rows])
    assert np.all(out.cpu().numpy()[~rows] == -7)
    # zero new tokens, and zero sequences: nothing is enqueued
    P.append_mapped(dev_bits(kn[:0]), dev_bits(vn[:0]), dev_i32(bt), dev_i32(cq * 0),
                    dev_i32(ck), gk, gv, page_size=ps)
    P.append_mapped(dev_bits(kn[:0]), dev_bits(vn[:0]), dev_i32(bt[:0]), dev_i32(cq[:1]),
                    dev_i32(ck[:1]), gk, gv, page_size=ps)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(gk), ok) and np.array_equal(host_bits(gv), ov)


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny_decode", "qwen3_decode", "mixed_step", "window_shared"])
def test_decode_parity(P, name):
    g = state(name)
    wl = g.wl
    o = OraclePools(wl)
    for layer in range(wl.num_layers):
        qd, _ = wl.queries(layer)
        say(f"[decode] {name} layer {layer}: B={wl.n_decode}")
        got = run_decode(P, g, qd)
        ref = oracle.decode(qd, o.k, o.v, wl.block_tables[:wl.n_decode], wl.decode_seq_lens(),
                            wl.page_size, wl.scale, wl.window)
        check_close(got, ref, f"{name} L{layer} decode")


@pytest.mark.parametrize("splits", [1, 2, 7, 0])
def test_split_count_invariance_and_determinism(P, splits):
    g = state("qwen3_decode")
    wl = g.wl
    qd, _ = wl.queries(0)
    say(f"[decode] qwen3_decode num_splits={splits}")
    a = run_decode(P, g, qd, num_splits=splits)
    b = run_decode(P, g, qd, num_splits=splits)
    assert np.array_equal(a, b), "decode is not deterministic"
    o = OraclePools(wl)
    ref = oracle.decode(qd, o.k, o.v, wl.block_tables, wl.decode_seq_lens(), wl.page_size, wl.scale)
    check_close(a, ref, f"splits={splits}")


@pytest.mark.parametrize("name", ["tiny_decode", "qwen3_decode", "window_shared", "edges"])
def test_stream_decode_any_partition(P, name):
    """Stream-K with many wave counts: every cut of the flattened page list
    must give the oracle's result, deterministically."""
    if name == "edges":
        wl = W.make("qwen3_decode", decode_ctx=("fixed", (0, 31, 32, 63, 64, 1023, 5)),
                    name="edges")
        g = GpuPools(wl)
        g.write("prefix")
        g.write("new")
    else:
        g = state(name)
        wl = g.wl
    o = OraclePools(wl)
    lens = wl.decode_seq_lens().copy()
    if name == "edges":
        lens[0] = 0  # an empty row
    auto = P.decode_stream_waves(wl.n_decode, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.page_size,
                                 int(lens.max()), wl.window)
    for layer in range(wl.num_layers):
        qd, _ = wl.queries(layer)
        ref = oracle.decode(qd, o.k, o.v, wl.block_tables[:wl.n_decode], lens, wl.page_size,
                            wl.scale, wl.window)
        for nw in sorted({1, 2, 3, 7, 64, 1000, auto}):
            say(f"[decode_stream] {name} layer {layer} num_waves={nw}")
            outs = []
            for _ in range(2):
                out, ws = P.decode_stream(dev_bits(qd), g.k, g.v,
                                          dev_i32(wl.block_tables[:wl.n_decode]), dev_i32(lens),
                                          page_size=wl.page_size, num_waves=nw, scale=wl.scale,
                                          window=wl.window)
                P.decode_stream_merge(ws, out, num_waves=nw, num_kv_heads=wl.num_kv_heads)
                torch.cuda.synchronize()
                outs.append(host_bits(out))
            assert np.array_equal(outs[0], outs[1]), "stream-K decode is not deterministic"
            check_close(outs[0], ref, f"{name} nw={nw}")
            if name == "edges":
                assert np.all(outs[0][0] == 0)  # the empty row


# group sizes around the stream-K split of wide groups (6 and 8 split into
# halves at head_dim >= 128; 7 and head_dim 64 do not), pages 16/32, a window
DECODE_SHAPES = [  # name, Hq, Hkv, D, page, window
    ("d128_g6_p16", 12, 2, 128, 16, 0),
    ("d128_g8_p32", 16, 2, 128, 32, 0),
    ("d128_g7_p32", 7, 1, 128, 32, 0),
    ("d64_g8_p16", 8, 1, 64, 16, 0),
    ("d256_g6_p32_win", 6, 1, 256, 32, 200),
    ("d256_g8_p16_kv2", 16, 2, 256, 16, 0),   # whole-group one-row workgroups, two KV heads
]


@pytest.mark.parametrize("shape", DECODE_SHAPES, ids=[s[0] for s in DECODE_SHAPES])
def test_decode_shapes(P, shape):
    name, hq, hkv, d, ps, win = shape
    cfg = W.Config(name, 20261203, hq, hkv, d, ps, window=win,
                   decode_ctx=("fixed", (1, 15, 16, 17, 33, 64, 300, 777, 1500)))
    wl = W.build(cfg)
    g = GpuPools(wl)
    g.write("prefix")
    g.write("new")
    o = OraclePools(wl)
    qd, _ = wl.queries(0)
    lens = wl.decode_seq_lens()
    ref = oracle.decode(qd, o.k, o.v, wl.block_tables[:wl.n_decode], lens, wl.page_size,
                        wl.scale, wl.window)
    say(f"[decode] {name}: automatic decomposition and 5 waves")
    got = run_decode(P, g, qd)
    check_close(got, ref, f"{name} decode")
    out, ws = P.decode_stream(dev_bits(qd), g.k, g.v, dev_i32(wl.block_tables[:wl.n_decode]),
                              dev_i32(lens), page_size=wl.page_size, num_waves=5, scale=wl.scale,
                              window=wl.window)
    P.decode_stream_merge(ws, out, num_waves=5, num_kv_heads=wl.num_kv_heads)
    torch.cuda.synchronize()
    check_close(host_bits(out), ref, f"{name} decode, 5 waves")
    # the same rows as one-row sequences of a varlen batch (single-row path)
    lq = np.ones(wl.n_decode, np.int32)
    out = P.prefill_varlen(dev_bits(qd), g.k, g.v, dev_i32(wl.block_tables[:wl.n_decode]),
                           dev_i32(wl.cu_lens(lq)), dev_i32(wl.cu_lens(lens)), 1, int(lens.max()),
                           page_size=wl.page_size, scale=wl.scale, window=wl.window)
    torch.cuda.synchronize()
    check_close(host_bits(out), ref, f"{name} decode rows through the varlen entry")
    # ... and cut into page runs by the split entry (partials merged)
    out = P.prefill_varlen_split(dev_bits(qd), g.k, g.v, dev_i32(wl.block_tables[:wl.n_decode]),
                                 dev_i32(wl.cu_lens(lq)), dev_i32(wl.cu_lens(lens)), 1,
                                 int(lens.max()), page_size=wl.page_size, num_splits=3,
                                 scale=wl.scale, window=wl.window)
    torch.cuda.synchronize()
    check_close(host_bits(out), ref, f"{name} decode rows through the split varlen entry")


@pytest.mark.parametrize("name", ["mixed_step", "window_shared"])
def test_mixed_single_launch(P, name):
    """Decode rows (one row each) and prompts/chunks in one varlen launch."""
    g = state(name)
    wl = g.wl
    o = OraclePools(wl)
    cq, ck = wl.cu_lens(wl.new_lens), wl.cu_lens(wl.total_lens)
    for layer in range(wl.num_layers):
        qd, qp = wl.queries(layer)
        q = np.concatenate([qd, qp])   # sequence order: decoders, then prefill sequences
        say(f"[mixed] {name} layer {layer}: {wl.n_decode} decode rows + {qp.shape[0]} prefill rows")
        out = P.prefill_varlen(dev_bits(q), g.k, g.v, dev_i32(wl.block_tables), dev_i32(cq),
                               dev_i32(ck), int(wl.new_lens.max()), int(wl.total_lens.max()),
                               page_size=wl.page_size, scale=wl.scale, window=wl.window)
        torch.cuda.synchronize()
        got = host_bits(out)
        ref = oracle.prefill_varlen(q, o.k, o.v, wl.block_tables, cq, ck, wl.page_size, wl.scale,
                                    wl.window)
        check_close(got, ref, f"{name} L{layer} single launch")
        # the decode rows agree with the decode entry's result within the same bar
        refd = oracle.decode(qd, o.k, o.v, wl.block_tables[:wl.n_decode], wl.decode_seq_lens(),
                             wl.page_size, wl.scale, wl.window)
        check_close(got[:wl.n_decode], refd, f"{name} L{layer} decode rows")


@pytest.mark.parametrize("name", ["mixed_step", "window_shared"])
@pytest.mark.parametrize("splits", [2, 4, 7])
def test_prefill_split_parity(P, name, splits):
    """pkv_prefill_varlen_split (each workgroup's keys in `splits` runs of
    tiles, partials merged by the split-K combine) on a mixed batch: within
    the bar of the oracle, and bit-identical on a second call."""
    g = state(name)
    wl = g.wl
    o = OraclePools(wl)
    cq, ck = wl.cu_lens(wl.new_lens), wl.cu_lens(wl.total_lens)
    for layer in range(wl.num_layers):
        qd, qp = wl.queries(layer)
        q = np.concatenate([qd, qp])
        say(f"[split prefill] {name} layer {layer}: {splits} splits")
        args = (dev_bits(q), g.k, g.v, dev_i32(wl.block_tables), dev_i32(cq), dev_i32(ck),
                int(wl.new_lens.max()), int(wl.total_lens.max()))
        kw = dict(page_size=wl.page_size, num_splits=splits, scale=wl.scale, window=wl.window)
        got = host_bits(P.prefill_varlen_split(*args, **kw))
        again = host_bits(P.prefill_varlen_split(*args, **kw))
        torch.cuda.synchronize()
        ref = oracle.prefill_varlen(q, o.k, o.v, wl.block_tables, cq, ck, wl.page_size, wl.scale,
                                    wl.window)
        check_close(got, ref, f"{name} L{layer} {splits} splits")
        assert np.array_equal(got, again)


@pytest.mark.parametrize("shape", [(8, 2, 128, 32, 0, 3), (4, 1, 64, 16, 0, 5), (8, 1, 256, 32, 300, 2)])
def test_prefill_split_many_blocks_every_row(P, shape):
    """Key splits on the batch of test_prefill_many_blocks_every_row (grouped
    query blocks, decode rows, an empty prompt, chunks): every row written
    and within the bar, for three head shapes (one windowed)."""
    hq, hkv, d, ps, window, splits = shape
    cfg = W.Config("many_blocks", 20260101, hq, hkv, d, ps, window=window,
                   decode_ctx=("fixed", (5, 300, 1000)),
                   prefill_new=("fixed", (1100, 1, 64, 65, 0, 700, 1025, 33)),
                   chunk=("uniform", 2, 200, 900, 1000))
    wl = W.build(cfg)
    g = GpuPools(wl)
    g.write("prefix")
    g.write("new")
    o = OraclePools(wl)
    cq, ck = wl.cu_lens(wl.new_lens), wl.cu_lens(wl.total_lens)
    qd, qp = wl.queries(0)
    q = np.concatenate([qd, qp])
    out = torch.full(q.shape, int(W.BF16_NAN), dtype=torch.int16, device="cuda")
    P.prefill_varlen_split(dev_bits(q), g.k, g.v, dev_i32(wl.block_tables), dev_i32(cq), dev_i32(ck),
                           int(wl.new_lens.max()), int(wl.total_lens.max()), page_size=wl.page_size,
                           num_splits=splits, scale=wl.scale, window=wl.window, out=out)
    torch.cuda.synchronize()
    ref = oracle.prefill_varlen(q, o.k, o.v, wl.block_tables, cq, ck, wl.page_size, wl.scale,
                                wl.window)
    check_close(host_bits(out), ref, f"many blocks {shape[:5]}, {splits} splits")


@pytest.mark.parametrize("name", ["qwen3_decode", "window_shared"])
def test_decode_split_partials(P, name):
    g = state(name)
    wl = g.wl
    qd, _ = wl.queries(0)
    lens = wl.decode_seq_lens()
    S, pps = P.decode_plan(wl.n_decode, wl.num_kv_heads, wl.page_size, int(lens.max()), wl.window)
    if S == 1:
        S, pps = P.decode_plan(wl.n_decode, wl.num_kv_heads, wl.page_size, int(lens.max()),
                               wl.window, 3)
    say(f"[decode_split] {name} S={S} pps={pps}")
    m, l, acc = P.decode_split(dev_bits(qd), g.k, g.v, dev_i32(wl.block_tables[:wl.n_decode]),
                               dev_i32(lens), int(lens.max()), page_size=wl.page_size,
                               num_splits=S, pages_per_split=pps, scale=wl.scale,
                               window=wl.window)
    torch.cuda.synchronize()
    m, l, acc = m.cpu().numpy(), l.cpu().numpy(), acc.cpu().numpy()
    o = OraclePools(wl)
    rm, rl, racc = oracle.decode_partials(qd, o.k, o.v, wl.block_tables, lens, wl.page_size,
                                          wl.scale, wl.window, pps, S)
    empty = ~np.isfinite(rm)
    assert np.array_equal(~np.isfinite(m), empty)
    assert np.all(l[empty] == 0) and np.all(acc[empty] == 0)
    ne = ~empty
    assert np.max(np.abs(m[ne] - rm[ne])) < 1e-3
    np.testing.assert_allclose(l[ne], rl[ne], rtol=2e-2)
    check_close_f = np.abs(acc[ne] / l[ne][:, None] - racc[ne] / rl[ne][:, None])
    assert check_close_f.max() < 2e-2 and check_close_f.mean() < 2e-3


def test_combine_from_oracle_partials(P):
    # The combine kernel alone, fed with the oracle's partials.
    wl = W.make("qwen3_decode")
    o = OraclePools(wl)
    qd, _ = wl.queries(0)
    lens = wl.decode_seq_lens()
    rm, rl, racc = oracle.decode_partials(qd, o.k, o.v, wl.block_tables, lens, wl.page_size,
                                          wl.scale, 0, 4, 9)
    say("[combine] qwen3_decode, 9 splits of 4 pages")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()  # noqa: E731
    out = P.decode_combine(t(rm), t(rl), t(racc))
    torch.cuda.synchronize()
    check_close(host_bits(out), oracle.combine_partials(rm, rl, racc), "combine")


def test_decode_page_permutation_bit_identical(P):
    wl = W.make("qwen3_decode")
    g1 = state("qwen3_decode")
    perm = np.random.default_rng(5).permutation(wl.num_pages).astype(np.int32)
    wl2 = W.make("qwen3_decode")
    wl2.block_tables = perm[wl.block_tables]
    say("[decode] page permutation")
    g2 = GpuPools(wl2)
    g2.write("prefix")
    g2.write("new")
    qd, _ = wl.queries(0)
    assert np.array_equal(run_decode(P, g1, qd), run_decode(P, g2, qd))


@pytest.mark.parametrize("name", ["mixed_step", "window_shared"])
def test_prefill_page_permutation_bit_identical(P, name):
    """Moving every page to another physical place (data moved, tables
    rewritten) leaves the single mixed launch (decode rows + prompts or
    chunks) and the split-key prefill bit-identical."""
    wl = W.make(name)
    g1 = state(name)
    perm = np.random.default_rng(6).permutation(wl.num_pages).astype(np.int32)
    wl2 = W.make(name)
    wl2.block_tables = perm[wl.block_tables]
    say(f"[prefill] page permutation: {name}")
    g2 = GpuPools(wl2)
    g2.write("prefix")
    g2.write("new")
    cq, ck = wl.cu_lens(wl.new_lens), wl.cu_lens(wl.total_lens)
    for layer in range(wl.num_layers):
        q = np.concatenate(wl.queries(layer))
        outs = []
        for g, w in ((g1, wl), (g2, wl2)):
            a = (dev_bits(q), g.k, g.v, dev_i32(w.block_tables), dev_i32(cq), dev_i32(ck),
                 int(wl.new_lens.max()), int(wl.total_lens.max()))
            kw = dict(page_size=wl.page_size, scale=wl.scale, window=wl.window)
            one = P.prefill_varlen(*a, **kw)
            split = P.prefill_varlen_split(*a, num_splits=3, **kw)
            torch.cuda.synchronize()
            outs.append((host_bits(one), host_bits(split)))
        assert np.array_equal(outs[0][0], outs[1][0]), f"{name} L{layer} single launch"
        assert np.array_equal(outs[0][1], outs[1][1]), f"{name} L{layer} split-key prefill"


CANARY = 0x5A5A


def test_decode_writes_no_row_past_the_batch(P):
    """Rows of `out` past the batch keep their contents, for every decomposition."""
    g = state("qwen3_decode")
    wl = g.wl
    qd, _ = wl.queries(0)
    lens = wl.decode_seq_lens()
    B = wl.n_decode
    for splits in (0, 1, 3):
        full = torch.full((B + 4, wl.num_q_heads, wl.head_dim), CANARY, dtype=torch.int16,
                          device="cuda")
        say(f"[canary] decode num_splits={splits}")
        P.decode(dev_bits(qd), g.k, g.v, dev_i32(wl.block_tables[:B]), dev_i32(lens),
                 int(lens.max()), page_size=wl.page_size, scale=wl.scale, num_splits=splits,
                 out=full[:B])
        torch.cuda.synchronize()
        assert torch.all(full[B:] == CANARY)
        assert np.all(np.isfinite(W.bf16_to_f32(host_bits(full[:B]))))
    # stream-K with an odd wave count, and its merge
    full = torch.full((B + 4, wl.num_q_heads, wl.head_dim), CANARY, dtype=torch.int16,
                      device="cuda")
    say("[canary] stream-K decode, 37 waves")
    _, ws = P.decode_stream(dev_bits(qd), g.k, g.v, dev_i32(wl.block_tables[:B]), dev_i32(lens),
                            page_size=wl.page_size, num_waves=37, scale=wl.scale, out=full[:B])
    P.decode_stream_merge(ws, full[:B], num_waves=37, num_kv_heads=wl.num_kv_heads)
    torch.cuda.synchronize()
    assert torch.all(full[B:] == CANARY)
    assert np.all(np.isfinite(W.bf16_to_f32(host_bits(full[:B]))))


@pytest.mark.parametrize("splits", [1, 3])
def test_prefill_stays_inside_total_q(P, splits):
    """cu_seq_lens_q running past total_q (a caller error) must not move any
    access out of the buffers: q rows past total_q are never read (they hold
    NaN, and every written row stays finite), out rows and workspace bytes
    past their sizes keep their canaries."""
    g = state("mixed_step")
    wl = g.wl
    cq = wl.cu_lens(wl.new_lens).copy()
    ck = wl.cu_lens(wl.total_lens)
    T = int(cq[-1])
    bad = cq.copy()
    bad[-1] += 40                       # the last sequence claims 40 rows past total_q
    q_full = torch.full((T + 64, wl.num_q_heads, wl.head_dim), int(W.BF16_NAN), dtype=torch.int16,
                        device="cuda")
    q_full[:T] = dev_bits(np.concatenate(wl.queries(0)))
    out_full = torch.full((T + 64, wl.num_q_heads, wl.head_dim), CANARY, dtype=torch.int16,
                          device="cuda")
    nb = P.prefill_split_workspace_bytes(T, wl.num_q_heads, wl.head_dim, splits)
    ws_full = torch.full((nb + 4096,), 0x5A, dtype=torch.uint8, device="cuda")
    say(f"[canary] prefill past total_q, splits={splits}")
    P.prefill_varlen_split(q_full[:T], g.k, g.v, dev_i32(wl.block_tables), dev_i32(bad),
                           dev_i32(ck), int(wl.new_lens.max()) + 40, int(wl.total_lens.max()),
                           page_size=wl.page_size, num_splits=splits, scale=wl.scale,
                           out=out_full[:T], workspace=ws_full[:nb] if nb else None)
    torch.cuda.synchronize()
    assert torch.all(out_full[T:] == CANARY)
    assert torch.all(ws_full[nb:] == 0x5A)
    got = host_bits(out_full[:T])
    assert np.all(np.isfinite(W.bf16_to_f32(got)))
    # the sequences before the last one are unaffected by its bad bound
    o = OraclePools(wl)
    n = wl.num_seqs - 1
    q = np.concatenate(wl.queries(0))
    ref = oracle.prefill_varlen(q[:cq[n]], o.k, o.v, wl.block_tables[:n], cq[:n + 1], ck[:n + 1],
                                wl.page_size, wl.scale)
    check_close(got[:cq[n]], ref, "rows before the bad sequence")


def test_decode_edge_lengths(P):
    # L = 1 returns V exactly; L = 0 gives zeros; page-boundary lengths.
    wl = W.make("qwen3_decode", decode_ctx=("fixed", (0, 31, 32, 63, 64, 1023)), name="edges")
    g = GpuPools(wl)
    g.write("prefix")
    g.write("new")
    qd, _ = wl.queries(0)
    say("[decode] edge lengths 1,32,33,64,65,1024 and an empty row")
    got = run_decode(P, g, qd)
    o = OraclePools(wl)
    ref = oracle.decode(qd, o.k, o.v, wl.block_tables, wl.decode_seq_lens(), wl.page_size, wl.scale)
    check_close(got, ref, "edge lengths")
    k, v = wl.kv_seq(0)
    for h in range(wl.num_q_heads):
        assert np.array_equal(got[0, h], v[0, h // 4])          # L = 1: exactly V
    lens = wl.decode_seq_lens().copy()
    lens[2] = 0
    out = P.decode(dev_bits(qd), g.k, g.v, dev_i32(wl.block_tables), dev_i32(lens), 1024,
                   page_size=wl.page_size)
    torch.cuda.synchronize()
    assert np.all(host_bits(out)[2] == 0)


def test_decode_peaked_softmax(P):
    # q = 30 x (the key of one token): that token's V must dominate.
    wl = W.make("qwen3_decode")
    g = state("qwen3_decode")
    o = OraclePools(wl)
    k, _ = wl.kv_seq(3)
    qd, _ = wl.queries(0)
    qd = qd.copy()
    L = int(wl.total_lens[3])
    qd[3] = W.bf16_bits((W.bf16_to_f32(k[L // 2]).repeat(4, axis=0) * 30).astype(np.float32))
    got = run_decode(P, g, qd)
    ref = oracle.decode(qd, o.k, o.v, wl.block_tables, wl.decode_seq_lens(), wl.page_size, wl.scale)
    check_close(got, ref, "peaked")


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["mixed_step", "window_shared"])
def test_prefill_parity(P, name):
    g = state(name)
    wl = g.wl
    o = OraclePools(wl)
    seqs = wl.prefill_ids()
    for layer in range(wl.num_layers):
        _, qp = wl.queries(layer)
        say(f"[prefill] {name} layer {layer}: N={len(seqs)} Tq={qp.shape[0]}")
        got = run_prefill(P, g, qp)
        ref = oracle.prefill_varlen(qp, o.k, o.v, wl.block_tables[seqs],
                                    wl.cu_lens(wl.new_lens[seqs]), wl.cu_lens(wl.total_lens[seqs]),
                                    wl.page_size, wl.scale, wl.window)
        check_close(got, ref, f"{name} L{layer} prefill")


@pytest.mark.parametrize("shape", [(8, 2, 128, 32, 0), (4, 1, 64, 16, 0), (8, 1, 256, 32, 300)])
def test_prefill_many_blocks_every_row(P, shape):
    """A launch whose longest sequence has many query blocks (the grouped
    dispatch order of the query blocks): decode rows, fresh prompts of ragged
    lengths (one of them empty), and chunks after a cached prefix in one
    batch.  The output starts as NaN, so a block that no workgroup took stays
    non-finite; every row is compared."""
    hq, hkv, d, ps, window = shape
    cfg = W.Config("many_blocks", 20260101, hq, hkv, d, ps, window=window,
                   decode_ctx=("fixed", (5, 300, 1000)),
                   prefill_new=("fixed", (1100, 1, 64, 65, 0, 700, 1025, 33)),
                   chunk=("uniform", 2, 200, 900, 1000))
    wl = W.build(cfg)
    g = GpuPools(wl)
    g.write("prefix")
    g.write("new")
    o = OraclePools(wl)
    cq, ck = wl.cu_lens(wl.new_lens), wl.cu_lens(wl.total_lens)
    qd, qp = wl.queries(0)
    q = np.concatenate([qd, qp])
    say(f"[prefill] many blocks {shape}: {wl.num_seqs} seqs, {q.shape[0]} rows")
    out = torch.full(q.shape, int(W.BF16_NAN), dtype=torch.int16, device="cuda")
    P.prefill_varlen(dev_bits(q), g.k, g.v, dev_i32(wl.block_tables), dev_i32(cq), dev_i32(ck),
                     int(wl.new_lens.max()), int(wl.total_lens.max()), page_size=wl.page_size,
                     scale=wl.scale, window=wl.window, out=out)
    torch.cuda.synchronize()
    ref = oracle.prefill_varlen(q, o.k, o.v, wl.block_tables, cq, ck, wl.page_size, wl.scale,
                                wl.window)
    check_close(host_bits(out), ref, f"many blocks {shape}")


@pytest.mark.parametrize("splits", [1, 3])
def test_varlen_over_1024_sequences(P, splits):
    """More sequences than the compact work list takes (1 024), so the launch
    uses the padded grid: 1 030 decode rows and three prompts of few query
    blocks, with and without key runs; the output starts as NaN and every
    row is compared."""
    cfg = W.Config("many_seqs", 20260102, 8, 2, 128, 16,
                   decode_ctx=("uniform", 1030, 1, 200), prefill_new=("fixed", (70, 1, 129)))
    wl = W.build(cfg)
    g = GpuPools(wl)
    g.write("prefix")
    g.write("new")
    o = OraclePools(wl)
    cq, ck = wl.cu_lens(wl.new_lens), wl.cu_lens(wl.total_lens)
    qd, qp = wl.queries(0)
    q = np.concatenate([qd, qp])
    say(f"[prefill] {wl.num_seqs} sequences, {q.shape[0]} rows, {splits} runs")
    out = torch.full(q.shape, int(W.BF16_NAN), dtype=torch.int16, device="cuda")
    P.prefill_varlen_split(dev_bits(q), g.k, g.v, dev_i32(wl.block_tables), dev_i32(cq),
                           dev_i32(ck), int(wl.new_lens.max()), int(wl.total_lens.max()),
                           page_size=wl.page_size, num_splits=splits, scale=wl.scale,
                           window=wl.window, out=out)
    torch.cuda.synchronize()
    ref = oracle.prefill_varlen(q, o.k, o.v, wl.block_tables, cq, ck, wl.page_size, wl.scale,
                                wl.window)
    check_close(host_bits(out), ref, f"{wl.num_seqs} sequences, {splits} runs")


def test_prefill_edge_cases(P):
    # ragged lengths around tile sizes, an empty sequence, a chunk after a prefix
    wl = W.make("mixed_step", decode_ctx=("fixed", ()), prefill_new=("fixed", (1, 31, 32, 0, 33, 127, 129)),
                name="prefill_edges")
    g = GpuPools(wl)
    g.write("prefix")
    g.write("new")
    _, qp = wl.queries(0)
    say("[prefill] ragged edges")
    got = run_prefill(P, g, qp)
    o = OraclePools(wl)
    seqs = wl.prefill_ids()
    ref = oracle.prefill_varlen(qp, o.k, o.v, wl.block_tables[seqs], wl.prefill_cu_q(),
                                wl.prefill_cu_k(), wl.page_size, wl.scale)
    check_close(got, ref, "prefill edges")
    # first row of a fresh prompt attends only itself: exactly its V
    cq = wl.prefill_cu_q()
    for j, s in enumerate(seqs):
        if wl.new_lens[s] == 0:
            continue
        _, v = wl.kv_seq(int(s))
        assert np.array_equal(got[cq[j]][0], v[0, 0])


def test_decode_equals_last_prefill_row_and_chunk_equals_full(P):
    g = state("mixed_step")
    wl = g.wl
    seqs = wl.prefill_ids()
    _, qp = wl.queries(0)
    full = run_prefill(P, g, qp)
    cq = wl.prefill_cu_q()
    last = qp[cq[1:] - 1]
    dec = run_decode(P, g, last, seqs=seqs)
    a, b = W.bf16_to_f32(dec).astype(np.float64), W.bf16_to_f32(full[cq[1:] - 1]).astype(np.float64)
    assert np.max(np.abs(a - b)) < 2e-2
    # the last 40 rows of sequence 0 as a chunk over its first Lk-40 tokens
    s0 = int(seqs[0])
    Lk = int(wl.total_lens[s0])
    out = P.prefill_varlen(dev_bits(qp[cq[1] - 40:cq[1]]), g.k, g.v, dev_i32(wl.block_tables[[s0]]),
                           dev_i32([0, 40]), dev_i32([0, Lk]), 40, Lk, page_size=wl.page_size)
    torch.cuda.synchronize()
    c = W.bf16_to_f32(host_bits(out)).astype(np.float64)
    f = W.bf16_to_f32(full[cq[1] - 40:cq[1]]).astype(np.float64)
    assert np.max(np.abs(c - f)) < 2e-2


# head_dim, group size (Hq/Hkv, including one that is not a power of two),
# page size and window: every prefill kernel instantiation family, with
# ragged prompts around the 32/64-row and 64-key tile edges and chunks after
# a cached prefix
PREFILL_SHAPES = [  # name, Hq, Hkv, D, page, window
    ("d64_g4_p16", 8, 2, 64, 16, 0),
    ("d64_g1_p32", 4, 4, 64, 32, 0),
    ("d64_g8_p32_win", 16, 2, 64, 32, 100),
    ("d128_g3_p32", 6, 2, 128, 32, 0),
    ("d128_g8_p16", 16, 2, 128, 16, 0),
    ("d128_g2_p16_win", 4, 2, 128, 16, 77),
    ("d256_g2_p16", 4, 2, 256, 16, 0),
]


@pytest.mark.parametrize("shape", PREFILL_SHAPES, ids=[s[0] for s in PREFILL_SHAPES])
def test_prefill_shapes(P, shape):
    name, hq, hkv, d, ps, win = shape
    cfg = W.Config(name, 20261202, hq, hkv, d, ps, window=win, decode_ctx=("fixed", ()),
                   prefill_new=("fixed", (1, 31, 63, 64, 65, 129, 0, 200)),
                   chunk=("uniform", 2, 100, 700, 70))
    wl = W.build(cfg)
    g = GpuPools(wl)
    g.write("prefix")
    g.write("new")
    _, qp = wl.queries(0)
    say(f"[prefill] {name}: N={wl.n_prefill} Tq={qp.shape[0]}")
    got = run_prefill(P, g, qp)
    o = OraclePools(wl)
    seqs = wl.prefill_ids()
    ref = oracle.prefill_varlen(qp, o.k, o.v, wl.block_tables[seqs], wl.prefill_cu_q(),
                                wl.prefill_cu_k(), wl.page_size, wl.scale, wl.window)
    check_close(got, ref, f"{name} prefill")


def test_prefill_deterministic(P):
    g = state("mixed_step")
    _, qp = g.wl.queries(0)
    assert np.array_equal(run_prefill(P, g, qp), run_prefill(P, g, qp))


# ---------------------------------------------------------------------------
# composed steps on one stream
# ---------------------------------------------------------------------------
def test_mixed_step_composed(P):
    """One append of all new tokens, then prefill of the 8 prompts and decode
    of the 56 decoders, on one stream, as the benchmark runs it."""
    wl = W.make("mixed_step")
    g = GpuPools(wl)
    g.write("prefix")
    k, v, lq, lk = wl.packed_tokens("new")
    qd, qp = wl.queries(0)
    say("[step] mixed_step composed")
    slots = P.slot_mapping(g.bt, dev_i32(wl.cu_lens(lq)), dev_i32(wl.cu_lens(lk)),
                           page_size=wl.page_size, num_pages=wl.num_pages, total_tokens=k.shape[0])
    P.append(dev_bits(k), dev_bits(v), slots, g.k, g.v)
    pre = run_prefill(P, g, qp)
    dec = run_decode(P, g, qd)
    o = OraclePools(wl)
    seqs = wl.prefill_ids()
    check_close(pre, oracle.prefill_varlen(qp, o.k, o.v, wl.block_tables[seqs], wl.prefill_cu_q(),
                                           wl.prefill_cu_k(), wl.page_size, wl.scale), "step prefill")
    check_close(dec, oracle.decode(qd, o.k, o.v, wl.block_tables, wl.decode_seq_lens(),
                                   wl.page_size, wl.scale), "step decode")
