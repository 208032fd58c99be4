"""The decode step with its append fused into the decode launch
(pkv_decode_append) against the same step as two launches
(pkv_append_mapped of one token per row, then pkv_decode) and against the
oracle.  The pools after the step must be bit-equal to the two-launch
step's and to the oracle's, and the outputs bit-equal to the two-launch
step's (the new row's values are the same bits whether they come from the
pool or from k_new) and within the bar of the oracle.  Covers every
decomposition (direct, stream-K with and without the split of wide query
groups, split-K + combine), head_dim 64/128/256/512, windows, padded rows
of length 0, page-boundary lengths and an unusable table entry."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from gpu_harness import (GpuPools, OraclePools, check_close, dev_bits, dev_i32,  # noqa: E402
                         host_bits, say)


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import paged_kv_attention_mapped_amd as P
    P.lib()
    return P


def _two_launch(P, wl, g, q, kn, vn, bt, lens, splits):
    """pkv_append_mapped of row b's token at position lens[b]-1, then pkv_decode."""
    ck = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    # a row of length 0 has no new token: cu_seq_lens_q repeats its last entry
    cq = np.concatenate([[0], np.cumsum(lens > 0)]).astype(np.int32)
    live = lens > 0
    P.append_mapped(dev_bits(kn[live]), dev_bits(vn[live]), dev_i32(bt), dev_i32(cq),
                    dev_i32(ck), g.k, g.v, page_size=wl.page_size, max_seqlen_q=1)
    out = P.decode(dev_bits(q), g.k, g.v, dev_i32(bt), dev_i32(lens), int(max(1, lens.max())),
                   page_size=wl.page_size, scale=wl.scale, window=wl.window, num_splits=splits)
    torch.cuda.synchronize()
    return host_bits(out)


def _fused(P, wl, g, q, kn, vn, bt, lens, splits):
    out = P.decode_append(dev_bits(q), dev_bits(kn), dev_bits(vn), g.k, g.v, dev_i32(bt),
                          dev_i32(lens), int(max(1, lens.max())), page_size=wl.page_size,
                          scale=wl.scale, window=wl.window, num_splits=splits)
    torch.cuda.synchronize()
    return host_bits(out)


CASES = [  # (label, workload name or Config, num_splits)
    ("tiny_direct", "tiny_decode", 0),
    ("qwen3_direct", "qwen3_decode", 0),
    ("qwen3_split3", "qwen3_decode", 3),
    ("mixed_decoders_stream", "mixed_step", 0),
    ("window_stream_halves", "window_shared", 0),
    ("window_split2", "window_shared", 2),
    ("d64_g8_p16", W.Config("d64_g8_p16", 20261204, 8, 1, 64, 16,
                            decode_ctx=("fixed", (1, 15, 16, 17, 33, 64, 300)))),
    ("d128_g6_p16_stream", W.Config("d128_g6_p16", 20261205, 12, 2, 128, 16,
                                    decode_ctx=("uniform", 40, 1, 700))),
    ("d128_g7_p32", W.Config("d128_g7_p32", 20261206, 7, 1, 128, 32,
                             decode_ctx=("fixed", (0, 31, 32, 63, 1000)))),
    ("d512_g8_p32", W.Config("d512_g8", 20261207, 8, 1, 512, 32,
                             decode_ctx=("fixed", (0, 31, 32, 500, 1100)))),
    ("d512_g4_p16_split", W.Config("d512_g4", 20261208, 4, 1, 512, 16, window=300,
                                   decode_ctx=("fixed", (3, 16, 299, 300, 900)))),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_append_decode(P, case):
    label, spec = case[0], case[1]
    splits = case[2] if len(case) > 2 else 0
    wl = W.make(spec) if isinstance(spec, str) else W.build(spec)
    dec = wl.decode_ids()
    lens = wl.decode_seq_lens()
    kn, vn, _, _ = wl.packed_tokens("new", dec)
    bt = wl.block_tables[dec]
    for layer in range(wl.num_layers):
        q, _ = wl.queries(layer)
        say(f"[fused] {label} layer {layer}: B={len(dec)} splits={splits}")
        ga, gb = GpuPools(wl), GpuPools(wl)
        ga.write("prefix")
        gb.write("prefix")
        got = _fused(P, wl, ga, q, kn, vn, bt, lens, splits)
        ref2 = _two_launch(P, wl, gb, q, kn, vn, bt, lens, splits)
        assert np.array_equal(got, ref2), "fused step differs from append + decode"
        assert torch.equal(ga.k, gb.k) and torch.equal(ga.v, gb.v), "pools differ"
        # the oracle: prefixes of every sequence, then the decoders' new tokens
        o = OraclePools(wl, parts=("prefix",))
        cq = np.arange(len(dec) + 1)
        ck = wl.cu_lens(wl.total_lens[dec])
        ok_, ov_ = oracle.append(o.k, o.v, kn, vn, oracle.slot_mapping(bt, cq, ck, wl.page_size))
        assert np.array_equal(host_bits(ga.k), ok_) and np.array_equal(host_bits(ga.v), ov_)
        ref = oracle.decode(q, ok_, ov_, bt, lens, wl.page_size, wl.scale, wl.window)
        check_close(got, ref, f"{label} L{layer}")
        zero = lens == 0
        assert np.all(got[zero] == 0)


@pytest.mark.parametrize("heads", [(32, 8, 128), (16, 2, 512)], ids=["d128", "d512"])
def test_fused_padded_rows_and_unusable_entries(P, heads):
    """Rows of length 0 (graph-bucket padding) write nothing and give zeros;
    a row whose last table entry is unusable (-1, or past the pool) writes
    nothing; results equal the two-launch step's bit for bit.  At head_dim
    512 the stream-K kernel appends (no splits), a launch of its own appends
    before the direct and split kernels."""
    hq, hkv, d = heads
    cfg = W.Config("pad", 20261209, hq, hkv, d, 32,
                   decode_ctx=("fixed", (40, 0, 95, 31, 200, 63, 7, 500)))
    wl = W.build(cfg)
    dec = wl.decode_ids()
    lens = wl.decode_seq_lens().copy()
    lens[[3, 6]] = 0                               # padded rows: no token, no keys
    kn, vn, _, _ = wl.packed_tokens("new", dec)
    bt = wl.block_tables[dec].copy()
    bt[2, (int(lens[2]) - 1) // wl.page_size] = -1            # the new token's page unusable
    bt[5, (int(lens[5]) - 1) // wl.page_size] = wl.num_pages  # past the pool
    q, _ = wl.queries(0)
    for splits in (0, 1, 2):
        say(f"[fused] padded rows and unusable entries, head_dim {d}, splits={splits}")
        ga, gb = GpuPools(wl), GpuPools(wl)
        ga.write("prefix")
        gb.write("prefix")
        before = host_bits(ga.k)
        got = _fused(P, wl, ga, q, kn, vn, bt, lens, splits)
        ref2 = _two_launch(P, wl, gb, q, kn, vn, bt, lens, splits)
        assert np.array_equal(got, ref2)
        assert torch.equal(ga.k, gb.k) and torch.equal(ga.v, gb.v)
        assert np.all(got[[3, 6]] == 0)
        # exactly the live rows with a usable page were written
        changed = np.flatnonzero((host_bits(ga.k) != before).any(axis=(0, 2)))
        assert len(changed) == 4, changed        # rows 0, 1, 4 and 7
