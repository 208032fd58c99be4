"""The seeded input generators: determinism and the stated shapes/ranges."""
import numpy as np
import pytest

import workloads as W


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_lengths_tables_and_pool(name):
    wl = W.make(name)
    cfg = W.CONFIGS[name]
    ps = wl.page_size
    tot = wl.total_lens
    npg = -(-tot // ps)
    used = wl.block_tables[np.arange(wl.max_pages_per_seq)[None, :] < npg[:, None]]
    # every used page is distinct and in range; the pad page is unused
    assert len(np.unique(used)) == used.size == int(npg.sum())
    assert used.min() >= 0 and used.max() < wl.num_pages
    assert wl.pad_page not in set(used.tolist())
    if cfg.decode_ctx is not None:
        if cfg.decode_ctx[0] == "uniform":
            _, n, lo, hi = cfg.decode_ctx
            ctx = wl.prefix_lens[:wl.n_decode]
            assert len(ctx) == n and ctx.min() >= lo and ctx.max() <= hi
        assert np.all(wl.new_lens[:wl.n_decode] == 1)
    if cfg.prefill_new is not None:
        _, n, lo, hi = cfg.prefill_new
        nl = wl.new_lens[wl.n_decode:wl.n_decode + n]
        assert nl.min() >= lo and nl.max() <= hi
        assert np.all(wl.prefix_lens[wl.n_decode:wl.n_decode + n] == 0)
    if cfg.chunk is not None:
        _, n, lo, hi, c = cfg.chunk
        pre = wl.prefix_lens[-n:]
        assert pre.min() >= lo and pre.max() <= hi and np.all(wl.new_lens[-n:] == c)


def test_tiny_decode_is_the_stated_case():
    wl = W.make("tiny_decode")
    assert wl.prefix_lens.tolist() == [5, 17, 32, 63]
    assert wl.num_pages == 32 and wl.page_size == 16
    assert (wl.num_q_heads, wl.num_kv_heads, wl.head_dim) == (2, 1, 64)
    assert abs(wl.scale - 1 / 8) < 1e-15


def test_same_seed_same_bytes_other_seed_differs():
    a = W.make("qwen3_decode")
    b = W.make("qwen3_decode")
    c = W.make("qwen3_decode", seed=123)
    assert np.array_equal(a.block_tables, b.block_tables)
    assert np.array_equal(a.kv_seq(3)[0], b.kv_seq(3)[0])
    assert np.array_equal(a.queries(0)[0], b.queries(0)[0])
    assert not np.array_equal(a.prefix_lens, c.prefix_lens)
    assert not np.array_equal(a.queries(1)[0], a.queries(0)[0])


def test_values_are_standard_normal_bf16():
    wl = W.make("qwen3_decode")
    k, v = wl.kv_seq(0)
    x = W.bf16_to_f32(k).astype(np.float64)
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02
    assert k.dtype == np.uint16 and k.shape == (int(wl.total_lens[0]), 8, 128)


def test_cached_generation_matches_lazy():
    wl = W.make("mixed_step")
    lazy = [wl.kv_seq(s)[1] for s in (0, 60)]
    wl.cache_all_kv([0, 60])
    assert all(np.array_equal(x, wl.kv_seq(s)[1]) for x, s in zip(lazy, (0, 60)))


def test_packed_tokens_layout():
    wl = W.make("window_shared")
    k, v, lq, lk = wl.packed_tokens("new")
    assert k.shape[0] == int(wl.new_lens.sum()) == 64 + 4 * 128
    assert np.array_equal(lk, wl.total_lens)
    s = wl.n_decode  # first chunk sequence
    off = int(lq[:s].sum())
    K, _ = wl.kv_seq(s)
    p = int(wl.prefix_lens[s])
    assert np.array_equal(k[off:off + 128], K[p:p + 128])
