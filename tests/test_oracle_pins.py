"""Pins for the CPU oracle: each check ties it to something other than itself.

Sources of truth used here: hand-derived fixtures from the pages' stated
rules (tests/golden), closed forms, special cases that reduce to a textbook
or library routine (a mean, a sigmoid, torch's scaled_dot_product_attention),
invariants, and brute force written independently on tiny inputs.
"""
import math
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].strip()
        if line:
            out.append([int(x) for x in line.split()])
    return out


def _bits(x):
    """float values exactly representable in bf16 -> bit patterns."""
    x = np.asarray(x, dtype=np.float32)
    b = (x.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_to_f64(b), x.astype(np.float64)), "value not bf16-exact"
    return b


def _pool(hkv, pages, ps, d, fill=W.BF16_NAN):
    return np.full((hkv, pages * ps, d), fill, dtype=np.uint16)


def _dense_pools(K, V, ps, perm=None, spare=1):
    """Place one sequence's [L, Hkv, D] K/V into fresh pools page by page
    (independently of the oracle's slot code) and return pools + table row."""
    L, hkv, d = K.shape
    npg = -(-L // ps)
    perm = np.arange(npg) if perm is None else np.asarray(perm)
    kp = _pool(hkv, npg + spare, ps, d)
    vp = _pool(hkv, npg + spare, ps, d)
    for lp in range(npg):
        rows = slice(lp * ps, min(L, (lp + 1) * ps))
        n = rows.stop - rows.start
        base = int(perm[lp]) * ps
        kp[:, base:base + n, :] = K[rows].transpose(1, 0, 2)
        vp[:, base:base + n, :] = V[rows].transpose(1, 0, 2)
    return kp, vp, perm.astype(np.int32)


# ---------------------------------------------------------------------------
# bf16 handling
# ---------------------------------------------------------------------------
def test_bf16_decode_known_patterns():
    b = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x4049, 0x0001, 0x7F80], dtype=np.uint16)
    f = oracle.bf16_to_f64(b)
    assert f[0] == 1.0 and f[1] == -2.0 and f[2] == 0.0 and math.copysign(1, f[3]) < 0
    assert f[4] == 3.140625
    assert f[5] == 2.0 ** -133
    assert math.isinf(f[6])
    assert math.isnan(oracle.bf16_to_f64(np.array([0x7FC0], np.uint16))[0])


def test_generator_rounding_matches_torch_bf16():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -1.00390625, 3.0e-39], np.float32)])
    ours = W.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------------------
# addressing, slot write and gather
# ---------------------------------------------------------------------------
def test_slot_mapping_golden():
    rows = _rows("slot_mapping.txt")
    ps = rows[0][0]
    bt = np.array(rows[1:4], dtype=np.int32)
    cq, ck, expect = rows[4], rows[5], rows[6]
    got = oracle.slot_mapping(bt, cq, ck, ps)
    assert got.tolist() == expect


def test_append_writes_exact_rows_and_skips_negative():
    hkv, d, ps = 2, 8, 4
    kp = _pool(hkv, 3, ps, d)
    vp = _pool(hkv, 3, ps, d)
    rng = np.random.default_rng(0)
    kn = rng.integers(0, 0x7F00, size=(3, hkv, d)).astype(np.uint16)
    vn = rng.integers(0, 0x7F00, size=(3, hkv, d)).astype(np.uint16)
    ko, vo = oracle.append(kp, vp, kn, vn, np.array([5, -1, 11]))
    ek, ev = kp.copy(), vp.copy()
    for h in range(hkv):
        ek[h, 5], ev[h, 5] = kn[0, h], vn[0, h]
        ek[h, 11], ev[h, 11] = kn[2, h], vn[2, h]
    assert np.array_equal(ko, ek) and np.array_equal(vo, ev)
    assert np.array_equal(kp, _pool(hkv, 3, ps, d))  # inputs untouched


def test_append_then_gather_round_trip_every_config_shape():
    wl = W.make("tiny_decode")
    kp = _pool(wl.num_kv_heads, wl.num_pages, wl.page_size, wl.head_dim)
    vp = kp.copy()
    for part in ("prefix", "new"):
        k, v, lq, lk = wl.packed_tokens(part)
        slots = oracle.slot_mapping(wl.block_tables, wl.cu_lens(lq), wl.cu_lens(lk), wl.page_size)
        kp, vp = oracle.append(kp, vp, k, v, slots)
    for s in range(wl.num_seqs):
        K, V = wl.kv_seq(s)
        L = int(wl.total_lens[s])
        gk = oracle.gather(kp, wl.block_tables[s], L, wl.page_size)
        assert np.array_equal(gk, oracle.bf16_to_f64(K).transpose(1, 0, 2))
        gv = oracle.gather(vp, wl.block_tables[s], L, wl.page_size)
        assert np.array_equal(gv, oracle.bf16_to_f64(V).transpose(1, 0, 2))
    # exactly the used rows were written; everything else is still poison
    used = np.zeros(wl.num_slots, bool)
    for s in range(wl.num_seqs):
        for i in range(int(wl.total_lens[s])):
            used[wl.block_tables[s, i // wl.page_size] * wl.page_size + i % wl.page_size] = True
    assert np.all(kp[:, ~used, :] == W.BF16_NAN)
    assert used.sum() == int(wl.total_lens.sum())


def test_gather_hand_example():
    # two pages of size 2, one head, D=1; logical page 0 -> physical 1, 1 -> 0
    pool = _bits(np.array([[[3.0], [4.0], [1.0], [2.0]]], np.float32))
    g = oracle.gather(pool, np.array([1, 0]), 3, 2)
    assert g[0, :, 0].tolist() == [1.0, 2.0, 3.0]


# ---------------------------------------------------------------------------
# masks
# ---------------------------------------------------------------------------
def test_window_rule_golden():
    for q, kv, win, ok in _rows("window_rule.txt"):
        keys = set(oracle.allowed_keys(q, win).tolist())
        assert (kv in keys) == bool(ok), (q, kv, win)


def test_split_ranges_golden():
    for L, ps, win, pps, s, a, b in _rows("split_ranges.txt"):
        assert oracle.split_page_range(L, ps, win, pps, s) == (a, b), (L, ps, win, pps, s)


# ---------------------------------------------------------------------------
# attention: closed forms
# ---------------------------------------------------------------------------
def _seq(rng, L, hkv, d):
    return (W.bf16_bits(rng.standard_normal((L, hkv, d)).astype(np.float32)),
            W.bf16_bits(rng.standard_normal((L, hkv, d)).astype(np.float32)))


def test_length_one_returns_v_exactly():
    rng = np.random.default_rng(1)
    K, V = _seq(rng, 1, 2, 16)
    kp, vp, row = _dense_pools(K, V, 16)
    q = W.bf16_bits(rng.standard_normal((1, 4, 16)).astype(np.float32))
    out = oracle.decode(q, kp, vp, row[None], np.array([1]), 16, 0.25)
    for h in range(4):
        assert np.array_equal(out[0, h], oracle.bf16_to_f64(V[0, h // 2]))
    outp = oracle.prefill_varlen(q, kp, vp, row[None], [0, 1], [0, 1], 16, 0.25)
    assert np.array_equal(outp, out)


@pytest.mark.parametrize("window", [0, 5, 1])
def test_identical_keys_give_mean_of_allowed_v(window):
    rng = np.random.default_rng(2)
    L, hkv, d = 37, 1, 8
    K, V = _seq(rng, L, hkv, d)
    K[:] = K[0]
    kp, vp, row = _dense_pools(K, V, 8, perm=rng.permutation(5))
    q = W.bf16_bits(rng.standard_normal((1, 3, d)).astype(np.float32))
    out = oracle.decode(q, kp, vp, row[None], np.array([L]), 8, 0.3, window)
    Vf = V.astype(np.uint32) << 16
    Vf = Vf.view(np.float32).astype(np.float64)
    lo = 0 if window <= 0 else L - window
    expect = Vf[lo:, 0, :].mean(axis=0)
    for h in range(3):
        np.testing.assert_allclose(out[0, h], expect, rtol=1e-12, atol=1e-14)


def test_zero_query_bottom_right_alignment_in_chunked_prefill():
    # q = 0 makes every allowed key equally weighted: row r of a chunk with
    # Lq new and Lk total tokens must average keys 0 .. Lk-Lq+r.
    rng = np.random.default_rng(3)
    Lk, Lq, d = 29, 6, 4
    K, V = _seq(rng, Lk, 1, d)
    kp, vp, row = _dense_pools(K, V, 4, perm=rng.permutation(8))
    q = np.zeros((Lq, 2, d), np.uint16)
    out = oracle.prefill_varlen(q, kp, vp, row[None], [0, Lq], [0, Lk], 4, 1.0)
    Vf = oracle.bf16_to_f64(V)[:, 0, :]
    for r in range(Lq):
        np.testing.assert_allclose(out[r, 0], Vf[: Lk - Lq + r + 1].mean(0), rtol=1e-12)


def test_window_one_returns_own_v():
    rng = np.random.default_rng(4)
    K, V = _seq(rng, 20, 1, 8)
    kp, vp, row = _dense_pools(K, V, 8)
    q = W.bf16_bits(rng.standard_normal((1, 1, 8)).astype(np.float32))
    out = oracle.decode(q, kp, vp, row[None], np.array([20]), 8, 0.5, window=1)
    assert np.array_equal(out[0, 0], oracle.bf16_to_f64(V[19, 0]))


def test_two_key_sigmoid_closed_form():
    # D=1: scores scale*q*k; out = (v0 + v1 e^{x1-x0}) / (1 + e^{x1-x0}).
    K = _bits(np.array([[[0.5]], [[-1.25]]], np.float32))
    V = _bits(np.array([[[2.0]], [[-3.0]]], np.float32))
    kp, vp, row = _dense_pools(K, V, 2)
    q = _bits(np.array([[[1.5]]], np.float32))
    scale = 0.7
    out = oracle.decode(q, kp, vp, row[None], np.array([2]), 2, scale)
    dx = scale * 1.5 * (-1.25 - 0.5)
    expect = (2.0 + -3.0 * math.exp(dx)) / (1.0 + math.exp(dx))
    assert abs(out[0, 0, 0] - expect) < 1e-14


def test_gqa_head_grouping_is_contiguous():
    # Each KV head holds a constant V; query head h must return the value of
    # KV head h // (Hq/Hkv).
    hkv, hq, d, L = 4, 8, 4, 9
    K = np.zeros((L, hkv, d), np.uint16)
    V = np.zeros((L, hkv, d), np.uint16)
    for kh in range(hkv):
        V[:, kh, :] = _bits(np.float32(kh + 1))
    kp, vp, row = _dense_pools(K, V, 4)
    rng = np.random.default_rng(5)
    q = W.bf16_bits(rng.standard_normal((1, hq, d)).astype(np.float32))
    out = oracle.decode(q, kp, vp, row[None], np.array([L]), 4, 1.0)
    for h in range(hq):
        assert np.all(out[0, h] == h // 2 + 1)


def test_peaked_softmax_picks_the_dominant_key():
    rng = np.random.default_rng(6)
    L, d = 40, 16
    K, V = _seq(rng, L, 1, d)
    qv = oracle.bf16_to_f64(K[17, 0]) * 30.0
    q = W.bf16_bits(qv.astype(np.float32))[None, None, :]
    kp, vp, row = _dense_pools(K, V, 8, perm=rng.permutation(5))
    out = oracle.decode(q, kp, vp, row[None], np.array([L]), 8, 1.0)
    np.testing.assert_allclose(out[0, 0], oracle.bf16_to_f64(V[17, 0]), atol=1e-6)


# ---------------------------------------------------------------------------
# attention: independent brute force and a library special case
# ---------------------------------------------------------------------------
def _brute(qf, Kf, Vf, Lq, Lk, scale, window):
    """Dense attention with scalar loops, an explicit Lq x Lk mask and
    math.exp; works on the logical (unpaged) arrays."""
    _, Hq, D = qf.shape
    Hkv = Kf.shape[1]
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(Lq)]
    for r in range(Lq):
        p = Lk - Lq + r
        mask = [(i <= p) and (window <= 0 or p - i < window) for i in range(Lk)]
        for h in range(Hq):
            kh = (h * Hkv) // Hq
            sc = []
            for i in range(Lk):
                if mask[i]:
                    acc = 0.0
                    for dd in range(D):
                        acc += float(qf[r, h, dd]) * float(Kf[i, kh, dd])
                    sc.append((i, acc * scale))
            if not sc:
                continue
            mx = max(x for _, x in sc)
            ws = [(i, math.exp(x - mx)) for i, x in sc]
            tot = math.fsum(w for _, w in ws)
            for dd in range(D):
                out[r][h][dd] = math.fsum(w * float(Vf[i, kh, dd]) for i, w in ws) / tot
    return np.array(out)


@pytest.mark.parametrize("Lq,Lk,hq,hkv,d,ps,window", [
    (1, 1, 1, 1, 8, 4, 0),
    (1, 13, 4, 2, 16, 4, 0),
    (5, 5, 2, 1, 8, 4, 0),
    (7, 19, 4, 1, 16, 8, 0),
    (9, 30, 4, 2, 8, 4, 6),
    (1, 70, 2, 1, 64, 16, 0),
    (3, 70, 4, 4, 32, 16, 17),
])
def test_brute_force_dense(Lq, Lk, hq, hkv, d, ps, window):
    rng = np.random.default_rng(100 + Lq * 7 + Lk)
    K, V = _seq(rng, Lk, hkv, d)
    q = W.bf16_bits(rng.standard_normal((Lq, hq, d)).astype(np.float32))
    npg = -(-Lk // ps)
    kp, vp, row = _dense_pools(K, V, ps, perm=rng.permutation(npg + 2)[:npg], spare=2)
    scale = 1.0 / math.sqrt(d)
    got = oracle.prefill_varlen(q, kp, vp, row[None], [0, Lq], [0, Lk], ps, scale, window)
    ref = _brute(oracle.bf16_to_f64(q), oracle.bf16_to_f64(K), oracle.bf16_to_f64(V),
                 Lq, Lk, scale, window)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    if Lq == 1:
        dec = oracle.decode(q, kp, vp, row[None], np.array([Lk]), ps, scale, window)
        np.testing.assert_allclose(dec, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("Lq,Lk,hq,hkv,d,window,block", [
    (1, 1, 1, 1, 8, 0, 512),
    (5, 5, 2, 1, 8, 0, 2),
    (7, 19, 4, 1, 16, 0, 3),
    (9, 30, 4, 2, 8, 6, 4),
    (3, 70, 4, 4, 32, 17, 512),
    (40, 40, 4, 2, 16, 0, 16),
])
def test_matrix_form_matches_brute_force(Lq, Lk, hq, hkv, d, window, block):
    # the matrix form of the row attention (used on long prompts) against the
    # scalar-loop brute force on the logical arrays, with row blocks that cut
    # the rows unevenly
    rng = np.random.default_rng(200 + Lq * 3 + Lk)
    K, V = _seq(rng, Lk, hkv, d)
    q = W.bf16_bits(rng.standard_normal((Lq, hq, d)).astype(np.float32))
    scale = 1.0 / math.sqrt(d)
    got = oracle.attend_rows_matrix(oracle.bf16_to_f64(q), oracle.bf16_to_f64(K).transpose(1, 0, 2),
                                    oracle.bf16_to_f64(V).transpose(1, 0, 2),
                                    np.arange(Lk - Lq, Lk), scale, window, block=block)
    ref = _brute(oracle.bf16_to_f64(q), oracle.bf16_to_f64(K), oracle.bf16_to_f64(V),
                 Lq, Lk, scale, window)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_matrix_form_closed_forms():
    rng = np.random.default_rng(21)
    Lk, d = 33, 8
    K, V = _seq(rng, Lk, 1, d)
    Kf = oracle.bf16_to_f64(K).transpose(1, 0, 2)
    Vf = oracle.bf16_to_f64(V).transpose(1, 0, 2)
    # q = 0: row at position p averages keys 0..p (bottom-right alignment),
    # or the last `window` of them
    q0 = np.zeros((6, 2, d))
    for window in (0, 5):
        out = oracle.attend_rows_matrix(q0, Kf, Vf, np.arange(27, 33), 1.0, window, block=4)
        for r, p in enumerate(range(27, 33)):
            lo = 0 if window <= 0 else p - window + 1
            np.testing.assert_allclose(out[r, 1], Vf[0, lo:p + 1].mean(0), rtol=1e-12)
    # position 0 returns V[0] exactly; a negative position (no allowed key) is zero
    qr = oracle.bf16_to_f64(W.bf16_bits(rng.standard_normal((2, 1, d)).astype(np.float32)))
    out = oracle.attend_rows_matrix(qr, Kf, Vf, np.array([0, -1]), 0.3, 0)
    assert np.array_equal(out[0, 0], Vf[0, 0]) and np.all(out[1] == 0)


def test_brute_force_tiny_decode_config():
    wl = W.make("tiny_decode")
    kp = _pool(wl.num_kv_heads, wl.num_pages, wl.page_size, wl.head_dim)
    vp = kp.copy()
    for part in ("prefix", "new"):
        k, v, lq, lk = wl.packed_tokens(part)
        slots = oracle.slot_mapping(wl.block_tables, wl.cu_lens(lq), wl.cu_lens(lk), wl.page_size)
        kp, vp = oracle.append(kp, vp, k, v, slots)
    qd, _ = wl.queries(0)
    got = oracle.decode(qd, kp, vp, wl.block_tables, wl.decode_seq_lens(), wl.page_size, wl.scale)
    for b in range(wl.n_decode):
        K, V = wl.kv_seq(b)
        L = int(wl.total_lens[b])
        ref = _brute(oracle.bf16_to_f64(qd[b:b + 1]), oracle.bf16_to_f64(K),
                     oracle.bf16_to_f64(V), 1, L, wl.scale, 0)
        np.testing.assert_allclose(got[b:b + 1], ref, atol=1e-12)


def test_torch_sdpa_special_case():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(9)
    Lq, Lk, hq, hkv, d, ps, window = 24, 90, 8, 2, 32, 16, 33
    K, V = _seq(rng, Lk, hkv, d)
    q = W.bf16_bits(rng.standard_normal((Lq, hq, d)).astype(np.float32))
    npg = -(-Lk // ps)
    kp, vp, row = _dense_pools(K, V, ps, perm=rng.permutation(npg))
    scale = 1.0 / math.sqrt(d)
    got = oracle.prefill_varlen(q, kp, vp, row[None], [0, Lq], [0, Lk], ps, scale, window)
    g = hq // hkv
    qt = torch.from_numpy(oracle.bf16_to_f64(q)).permute(1, 0, 2)                 # [Hq, Lq, D]
    kt = torch.from_numpy(oracle.bf16_to_f64(K)).permute(1, 0, 2).repeat_interleave(g, 0)
    vt = torch.from_numpy(oracle.bf16_to_f64(V)).permute(1, 0, 2).repeat_interleave(g, 0)
    qpos = torch.arange(Lk - Lq, Lk)[:, None]
    kpos = torch.arange(Lk)[None, :]
    mask = (kpos <= qpos) & (qpos - kpos < window)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    np.testing.assert_allclose(got, ref.permute(1, 0, 2).numpy(), atol=1e-12)


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------
def test_page_permutation_invariance_is_bit_exact():
    rng = np.random.default_rng(11)
    L, hkv, hq, d, ps = 45, 2, 4, 16, 8
    K, V = _seq(rng, L, hkv, d)
    q = W.bf16_bits(rng.standard_normal((1, hq, d)).astype(np.float32))
    a = oracle.decode(q, *_dense_pools(K, V, ps)[:2], np.arange(6, dtype=np.int32)[None],
                      np.array([L]), ps, 0.25)
    kp, vp, row = _dense_pools(K, V, ps, perm=rng.permutation(9)[:6], spare=3)
    b = oracle.decode(q, kp, vp, row[None], np.array([L]), ps, 0.25)
    assert np.array_equal(a, b)


def test_window_wider_than_context_equals_no_window():
    rng = np.random.default_rng(12)
    K, V = _seq(rng, 33, 1, 8)
    kp, vp, row = _dense_pools(K, V, 8)
    q = W.bf16_bits(rng.standard_normal((1, 2, 8)).astype(np.float32))
    a = oracle.decode(q, kp, vp, row[None], np.array([33]), 8, 0.3, window=0)
    b = oracle.decode(q, kp, vp, row[None], np.array([33]), 8, 0.3, window=33)
    c = oracle.decode(q, kp, vp, row[None], np.array([33]), 8, 0.3, window=32)
    assert np.array_equal(a, b) and not np.allclose(a, c)


def test_chunked_prefill_equals_unchunked_and_decode_equals_last_row():
    rng = np.random.default_rng(13)
    Lk, hkv, hq, d, ps = 50, 1, 2, 16, 8
    K, V = _seq(rng, Lk, hkv, d)
    kp, vp, row = _dense_pools(K, V, ps, perm=rng.permutation(7))
    q = W.bf16_bits(rng.standard_normal((Lk, hq, d)).astype(np.float32))
    full = oracle.prefill_varlen(q, kp, vp, row[None], [0, Lk], [0, Lk], ps, 0.25, 0)
    # the last 12 rows as a chunk over a 38-token cached prefix
    chunk = oracle.prefill_varlen(q[38:], kp, vp, row[None], [0, 12], [0, Lk], ps, 0.25, 0)
    np.testing.assert_allclose(chunk, full[38:], atol=1e-14)
    dec = oracle.decode(q[Lk - 1:], kp, vp, row[None], np.array([Lk]), ps, 0.25)
    np.testing.assert_allclose(dec[0], full[-1], atol=1e-14)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(14)
    L, hkv, hq, d, ps = 21, 2, 6, 8, 4
    K, V = _seq(rng, L, hkv, d)
    q = W.bf16_bits(rng.standard_normal((1, hq, d)).astype(np.float32))
    kp, vp, row = _dense_pools(K, V, ps)
    a = oracle.decode(q, kp, vp, row[None], np.array([L]), ps, 0.4)
    Kr, Vr = np.repeat(K, 3, axis=1), np.repeat(V, 3, axis=1)
    kp2, vp2, row2 = _dense_pools(Kr, Vr, ps)
    b = oracle.decode(q, kp2, vp2, row2[None], np.array([L]), ps, 0.4)
    np.testing.assert_allclose(a, b, atol=1e-14)


def test_batch_order_permutes_outputs():
    wl = W.make("tiny_decode")
    kp = _pool(wl.num_kv_heads, wl.num_pages, wl.page_size, wl.head_dim)
    vp = kp.copy()
    for part in ("prefix", "new"):
        k, v, lq, lk = wl.packed_tokens(part)
        kp, vp = oracle.append(kp, vp, k, v, oracle.slot_mapping(
            wl.block_tables, wl.cu_lens(lq), wl.cu_lens(lk), wl.page_size))
    qd, _ = wl.queries(0)
    lens = wl.decode_seq_lens()
    a = oracle.decode(qd, kp, vp, wl.block_tables, lens, wl.page_size, wl.scale)
    p = np.array([2, 0, 3, 1])
    b = oracle.decode(qd[p], kp, vp, wl.block_tables[p], lens[p], wl.page_size, wl.scale)
    assert np.array_equal(a[p], b)


@pytest.mark.parametrize("window,pps,S", [(0, 1, 5), (0, 2, 3), (0, 8, 1), (9, 1, 4), (30, 2, 3)])
def test_split_partials_combine_to_full_attention(window, pps, S):
    rng = np.random.default_rng(15)
    hkv, hq, d, ps = 2, 4, 8, 8
    lens = np.array([1, 8, 9, 33, 40])
    bts, kp_list = [], []
    npg = [-(-L // ps) for L in lens]
    P = sum(npg) + 1
    perm = rng.permutation(P)
    kp = _pool(hkv, P, ps, d)
    vp = _pool(hkv, P, ps, d)
    bt = np.full((len(lens), max(npg)), perm[-1], np.int32)
    off = 0
    for b, L in enumerate(lens):
        K, V = _seq(rng, int(L), hkv, d)
        bt[b, :npg[b]] = perm[off:off + npg[b]]
        for i in range(L):
            r = bt[b, i // ps] * ps + i % ps
            kp[:, r, :] = K[i]
            vp[:, r, :] = V[i]
        off += npg[b]
    q = W.bf16_bits(rng.standard_normal((len(lens), hq, d)).astype(np.float32))
    S_needed = max(-(-npg_i // pps) for npg_i in npg)
    S = max(S, S_needed)
    m2, l, acc = oracle.decode_partials(q, kp, vp, bt, lens, ps, 0.35, window, pps, S)
    full = oracle.decode(q, kp, vp, bt, lens, ps, 0.35, window)
    np.testing.assert_allclose(oracle.combine_partials(m2, l, acc), full, atol=1e-13)
    # empty splits carry (-inf, 0, 0)
    empty = ~np.isfinite(m2)
    assert np.all(l[empty] == 0) and np.all(acc[empty] == 0)


def test_split_partials_closed_form_with_zero_query():
    # q = 0: every score is 0, so m2 = 0, l = number of keys in the split and
    # acc = the plain sum of their V rows.
    rng = np.random.default_rng(16)
    L, d, ps = 29, 4, 4
    K, V = _seq(rng, L, 1, d)
    kp, vp, row = _dense_pools(K, V, ps, perm=rng.permutation(8))
    q = np.zeros((1, 1, d), np.uint16)
    m2, l, acc = oracle.decode_partials(q, kp, vp, row[None], np.array([L]), ps, 1.0, 0, 3, 3)
    Vf = oracle.bf16_to_f64(V)[:, 0, :]
    for s, (a, b) in enumerate([(0, 12), (12, 24), (24, 29)]):
        assert m2[0, 0, s] == 0.0 and l[0, 0, s] == b - a
        np.testing.assert_allclose(acc[0, 0, s], Vf[a:b].sum(0), rtol=1e-13)


def test_empty_sequence_gives_zero_row():
    q = np.full((1, 2, 4), 0x3F80, np.uint16)
    kp = _pool(1, 1, 4, 4)
    out = oracle.decode(q, kp, kp, np.zeros((1, 1), np.int32), np.array([0]), 4, 1.0)
    assert np.all(out == 0)
