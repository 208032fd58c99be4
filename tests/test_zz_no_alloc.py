"""pkv_decode_noalloc, the decode for callers that cannot allocate (its
partials live in the library's per-GPU scratch array), against pkv_decode
with a workspace of its own: bit-identical outputs on consecutive calls,
each later call with a smaller input than the one before, for both
decompositions that use the scratch (stream-K, split-K), and within the
bar of the oracle."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from gpu_harness import GpuPools, OraclePools, check_close, dev_bits, dev_i32, host_bits, say  # noqa: E402


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import paged_kv_attention_mapped_amd as P
    P.lib()
    return P


def _pools(wl):
    g = GpuPools(wl)
    g.write("prefix")
    g.write("new")
    return g, OraclePools(wl)


def _check(P, wl, g, o, seqs, splits, want):
    q, _ = wl.queries(0)
    q, bt = q[seqs], wl.block_tables[seqs]
    lens = wl.total_lens[seqs].astype(np.int32)
    B = len(seqs)
    method, _ = P.decode_method(B, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.page_size,
                                int(lens.max()), wl.window, splits)
    assert method == want, (method, want)        # a decomposition that uses the scratch
    say(f"[no-alloc] {wl.name}: B={B} splits={splits} ({method})")
    args = (dev_bits(q), g.k, g.v, dev_i32(bt), dev_i32(lens), int(lens.max()))
    kw = dict(page_size=wl.page_size, scale=wl.scale, window=wl.window, num_splits=splits)
    ref_gpu = host_bits(P.decode(*args, **kw))
    out = torch.full(q.shape, int(W.BF16_NAN), dtype=torch.int16, device="cuda")
    P.decode_noalloc(*args, out=out, **kw)
    torch.cuda.synchronize()
    got = host_bits(out)
    assert np.array_equal(got, ref_gpu), "no-alloc decode differs from pkv_decode"
    ref = oracle.decode(q, o.k, o.v, bt, lens, wl.page_size, wl.scale, wl.window)
    check_close(got, ref, f"no-alloc {wl.name} B={B}")


def test_decode_noalloc_consecutive_calls(P):
    # stream-K (the head_dim 256 group of 8 is cut into two virtual heads):
    # 64 windowed decoders, then 10 of them
    wl = W.make("window_shared")
    g, o = _pools(wl)
    _check(P, wl, g, o, np.arange(64), 0, "stream")
    _check(P, wl, g, o, np.arange(10), 0, "stream")
    # split-K partials in the same scratch: 32 rows in 5 splits, then 7 rows in 3
    wq = W.make("qwen3_decode")
    gq, oq = _pools(wq)
    _check(P, wq, gq, oq, np.arange(32), 5, "split")
    _check(P, wq, gq, oq, np.arange(7), 3, "split")
    # and stream-K again after split-K: the scratch keeps the last call's
    # contents, which a call must not depend on
    _check(P, wl, g, o, np.arange(40), 0, "stream")
