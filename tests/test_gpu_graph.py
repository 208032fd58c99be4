"""Step graphs: a decode step (fused addressing + append, stream-K decode,
merge) captured once per batch-size bucket and replayed with new inputs.
Every replay is checked bit for bit against the same calls run eagerly on a
second set of buffers, and against the oracle; eager host-to-device copies
and synchronisations run between the replays.  Padded rows (seq_len 0, no
new token) must come out zero and leave the pool untouched."""
import zlib

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from gpu_harness import check_close, dev_bits, host_bits, say  # noqa: E402

BUCKETS = (2, 8)
# live batch of each step; the step runs in the smallest bucket >= it
STEP_BATCHES = (5, 8, 1, 2, 7, 3)

GRAPH_SHAPES = {
    # name: (Hq, Hkv, D, page_size, window)
    "d128_g4_p32": (32, 8, 128, 32, 0),
    "d256_g8_p16_win": (8, 1, 256, 16, 100),
}


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import paged_kv_attention_mapped_amd as P
    P.lib()
    return P


class DecodeBuffers:
    """Fixed-size step inputs and outputs; a bucket uses their first rows."""

    def __init__(self, P, hq, hkv, d, ps, maxp, num_pages, window, bmax):
        dev = "cuda"
        self.P, self.hq, self.hkv, self.d, self.ps, self.window = P, hq, hkv, d, ps, window
        self.q = torch.zeros((bmax, hq, d), dtype=torch.int16, device=dev)
        self.k_new = torch.zeros((bmax, hkv, d), dtype=torch.int16, device=dev)
        self.v_new = torch.zeros((bmax, hkv, d), dtype=torch.int16, device=dev)
        self.bt = torch.zeros((bmax, maxp), dtype=torch.int32, device=dev)
        self.seq_lens = torch.zeros(bmax, dtype=torch.int32, device=dev)
        self.cu_q = torch.zeros(bmax + 1, dtype=torch.int32, device=dev)
        self.cu_k = torch.zeros(bmax + 1, dtype=torch.int32, device=dev)
        self.max_len = maxp * ps
        self.waves = {b: P.decode_stream_waves(b, hq, hkv, d, ps, self.max_len, window)
                      for b in BUCKETS}
        need = max(int(P.lib().pkv_decode_stream_workspace_bytes(n, hq, hkv, d))
                   for n in self.waves.values())
        # the fused step's workspace (whatever decomposition pkv_decode picks)
        need = max([need] + [P.decode_workspace_bytes(b, hq, d, hkv, ps, self.max_len, window)
                             for b in BUCKETS])
        self.ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def step(self, bucket, k_pool, v_pool, out, ws=None):
        """The decode step of one bucket: enqueue only, no allocation."""
        P, b = self.P, bucket
        ws = self.ws if ws is None else ws
        P.append_mapped(self.k_new[:b], self.v_new[:b], self.bt[:b], self.cu_q[:b + 1],
                        self.cu_k[:b + 1], k_pool, v_pool, page_size=self.ps, max_seqlen_q=1)
        P.decode_stream(self.q[:b], k_pool, v_pool, self.bt[:b], self.seq_lens[:b],
                        page_size=self.ps, num_waves=self.waves[b], window=self.window,
                        workspace=ws, out=out[:b])
        P.decode_stream_merge(ws, out[:b], num_waves=self.waves[b], num_kv_heads=self.hkv)


    def fused_step(self, bucket, k_pool, v_pool, out, ws=None):
        """The decode step with the append fused into the decode launch."""
        P, b = self.P, bucket
        ws = self.ws if ws is None else ws
        P.decode_append(self.q[:b], self.k_new[:b], self.v_new[:b], k_pool, v_pool, self.bt[:b],
                        self.seq_lens[:b], self.max_len, page_size=self.ps, window=self.window,
                        workspace=ws, out=out[:b])

    def kernel_nodes(self, bucket, fused):
        if not fused:
            return 3                                  # append, stream-K decode, merge
        m, _ = self.P.decode_method(bucket, self.hq, self.hkv, self.d, self.ps, self.max_len,
                                    self.window)
        return {"direct": 1, "stream": 2, "split": 2}[m]


@pytest.mark.parametrize("fused", [False, True], ids=["append_then_stream", "fused_append"])
@pytest.mark.parametrize("name", sorted(GRAPH_SHAPES))
def test_decode_step_graph_buckets(P, name, fused):
    hq, hkv, d, ps, window = GRAPH_SHAPES[name]
    bmax, maxp = max(BUCKETS), 12
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    num_pages = bmax * maxp + 4
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = perm[:bmax * maxp].reshape(bmax, maxp)
    scale = 1.0 / np.sqrt(d)

    # cached context of every sequence, written on the host through the oracle
    lens = rng.integers(0, maxp * ps - len(STEP_BATCHES) - 1, bmax, endpoint=True)
    lens[1] = 0                                       # a sequence that starts empty
    shape = (hkv, num_pages * ps, d)
    ok = np.full(shape, W.BF16_NAN, np.uint16)
    ov = np.full(shape, W.BF16_NAN, np.uint16)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    kc = W.bf16_bits(rng.standard_normal((int(cu[-1]), hkv, d), dtype=np.float32))
    vc = W.bf16_bits(rng.standard_normal((int(cu[-1]), hkv, d), dtype=np.float32))
    ok, ov = oracle.append(ok, ov, kc, vc, oracle.slot_mapping(bt, cu, cu, ps))

    # graph pools and eager pools start from the same bits
    gk, gv = dev_bits(ok), dev_bits(ov)
    ek, ev = dev_bits(ok), dev_bits(ov)
    buf = DecodeBuffers(P, hq, hkv, d, ps, maxp, num_pages, window, bmax)
    buf.bt.copy_(torch.from_numpy(bt).cuda())
    g_out = torch.zeros((bmax, hq, d), dtype=torch.bfloat16, device="cuda")
    e_out = torch.zeros_like(g_out)
    e_ws = torch.empty_like(buf.ws)

    step = buf.fused_step if fused else buf.step
    s = torch.cuda.Stream()
    graphs = {}
    with torch.cuda.stream(s):
        for b in BUCKETS:   # warm-up launch before capture (zero-length rows, no tokens)
            step(b, gk, gv, g_out)
        s.synchronize()
        for b in BUCKETS:
            graphs[b] = P.capture_graph(lambda b=b: step(b, gk, gv, g_out), s)
            # kernels only; with the fused append no separate append node
            assert graphs[b].nodes() == (buf.kernel_nodes(b, fused), 0), graphs[b].nodes()

    for i, B in enumerate(STEP_BATCHES):
        bucket = min(b for b in BUCKETS if b >= B)
        say(f"[graph] {name} fused={fused} step {i}: live batch {B} in bucket {bucket}")
        # this step's inputs: live rows 0..B-1 get one new token; padded rows none
        q = W.bf16_bits(rng.standard_normal((bmax, hq, d), dtype=np.float32))
        kn = W.bf16_bits(rng.standard_normal((bmax, hkv, d), dtype=np.float32))
        vn = W.bf16_bits(rng.standard_normal((bmax, hkv, d), dtype=np.float32))
        sl = np.zeros(bmax, np.int64)
        sl[:B] = lens[:B] + 1
        cq = np.minimum(np.arange(bmax + 1), B)
        ck = np.concatenate([[0], np.cumsum(sl)])
        with torch.cuda.stream(s):
            for t, a in ((buf.q, q), (buf.k_new, kn), (buf.v_new, vn)):
                t.copy_(torch.from_numpy(a.view(np.int16)).cuda())
            buf.seq_lens.copy_(torch.from_numpy(sl.astype(np.int32)).cuda())
            buf.cu_q.copy_(torch.from_numpy(cq.astype(np.int32)).cuda())
            buf.cu_k.copy_(torch.from_numpy(ck.astype(np.int32)).cuda())
            g_out.fill_(1.0)
            e_out.fill_(1.0)
            graphs[bucket].launch(s)
            step(bucket, ek, ev, e_out, ws=e_ws)   # the same calls, eagerly
        s.synchronize()

        # graph replay == eager, bit for bit (outputs and pools)
        assert torch.equal(g_out[:bucket], e_out[:bucket])
        assert torch.equal(gk, ek) and torch.equal(gv, ev)
        # oracle: append the live rows' tokens, then decode them
        slots = oracle.slot_mapping(bt[:B], cq[:B + 1], ck[:B + 1], ps)
        ok, ov = oracle.append(ok, ov, kn[:B], vn[:B], slots)
        assert np.array_equal(host_bits(gk), ok) and np.array_equal(host_bits(gv), ov)
        ref = oracle.decode(q[:B], ok, ov, bt[:B], sl[:B], ps, scale, window)
        got = host_bits(g_out)
        check_close(got[:B], ref, f"{name} step {i}")
        assert np.all(got[B:bucket] == 0)                      # padded rows
        lens[:B] += 1

    for gr in graphs.values():
        gr.destroy()


def test_mixed_step_graph_replays(P):
    """A mixed step (fused append of every new row, then decode rows and a
    chunk in one varlen launch) captured once and replayed with new queries
    and new rows: each replay equals the eager calls bit for bit and the oracle
    within the bar.  Prefill launches size their grid from host bounds only,
    so they are replay-safe like the decode launches."""
    hq, hkv, d, ps = 8, 2, 128, 16
    rng = np.random.default_rng(4242)
    nseq, maxp = 5, 16
    num_pages = nseq * maxp
    bt = rng.permutation(num_pages).astype(np.int32).reshape(nseq, maxp)
    prefix = np.array([40, 0, 100, 7, 60])
    new = np.array([1, 1, 1, 33, 1])          # four decode rows and a 33-row chunk
    total = prefix + new
    scale = 1.0 / np.sqrt(d)
    shape = (hkv, num_pages * ps, d)
    ok = np.full(shape, W.BF16_NAN, np.uint16)
    ov = np.full(shape, W.BF16_NAN, np.uint16)
    cu_p = np.concatenate([[0], np.cumsum(prefix)])
    kc = W.bf16_bits(rng.standard_normal((int(cu_p[-1]), hkv, d), dtype=np.float32))
    vc = W.bf16_bits(rng.standard_normal((int(cu_p[-1]), hkv, d), dtype=np.float32))
    ok, ov = oracle.append(ok, ov, kc, vc, oracle.slot_mapping(bt, cu_p, cu_p, ps))
    gk, gv, ek, ev = dev_bits(ok), dev_bits(ov), dev_bits(ok), dev_bits(ov)
    T = int(new.sum())
    cq_h = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    ck_h = np.concatenate([[0], np.cumsum(total)]).astype(np.int32)
    q = torch.zeros((T, hq, d), dtype=torch.int16, device="cuda")
    kn = torch.zeros((T, hkv, d), dtype=torch.int16, device="cuda")
    vn = torch.zeros((T, hkv, d), dtype=torch.int16, device="cuda")
    d_bt = torch.from_numpy(bt).cuda()
    cq = torch.from_numpy(cq_h).cuda()
    ck = torch.from_numpy(ck_h).cuda()
    g_out = torch.zeros((T, hq, d), dtype=torch.bfloat16, device="cuda")
    e_out = torch.zeros_like(g_out)

    def step(kp, vp, out):
        P.append_mapped(kn, vn, d_bt, cq, ck, kp, vp, page_size=ps, max_seqlen_q=int(new.max()))
        P.prefill_varlen(q, kp, vp, d_bt, cq, ck, int(new.max()), int(total.max()),
                         page_size=ps, scale=scale, out=out)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step(gk, gv, g_out)          # warm-up launch before capture
        s.synchronize()
        graph = P.capture_graph(lambda: step(gk, gv, g_out), s)
    assert graph.nodes() == (2, 0)
    for i in range(4):
        qh = W.bf16_bits(rng.standard_normal((T, hq, d), dtype=np.float32))
        knh = W.bf16_bits(rng.standard_normal((T, hkv, d), dtype=np.float32))
        vnh = W.bf16_bits(rng.standard_normal((T, hkv, d), dtype=np.float32))
        with torch.cuda.stream(s):
            q.copy_(dev_bits(qh)); kn.copy_(dev_bits(knh)); vn.copy_(dev_bits(vnh))
            g_out.fill_(5.0)
            e_out.fill_(5.0)
            graph.launch(s)
            step(ek, ev, e_out)
        s.synchronize()
        say(f"[graph] mixed step replay {i}")
        assert torch.equal(g_out, e_out)
        assert torch.equal(gk, ek) and torch.equal(gv, ev)
        ok, ov = oracle.append(ok, ov, knh, vnh, oracle.slot_mapping(bt, cq_h, ck_h, ps))
        assert np.array_equal(host_bits(gk), ok) and np.array_equal(host_bits(gv), ov)
        ref = oracle.prefill_varlen(qh, ok, ov, bt, cq_h, ck_h, ps, scale)
        check_close(host_bits(g_out), ref, f"mixed step replay {i}")
    graph.destroy()
