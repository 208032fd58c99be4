"""Device page allocator against the oracle allocator, bit for bit (tables,
free stack, count, status), and a captured decode step that allocates its
own pages on the device as sequences cross page boundaries."""
import os
import zlib

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from gpu_harness import check_close, dev_bits, dev_i32, host_bits, say  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_alloc.txt")


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import paged_kv_attention_mapped_amd as P
    P.lib()
    return P


class DevState:
    """Block tables, free stack, count and status on the GPU."""

    def __init__(self, bt, free, count):
        self.bt = dev_i32(bt)
        self.free = dev_i32(free)
        self.count = dev_i32([count])
        self.status = dev_i32([-9])

    def host(self):
        torch.cuda.synchronize()
        return (self.bt.cpu().numpy().astype(np.int64), self.free.cpu().numpy().astype(np.int64),
                int(self.count.item()), int(self.status.item()))


def check_same(dev, ref, what):
    bt, free, count, st = dev.host()
    rbt, rfree, rcount, rst = ref
    assert st == rst, (what, st, rst)
    assert count == rcount, (what, count, rcount)
    assert np.array_equal(bt, rbt), what
    assert np.array_equal(free[:count], rfree[:count]), what


def run_op(P, dev, ref, op, ps, num_pages):
    bt, free, count, _ = ref
    if op[0] == "alloc":
        cq, ck = op[1], op[2]
        ref = oracle.page_alloc(cq, ck, bt, free, count, ps)
        P.page_alloc(dev_i32(cq), dev_i32(ck), dev.bt, dev.free, dev.count, page_size=ps,
                     status=dev.status)
    else:
        lens, rel = op[1], op[2]
        ref = oracle.page_free(lens, rel, bt, free, count, ps, num_pages)
        P.page_free(dev_i32(lens), dev_i32(rel), dev.bt, dev.free, dev.count, page_size=ps,
                    status=dev.status)
    check_same(dev, ref, op[0])
    return ref


def test_allocator_worked_example(P):
    lines = [ln.split("#", 1)[0].strip() for ln in open(GOLDEN)]
    lines = [ln for ln in lines if ln]
    hdr = {}
    while "/" not in lines[0]:
        k, v = lines.pop(0).split(" ", 1)
        hdr[k] = [int(x) for x in v.split()]
    ps, num_pages = hdr["page_size"][0], hdr["num_pages"][0]
    nseq, width = hdr["table"]
    bt = np.full((nseq, width), -1, np.int64)
    free = np.array(hdr["free"], np.int64)
    ref = (bt, free, len(free), 0)
    dev = DevState(bt, free, len(free))
    for op in lines[0::2]:
        name, rest = op.split(" ", 1)
        a, b = [np.array([int(x) for x in t.split()], np.int64) for t in rest.split("/")]
        if name == "alloc":
            op_t = ("alloc", np.concatenate([[0], np.cumsum(a)]), np.concatenate([[0], np.cumsum(b)]))
        else:
            op_t = ("free", a, b)
        say(f"[alloc] worked example: {op}")
        ref = run_op(P, dev, ref, op_t, ps, num_pages)


@pytest.mark.parametrize("nseq,width,num_pages", [(7, 5, 24), (2500, 3, 6000)])
def test_allocator_random_vs_oracle(P, nseq, width, num_pages):
    """Random alloc/free sequences; 2500 sequences span several scan chunks."""
    rng = np.random.default_rng(zlib.crc32(f"{nseq}".encode()))
    ps = 16
    bt = np.full((nseq, width), -1, np.int64)
    free = rng.permutation(num_pages).astype(np.int64)
    ref = (bt, free, num_pages, 0)
    dev = DevState(bt, free, num_pages)
    lens = np.zeros(nseq, np.int64)
    say(f"[alloc] random: {nseq} sequences, {width}-entry rows, {num_pages} pages")
    for step in range(24):
        if rng.random() < 0.65:
            lq = rng.integers(0, 24, nseq) * (rng.random(nseq) < 0.6)
            if step % 7 == 6:
                lq[rng.integers(nseq)] = width * ps + 1          # forces status 1
            lk = lens + lq
            op = ("alloc", np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)]))
            ref = run_op(P, dev, ref, op, ps, num_pages)
            if ref[3] == oracle.ALLOC_OK:
                lens = lk
        else:
            rel = (rng.random(nseq) < 0.3).astype(np.int64)
            ref = run_op(P, dev, ref, ("free", lens, rel), ps, num_pages)
            lens = np.where(rel.astype(bool), 0, lens)


def test_decode_graph_allocates_pages(P):
    """Step graph = page alloc + fused append + decode; sequences grow one token
    per replay and cross page boundaries, the pages coming from the device stack."""
    hq, hkv, d, ps, nseq, width = 8, 2, 128, 16, 6, 8
    num_pages = nseq * width
    rng = np.random.default_rng(77)
    scale = 1.0 / np.sqrt(d)
    free0 = rng.permutation(num_pages).astype(np.int64)
    # prompts written eagerly through the oracle allocator and the oracle append
    lens = rng.integers(10, 40, nseq)
    lens[2] = 0                                          # an empty sequence
    bt = np.full((nseq, width), -1, np.int64)
    cu = np.concatenate([[0], np.cumsum(lens)])
    bt, free, count, st = oracle.page_alloc(cu, cu, bt, free0, num_pages, ps)
    assert st == 0
    shape = (hkv, num_pages * ps, d)
    ok = np.full(shape, W.BF16_NAN, np.uint16)
    ov = np.full(shape, W.BF16_NAN, np.uint16)
    kc = W.bf16_bits(rng.standard_normal((int(cu[-1]), hkv, d), dtype=np.float32))
    vc = W.bf16_bits(rng.standard_normal((int(cu[-1]), hkv, d), dtype=np.float32))
    ok, ov = oracle.append(ok, ov, kc, vc, oracle.slot_mapping(bt, cu, cu, ps))

    dev = DevState(bt, free, count)
    kp, vp = dev_bits(ok), dev_bits(ov)
    q = torch.zeros((nseq, hq, d), dtype=torch.int16, device="cuda")
    kn = torch.zeros((nseq, hkv, d), dtype=torch.int16, device="cuda")
    vn = torch.zeros((nseq, hkv, d), dtype=torch.int16, device="cuda")
    cq = dev_i32(np.arange(nseq + 1))
    ck = torch.zeros(nseq + 1, dtype=torch.int32, device="cuda")
    sl = torch.zeros(nseq, dtype=torch.int32, device="cuda")
    out = torch.zeros((nseq, hq, d), dtype=torch.bfloat16, device="cuda")
    assert P.decode_method(nseq, hq, hkv, d, ps, width * ps)[0] == "direct"

    def step():
        P.page_alloc(cq, ck, dev.bt, dev.free, dev.count, page_size=ps, status=dev.status)
        P.append_mapped(kn, vn, dev.bt, cq, ck, kp, vp, page_size=ps, max_seqlen_q=1)
        P.decode(q, kp, vp, dev.bt, sl, width * ps, page_size=ps, scale=scale, out=out)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        graph = P.capture_graph(step, s)
    assert graph.nodes() == (3, 0)
    ref = (bt, free, count, 0)
    for i in range(20):
        qh = W.bf16_bits(rng.standard_normal((nseq, hq, d), dtype=np.float32))
        knh = W.bf16_bits(rng.standard_normal((nseq, hkv, d), dtype=np.float32))
        vnh = W.bf16_bits(rng.standard_normal((nseq, hkv, d), dtype=np.float32))
        new = lens + 1
        with torch.cuda.stream(s):
            q.copy_(dev_bits(qh)); kn.copy_(dev_bits(knh)); vn.copy_(dev_bits(vnh))
            ck.copy_(dev_i32(np.concatenate([[0], np.cumsum(new)])))
            sl.copy_(dev_i32(new))
            out.fill_(3.0)
            graph.launch(s)
        s.synchronize()
        # oracle: the same allocation, append and decode
        cqh = np.arange(nseq + 1)
        ckh = np.concatenate([[0], np.cumsum(new)])
        ref = oracle.page_alloc(cqh, ckh, ref[0], ref[1], ref[2], ps)
        assert ref[3] == 0
        check_same(dev, ref, f"replay {i}")
        ok, ov = oracle.append(ok, ov, knh, vnh, oracle.slot_mapping(ref[0], cqh, ckh, ps))
        assert np.array_equal(host_bits(kp), ok) and np.array_equal(host_bits(vp), ov)
        refo = oracle.decode(qh, ok, ov, ref[0], new, ps, scale)
        check_close(host_bits(out), refo, f"allocating step {i}")
        lens = new
    graph.destroy()
