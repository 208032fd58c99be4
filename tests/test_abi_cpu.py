"""The C ABI on the host: the library loads, exports every declared entry
point, and rejects bad arguments before anything reaches the GPU.  No call
here enqueues GPU work (every case returns during host validation)."""
import ctypes
import os
import re

import pytest

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


@pytest.fixture(scope="module")
def P():
    import paged_kv_attention_mapped_amd as P
    if not os.path.exists(P.lib_path()):
        from paged_kv_attention_mapped_amd import build
        build.build()
    P.lib()
    return P


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:pkv_status|size_t|const char\*)\s+(pkv_\w+)\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert declared() == sorted([
        "pkv_append", "pkv_append_mapped", "pkv_decode", "pkv_decode_append", "pkv_decode_combine", "pkv_decode_noalloc",
        "pkv_decode_method", "pkv_decode_plan", "pkv_decode_split",
        "pkv_device_info", "pkv_graph_begin", "pkv_graph_destroy", "pkv_graph_end",
        "pkv_graph_launch", "pkv_graph_nodes", "pkv_page_alloc", "pkv_page_free",
        "pkv_decode_stream", "pkv_decode_stream_merge", "pkv_decode_stream_waves",
        "pkv_decode_stream_workspace_bytes", "pkv_decode_workspace_bytes", "pkv_prefill_varlen",
        "pkv_prefill_split_workspace_bytes", "pkv_prefill_varlen_split",
        "pkv_slot_mapping", "pkv_status_string", "pkv_stream_read"])


def test_library_exports_every_declared_symbol(P):
    lib = P.lib()
    for name in declared():
        assert hasattr(lib, name), name
    assert sorted(P.exported_symbols()) == declared()


def test_status_strings(P):
    s = P.lib().pkv_status_string
    assert s(0) == b"ok"
    assert s(1) == b"null argument"
    assert s(3) == b"unsupported configuration"
    assert s(4) == b"workspace too small"
    assert s(99) == b"unknown status"


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails validation first


def _decode(P, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, maxp=4, lens=FAKE, B=2, hq=8, hkv=2, d=128, ps=32,
             pages=10, maxlen=100, scale=1.0, window=0, splits=0, ws=None, wsb=0, out=FAKE)
    a.update(kw)
    return P.lib().pkv_decode(a["q"], a["k"], a["v"], a["bt"], a["maxp"], a["lens"], a["B"],
                              a["hq"], a["hkv"], a["d"], a["ps"], a["pages"], a["maxlen"],
                              a["scale"], a["window"], a["splits"], a["ws"], a["wsb"], a["out"],
                              None)


def test_decode_validation(P):
    assert _decode(P, q=None) == 1
    assert _decode(P, d=96) == 3
    assert _decode(P, ps=8) == 3
    assert _decode(P, hq=6, hkv=4) == 2
    assert _decode(P, hq=32, hkv=2) == 3   # group 16 is not built
    assert _decode(P, B=-1) == 2
    assert _decode(P, maxp=0) == 2
    # 2 splits requested: needs a workspace
    assert _decode(P, splits=2, ws=None) == 1
    assert _decode(P, splits=2, ws=FAKE, wsb=16) == 4
    assert _decode(P, B=0) == 0            # empty batch: nothing to do


def _decode_append(P, **kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, k=FAKE, v=FAKE, bt=FAKE, maxp=4, lens=FAKE, B=2, hq=8,
             hkv=2, d=128, ps=32, pages=10, maxlen=100, scale=1.0, window=0, splits=0, ws=None,
             wsb=0, out=FAKE)
    a.update(kw)
    return P.lib().pkv_decode_append(a["q"], a["kn"], a["vn"], a["k"], a["v"], a["bt"], a["maxp"],
                                     a["lens"], a["B"], a["hq"], a["hkv"], a["d"], a["ps"],
                                     a["pages"], a["maxlen"], a["scale"], a["window"], a["splits"],
                                     a["ws"], a["wsb"], a["out"], None)


def test_decode_append_validation(P):
    # the decode checks, plus the new rows
    assert _decode_append(P, kn=None) == 1
    assert _decode_append(P, vn=None) == 1
    assert _decode_append(P, q=None) == 1
    assert _decode_append(P, out=None) == 1
    assert _decode_append(P, d=96) == 3
    assert _decode_append(P, hq=6, hkv=4) == 2
    assert _decode_append(P, splits=2, ws=None) == 1
    assert _decode_append(P, splits=2, ws=FAKE, wsb=16) == 4
    assert _decode_append(P, ps=32, pages=1 << 26) == 2     # slots past 2^31
    assert _decode_append(P, B=0, kn=None, vn=None) == 0   # empty batch: nothing to do


def test_decode_noalloc_validation(P):
    L = P.lib()

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, maxp=4, lens=FAKE, B=2, hq=8, hkv=2, d=128,
                 ps=32, pages=10, maxlen=100, scale=1.0, window=0, splits=0, out=FAKE)
        a.update(kw)
        return L.pkv_decode_noalloc(a["q"], a["k"], a["v"], a["bt"], a["maxp"], a["lens"], a["B"],
                                    a["hq"], a["hkv"], a["d"], a["ps"], a["pages"], a["maxlen"],
                                    a["scale"], a["window"], a["splits"], a["out"], None)
    assert call(q=None) == 1
    assert call(d=96) == 3
    assert call(B=-1) == 2
    assert call(splits=-1) == 2
    assert call(B=0) == 0
    # partials beyond the 16 MiB scratch are refused before any HIP call:
    # 4096 rows x 32 heads x 64 splits x 130 floats
    assert P.decode_workspace_bytes(4096, 32, 128, 8, 32, 65536, 0, 64) > 16 << 20
    assert call(B=4096, hq=32, hkv=8, maxp=2048, maxlen=65536, splits=64) == 4


def test_prefill_and_append_validation(P):
    L = P.lib()
    f = L.pkv_prefill_varlen
    args = [FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, 2, 10, 8, 8, 8, 2, 128, 32, 10, 1.0, 0, FAKE, None]
    a = list(args); a[0] = None
    assert f(*a) == 1
    a = list(args); a[13] = 80
    assert f(*a) == 3
    a = list(args); a[11] = 7
    assert f(*a) == 2
    a = list(args); a[8] = 0
    assert f(*a) == 0
    assert L.pkv_append(None, FAKE, FAKE, 4, 2, 128, FAKE, FAKE, 100, None) == 1
    assert L.pkv_append(FAKE, FAKE, FAKE, 4, 2, 100, FAKE, FAKE, 100, None) == 3
    assert L.pkv_append(FAKE, FAKE, FAKE, 0, 2, 128, FAKE, FAKE, 100, None) == 0
    assert L.pkv_slot_mapping(None, 4, FAKE, FAKE, 2, 5, 32, 10, FAKE, None) == 1
    assert L.pkv_slot_mapping(FAKE, 4, FAKE, FAKE, 2, 0, 32, 10, FAKE, None) == 0
    assert L.pkv_decode_combine(FAKE, FAKE, FAKE, 2, 8, 128, 0, FAKE, None) == 2
    assert L.pkv_decode_split(FAKE, FAKE, FAKE, FAKE, 4, FAKE, 2, 8, 2, 128, 32, 10, 1000, 1.0,
                              0, 2, 4, FAKE, FAKE, FAKE, None) == 2   # 2*4 pages < 32 needed


def test_decode_plan(P):
    # the workload shapes: (B, Hkv, ps, max_seq_len, window) -> splits cover every key page
    for B, hkv, ps, L, w in [(256, 8, 32, 8193, 0), (32, 8, 32, 1025, 0), (4, 1, 16, 64, 0),
                             (64, 1, 32, 4097, 512), (56, 8, 32, 2049, 0), (1, 1, 16, 1, 0)]:
        s, pps = P.decode_plan(B, hkv, ps, L, w)
        pages = -(-L // ps)
        if w:
            pages = min(pages, -(-(w - 1) // ps) + 1)
        assert s * pps >= pages and (s - 1) * pps < pages
        need = P.decode_workspace_bytes(B, hkv * 4, 128, hkv, ps, L, w, s)
        assert need == (0 if s == 1 else B * hkv * 4 * s * 130 * 4)
    assert P.decode_plan(256, 8, 32, 8193) == (9, 32)
    # stream-K: waves bounded by the work and by the device (256 CUs assumed without a GPU)
    assert P.decode_stream_waves(4, 2, 1, 64, 16, 64) == 4
    assert P.decode_stream_waves(256, 32, 8, 128, 32, 8193) == 256 * 4 * 2
    nw = P.decode_stream_waves(256, 32, 8, 128, 32, 8193)
    # a window of 512 keys touches at most 17 pages of 32: 64 rows x 1 KV head x 17 = 1088
    # units; a group of 8 with head_dim >= 128 counts each KV head twice; >= 4 units per wave
    assert P.decode_stream_waves(64, 8, 1, 256, 32, 4096, 512) == 2 * 1088 // 4
    assert P.decode_stream_waves(64, 8, 1, 64, 32, 4096, 512) == 1088 // 4
    assert P.decode_workspace_bytes(256, 32, 128, 8, 32, 8193) == \
        P.lib().pkv_decode_stream_workspace_bytes(nw, 32, 8, 128)
    assert P.decode_plan(4, 8, 32, 1000, 0, 7) == (7, 5)
    assert P.decode_plan(4, 8, 32, 1000, 0, 1)[0] == 1


def test_stream_read_validation(P):
    f = P.lib().pkv_stream_read
    assert f(FAKE, 100, 4, FAKE, None) == 2          # not a multiple of 16
    assert f(FAKE, 1024, 0, FAKE, None) == 2         # no workgroups
    assert f(None, 1024, 4, FAKE, None) == 1
    assert f(FAKE, 1024, 4, None, None) == 1
    assert f(None, 0, 4, None, None) == 0            # nothing to read


def test_device_info_rejects_null(P):
    # validation happens before any runtime query, so this needs no GPU
    assert P.lib().pkv_device_info(None, None) == 1


def test_append_mapped_validation(P):
    f = P.lib().pkv_append_mapped
    args = [FAKE, FAKE, FAKE, 4, FAKE, FAKE, 2, 5, 3, 32, 10, 2, 128, FAKE, FAKE, None, None]
    a = list(args); a[0] = None
    assert f(*a) == 1
    a = list(args); a[2] = None
    assert f(*a) == 1
    a = list(args); a[12] = 96
    assert f(*a) == 3
    a = list(args); a[3] = 0
    assert f(*a) == 2
    a = list(args); a[10] = 0
    assert f(*a) == 2
    a = list(args); a[8] = -1
    assert f(*a) == 2
    a = list(args); a[9] = 1 << 20; a[10] = 1 << 12  # pool of 2^32 slots does not fit int32
    assert f(*a) == 2
    a = list(args); a[8] = 1 << 26                   # 2^26 rows x 32 chunks >= 2^31
    assert f(*a) == 2
    a = list(args); a[7] = 0; a[0] = None            # no tokens: nothing to check or enqueue
    assert f(*a) == 0
    a = list(args); a[8] = 0; a[0] = None            # no rows per sequence
    assert f(*a) == 0
    a = list(args); a[6] = 0
    assert f(*a) == 0


def test_graph_validation(P):
    L = P.lib()
    h = ctypes.c_void_p(None)
    assert L.pkv_graph_begin(None) == 1              # the null stream cannot be captured
    assert L.pkv_graph_end(None, ctypes.byref(h)) == 1
    assert L.pkv_graph_end(FAKE, None) == 1
    assert L.pkv_graph_launch(None, None) == 1
    k, o = ctypes.c_int32(0), ctypes.c_int32(0)
    assert L.pkv_graph_nodes(None, ctypes.byref(k), ctypes.byref(o)) == 1
    assert L.pkv_graph_destroy(None) == 0
    with pytest.raises(ValueError):
        P.capture_graph(lambda: None, None)


def test_decode_method(P):
    # small batches: one kernel, one workgroup per (sequence, KV head) row
    assert P.decode_method(4, 2, 1, 64, 16, 64) == ("direct", 1)
    assert P.decode_method(32, 32, 8, 128, 32, 1025) == ("direct", 1)      # 256 rows
    assert P.lib().pkv_decode_workspace_bytes(32, 32, 128, 8, 32, 1025, 0, 0) == 0
    # larger batches, or a group that stream-K splits in two: stream-K
    assert P.decode_method(56, 32, 8, 128, 32, 2049) == \
        ("stream", P.decode_stream_waves(56, 32, 8, 128, 32, 2049))
    assert P.decode_method(64, 8, 1, 256, 32, 4097, 512)[0] == "stream"
    assert P.decode_method(256, 32, 8, 128, 32, 8193) == ("stream", 2048)
    # past the stream-K row limit, or when splits are asked for: split-K
    assert P.decode_method(4096, 32, 8, 128, 32, 8192) == ("split", 8)   # 32-page splits
    assert P.decode_method(4096, 32, 8, 128, 32, 1024) == ("direct", 1)  # one split suffices
    assert P.decode_method(4, 8, 2, 128, 32, 1000, 0, 3) == ("split", 3)
    assert P.decode_method(4, 8, 2, 128, 32, 1000, 0, 1) == ("direct", 1)
    assert P.lib().pkv_decode_method(4, 8, 2, 96, 32, 100, 0, 0, None, None) == 3
    assert P.lib().pkv_decode_method(4, 8, 3, 128, 32, 100, 0, 0, None, None) == 2


def test_page_allocator_validation(P):
    L = P.lib()
    a = [FAKE, FAKE, 3, FAKE, 4, 16, FAKE, FAKE, 32, None, None]
    for i, code in ((0, 1), (3, 1), (6, 1), (7, 1)):
        b = list(a); b[i] = None
        assert L.pkv_page_alloc(*b) == code
        assert L.pkv_page_free(*b) == code
    for i, v in ((2, -1), (4, 0), (5, 0), (8, 0)):
        b = list(a); b[i] = v
        assert L.pkv_page_alloc(*b) == 2
        assert L.pkv_page_free(*b) == 2
    b = list(a); b[2] = 0; b[0] = None      # no sequences: nothing to do
    assert L.pkv_page_alloc(*b) == 0 and L.pkv_page_free(*b) == 0


def test_head_dim_512_plans(P):
    # head_dim 512 streams over workgroups (one per compute unit; 256 assumed
    # without a GPU), its units being 32-key tiles, at least 4 per workgroup
    assert P.decode_method(4, 8, 1, 512, 32, 100) == ("stream", 4)        # 4 rows x 4 tiles
    assert P.decode_method(256, 8, 1, 512, 32, 8192) == ("stream", 256)
    assert P.decode_method(16, 8, 1, 512, 16, 4096, 512) == ("stream", 16 * 17 // 4)  # window: 17 tiles
    # splits asked for: split-K with that many splits
    assert P.decode_method(256, 8, 1, 512, 32, 8192, 0, 4) == ("split", 4)
    parts = (2 * 256 * 8 * 514 * 4 + 255) // 256 * 256
    assert P.decode_workspace_bytes(256, 8, 512, 1, 32, 8192) == parts + 2 * 256 * 8 * 4
    assert P.lib().pkv_decode_stream_workspace_bytes(8, 8, 1, 512) > 0


def test_prefill_split_validation(P):
    L = P.lib()
    # workspace: two 256-byte aligned [Tq, Hq, S] float arrays, [Tq, Hq, S, D] floats
    # (256-byte aligned), then the [Tq] int32 split counts of the rows
    cells = 576 * 8 * 4
    assert L.pkv_prefill_split_workspace_bytes(576, 8, 256, 4) == (
        2 * ((cells * 4 + 255) // 256 * 256) + cells * 256 * 4 + 576 * 4)
    assert L.pkv_prefill_split_workspace_bytes(576, 8, 256, 1) == 0
    assert L.pkv_prefill_split_workspace_bytes(0, 8, 256, 4) == 0
    need = L.pkv_prefill_split_workspace_bytes(100, 8, 128, 3)
    # q, k, v, bt, max_pages, cu_q, cu_k, N, Tq, max_q, max_k, Hq, Hkv, D, ps, P, scale, W, S, ws, ws_bytes, out, stream
    args = [FAKE, FAKE, FAKE, FAKE, 8, FAKE, FAKE, 2, 100, 60, 200, 8, 2, 128, 32, 64, 0.1, 0, 3,
            FAKE, need, FAKE, None]
    f = L.pkv_prefill_varlen_split
    for s_bad in (0, -1, 65):
        a = list(args); a[18] = s_bad
        assert f(*a) == 2
    a = list(args); a[13] = 512                        # head_dim 512 is not split
    assert f(*a) == 3
    a = list(args); a[19] = None                       # splitting needs the workspace
    assert f(*a) == 1
    a = list(args); a[20] = need - 1
    assert f(*a) == 4
    a = list(args); a[8] = 0; a[0] = None              # no rows: nothing to check or enqueue
    assert f(*a) == 0
