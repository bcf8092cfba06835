"""The C ABI on the host, without a GPU: libengram.so loads, exports every
function include/engram.h declares, and refuses bad arguments before any
launch (metrale "engram_v41" module index, invariants: refusals happen before
any copy or launch).  Every call here is refused by the host checks, so no
kernel is launched; fake device addresses are never dereferenced."""
import ctypes
import os
import re

import numpy as np
import pytest

import gram_hashed_embedding_engram_amd as E

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "engram.h")
FAKE = 0x7F0000000000          # 256-byte aligned stand-in for device memory


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(E.LIB_PATH):
        import gram_hashed_embedding_engram_amd.build as B
        B.build()
    return E.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(engram_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(L, n), n
    assert sorted(E.EXPORTS) == names
    assert L.engram_abi_version() == 7 == E.ABI_VERSION
    assert "#define ENGRAM_ABI_VERSION %d" % E.ABI_VERSION in open(HEADER).read()


def tables_c(nl=2, ng=4, nh=8, vocab=1000, mult=None, primes=None, offsets=None):
    cols = (ng - 1) * nh
    mult = np.ones((nl, ng), np.int64) * 3 if mult is None else mult
    primes = np.full((nl, cols), 101, np.int64) if primes is None else primes
    offsets = (np.arange(nl * cols, dtype=np.int64).reshape(nl, cols) * 101
               if offsets is None else offsets)
    keep = (mult, primes, offsets)
    c = E.HashTablesC(nl, ng, nh, 0, vocab, 0, FAKE, mult.ctypes.data, primes.ctypes.data,
                      offsets.ctypes.data)
    return c, keep


def rc_msg(rc):
    return rc, E.last_error()


def test_hash_refusals(L):
    c, keep = tables_c()
    call = lambda tab, T=4, start=0, max_seq=16: rc_msg(L.engram_hash(
        ctypes.byref(tab), FAKE, T, start, FAKE, max_seq, FAKE, None, None))
    rc, msg = call(c, T=10, start=8, max_seq=16)
    assert rc == E.E_RANGE and "16 positions, 10 tokens from position 8" in msg
    # positions near 2^63: refused without the sum start + T overflowing
    big = (1 << 62) + 1
    assert call(c, T=big, start=big, max_seq=1 << 62)[0] == E.E_RANGE
    assert call(c, T=2, start=(1 << 63) - 1, max_seq=(1 << 63) - 1)[0] == E.E_RANGE
    assert call(c, T=(1 << 63) - 1, start=1, max_seq=(1 << 63) - 1)[0] == E.E_RANGE
    bad, k2 = tables_c(ng=1)
    assert call(bad)[0] == E.E_ARG
    bad, k3 = tables_c(ng=9, primes=np.full((2, 64), 101, np.int64),
                       offsets=np.zeros((2, 64), np.int64), mult=np.ones((2, 9), np.int64))
    assert call(bad)[0] == E.E_UNSUPPORTED
    bad, k4 = tables_c(nl=5, mult=np.ones((5, 4), np.int64),
                       primes=np.full((5, 24), 7, np.int64), offsets=np.zeros((5, 24), np.int64))
    assert call(bad)[0] == E.E_UNSUPPORTED
    m = np.ones((2, 4), np.int64)
    m[1, 2] = -5
    bad, k5 = tables_c(mult=m)
    rc, msg = call(bad)
    assert rc == E.E_ARG and "multipliers" in msg
    p = np.full((2, 24), 101, np.int64)
    p[0, 3] = 0
    bad, k6 = tables_c(primes=p)
    rc, msg = call(bad)
    assert rc == E.E_ARG and "primes" in msg
    o = np.zeros((2, 24), np.int64)
    o[1, 1] = -1
    bad, k7 = tables_c(offsets=o)
    assert call(bad)[0] == E.E_ARG
    # NULL pointers
    assert L.engram_hash(ctypes.byref(c), None, 4, 0, FAKE, 16, FAKE, None, None) == E.E_ARG
    assert L.engram_hash(None, FAKE, 4, 0, FAKE, 16, FAKE, None, None) == E.E_ARG
    # the batched form: same checks, B = 0 or T = 0 launch nothing
    hb = lambda B, T=4, start=0, max_seq=16, ids=FAKE: L.engram_hash_batch(
        ctypes.byref(c), ids, B, T, start, FAKE, max_seq, FAKE, None, None)
    assert hb(-1) == E.E_ARG
    assert hb(3, T=10, start=8) == E.E_RANGE
    assert hb(3, ids=None) == E.E_ARG
    assert hb(0, ids=None) == E.OK and hb(3, T=0, ids=None) == E.OK


def test_map_host_refusals(L):
    # NULL host address or NULL result slot: refused before any runtime call
    out = ctypes.c_void_p(0)
    rc, msg = rc_msg(L.engram_map_host(None, ctypes.byref(out)))
    assert rc == E.E_ARG and "NULL" in msg and out.value is None
    buf = np.zeros(64, np.uint8)
    assert L.engram_map_host(buf.ctypes.data, None) == E.E_ARG


def test_stream_read_refusals(L):
    R = E.STREAM_ROW_BYTES
    assert "#define ENGRAM_STREAM_ROW_BYTES %d" % R in open(HEADER).read()
    assert "#define ENGRAM_STREAM_SINK_WORDS %d" % E.STREAM_SINK_WORDS in open(HEADER).read()
    rc, msg = rc_msg(L.engram_stream_read(FAKE, R + 4, FAKE, None))
    assert rc == E.E_ARG and "multiple" in msg
    assert L.engram_stream_read(FAKE, 0, FAKE, None) == E.E_ARG
    assert L.engram_stream_read(None, R, FAKE, None) == E.E_ARG
    assert L.engram_stream_read(FAKE, R, None, None) == E.E_ARG
    rc, msg = rc_msg(L.engram_stream_read(FAKE + 8, R, FAKE, None))
    assert rc == E.E_ARG and "misaligned" in msg


def test_gather_refusals(L):
    t = E.TableC(E.FMT_Q2K, 128, 0, 0, 100, FAKE, None)
    rc, msg = rc_msg(L.engram_gather_dequant(ctypes.byref(t), FAKE, 4, 24, 48, FAKE, None, None))
    assert rc == E.E_UNSUPPORTED and "head_dim is 256 (got 128)" in msg
    t = E.TableC(E.FMT_Q2K, 256, 0, 0, 100, FAKE + 2, None)
    assert L.engram_gather_dequant(ctypes.byref(t), FAKE, 4, 24, 48, FAKE, None, None) == E.E_ARG
    t = E.TableC(E.FMT_E4M3, 256, 100, 0, 100, FAKE, FAKE)
    assert L.engram_gather_dequant(ctypes.byref(t), FAKE, 4, 24, 48, FAKE, None,
                                   None) == E.E_UNSUPPORTED
    t = E.TableC(E.FMT_E4M3, 256, 128, 0, 100, FAKE, None)
    assert L.engram_gather_dequant(ctypes.byref(t), FAKE, 4, 24, 48, FAKE, None, None) == E.E_ARG
    t = E.TableC(7, 256, 128, 0, 100, FAKE, FAKE)
    assert L.engram_gather_dequant(ctypes.byref(t), FAKE, 4, 24, 48, FAKE, None,
                                   None) == E.E_UNSUPPORTED
    t = E.TableC(E.FMT_Q2K, 256, 0, 0, 100, FAKE, None)
    # id_stride below cols, misaligned output
    assert L.engram_gather_dequant(ctypes.byref(t), FAKE, 4, 24, 23, FAKE, None, None) == E.E_ARG
    assert L.engram_gather_dequant(ctypes.byref(t), FAKE, 4, 24, 48, FAKE + 8, None,
                                   None) == E.E_ARG
    # T = 0 is a no-op that launches nothing
    assert L.engram_gather_dequant(ctypes.byref(t), FAKE, 0, 24, 48, FAKE, None, None) == E.OK
    # row counts past 2^40 ids (T * cols would overflow) and id strides
    # wider than any hash geometry
    assert L.engram_gather_dequant(ctypes.byref(t), FAKE, 1 << 60, 24, 48, FAKE, None,
                                   None) == E.E_RANGE
    assert L.engram_gather_dequant(ctypes.byref(t), FAKE, 4, 24, 1 << 40, FAKE, None,
                                   None) == E.E_RANGE


def test_project_refusals(L):
    assert L.engram_project(FAKE, FAKE, FAKE, 4, 100, 256, None) == E.E_UNSUPPORTED
    assert L.engram_project(FAKE, FAKE, FAKE, 4, 6144, 20481, None) == E.E_UNSUPPORTED
    assert L.engram_project(FAKE, FAKE, FAKE, -1, 6144, 20480, None) == E.E_ARG
    assert L.engram_project(None, FAKE, FAKE, 4, 6144, 20480, None) == E.E_ARG
    assert L.engram_project(FAKE + 8, FAKE, FAKE, 4, 6144, 20480, None) == E.E_ARG
    assert L.engram_project(FAKE, FAKE, FAKE, 1 << 20, 1 << 14, 64, None) == E.E_UNSUPPORTED
    # token and output counts whose element counts would overflow 2^63
    assert L.engram_project(FAKE, FAKE, FAKE, (1 << 62) - 7, 64, 64, None) == E.E_UNSUPPORTED
    assert L.engram_project(FAKE, FAKE, FAKE, 4, 64, (1 << 62) - 16, None) == E.E_UNSUPPORTED
    assert L.engram_project(FAKE, FAKE, FAKE, 0, 6144, 20480, None) == E.OK


def test_project_q2k_refusals(L):
    f = L.engram_project_q2k
    assert f(FAKE, FAKE, FAKE, 2, 6144, 20480, None) == E.E_UNSUPPORTED     # one token only
    assert f(FAKE, FAKE, FAKE, 1, 6000, 20480, None) == E.E_UNSUPPORTED     # K % 256
    assert f(FAKE, FAKE, FAKE, 1, 8448, 20480, None) == E.E_UNSUPPORTED     # K > 8192
    assert f(FAKE, FAKE, FAKE, 1, 6144, 0, None) == E.E_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, -1, 6144, 20480, None) == E.E_ARG
    assert f(None, FAKE, FAKE, 1, 6144, 20480, None) == E.E_ARG
    assert f(FAKE + 8, FAKE, FAKE, 1, 6144, 20480, None) == E.E_ARG        # x 16-byte
    assert f(FAKE, FAKE + 2, FAKE, 1, 6144, 20480, None) == E.E_ARG        # blocks 4-byte
    assert f(None, None, None, 0, 6144, 20480, None) == E.OK
    d = L.engram_dequant_q2k
    assert d(FAKE, -1, FAKE, None) == E.E_ARG
    assert d(None, 3, FAKE, None) == E.E_ARG
    assert d(FAKE + 2, 3, FAKE, None) == E.E_ARG
    assert d(FAKE, 3, FAKE + 8, None) == E.E_ARG
    assert d(None, 0, None, None) == E.OK


def test_gate_refusals(L):
    f = lambda T=4, hc=4, dim=4096, eps=1e-6, h=FAKE: L.engram_gate_apply(
        h, FAKE, FAKE, T, hc, dim, ctypes.c_float(eps), None)
    assert f(hc=0) == E.E_UNSUPPORTED and f(hc=5) == E.E_UNSUPPORTED
    assert f(dim=300) == E.E_UNSUPPORTED
    assert f(eps=float("nan")) == E.E_ARG and f(eps=-1.0) == E.E_ARG
    assert f(h=None) == E.E_ARG and f(h=FAKE + 4) == E.E_ARG
    assert L.engram_qk_product(None, FAKE, FAKE, 10, None) == E.E_ARG
    assert L.engram_qk_product(FAKE, FAKE, FAKE, 0, None) == E.OK


def make_cfg(max_tokens=64, max_seq=512, hc=4, dim=4096, head_dim=256, tables=None, batch=0):
    c, keep = tables or tables_c()
    cfg = E.ConfigC(hc, head_dim, dim, 1e-6, batch, max_tokens, max_seq, c)
    return cfg, keep


def test_workspace_layout(L):
    cfg, keep = make_cfg()
    n = L.engram_workspace_bytes(ctypes.byref(cfg))
    r256 = lambda v: (v + 255) // 256 * 256
    want = (r256(8 * 512) + r256(8 * 64 * 2 * 24) + r256(2 * 64 * 24 * 256)
            + r256(2 * 64 * 4096 * 5) + 256)
    assert n == want
    bad, _ = make_cfg(max_tokens=0)
    assert L.engram_workspace_bytes(ctypes.byref(bad)) == 0
    # batch sequences: a history row each, batch*max_tokens tokens of buffers
    one, _ = make_cfg(batch=1)
    assert L.engram_workspace_bytes(ctypes.byref(one)) == want
    b3, _ = make_cfg(batch=3)
    assert L.engram_workspace_bytes(ctypes.byref(b3)) == (
        r256(8 * 512 * 3) + r256(8 * 192 * 2 * 24) + r256(2 * 192 * 24 * 256)
        + r256(2 * 192 * 4096 * 5) + 256)
    for bad_batch in (-1, 4097):
        bad, _ = make_cfg(batch=bad_batch)
        assert L.engram_workspace_bytes(ctypes.byref(bad)) == 0
    # sizes whose byte counts would overflow 2^64 are refused, not wrapped
    for kw in ({"max_seq": 1 << 61}, {"max_tokens": 1 << 60}, {"dim": 1 << 40},
               {"batch": 4096, "max_seq": 1 << 30}, {"batch": 4096, "max_tokens": 1 << 20}):
        bad, _ = make_cfg(**kw)
        assert L.engram_workspace_bytes(ctypes.byref(bad)) == 0, kw


def test_context_refusals_and_state(L):
    cfg, keep = make_cfg()
    n = L.engram_workspace_bytes(ctypes.byref(cfg))
    h = ctypes.c_void_p()
    assert L.engram_ctx_create(ctypes.byref(cfg), FAKE, n - 1, ctypes.byref(h)) == E.E_RANGE
    assert L.engram_ctx_create(ctypes.byref(cfg), FAKE + 16, n, ctypes.byref(h)) == E.E_ARG
    bad, k2 = make_cfg(hc=5)
    assert L.engram_ctx_create(ctypes.byref(bad), FAKE, 1 << 40, ctypes.byref(h)) \
        == E.E_UNSUPPORTED
    bad, k3 = make_cfg(dim=1000)
    assert L.engram_ctx_create(ctypes.byref(bad), FAKE, 1 << 40, ctypes.byref(h)) \
        == E.E_UNSUPPORTED
    for kw in ({"max_seq": 1 << 61}, {"max_tokens": 1 << 60}, {"dim": 1 << 40}):
        bad, _ = make_cfg(**kw)
        assert L.engram_ctx_create(ctypes.byref(bad), FAKE, 1 << 62, ctypes.byref(h)) \
            == E.E_UNSUPPORTED, kw
    assert L.engram_ctx_create(ctypes.byref(cfg), FAKE, n, ctypes.byref(h)) == E.OK
    try:
        assert L.engram_position(h) == 0
        ptrs = [ctypes.c_void_p() for _ in range(4)]
        assert L.engram_ctx_buffers(h, *[ctypes.byref(p) for p in ptrs]) == E.OK
        hist, rid, rows, kv, err = FAKE, *[p.value for p in ptrs]
        assert rid == FAKE + 4096 and rows == rid + 8 * 64 * 48
        assert err == FAKE + n - 256
        # forward / Q2_K wkv before any layer is registered
        rc, msg = rc_msg(L.engram_ctx_set_wkv_q2k(h, 0, FAKE))
        assert rc == E.E_STATE and "no weights" in msg
        rc, msg = rc_msg(L.engram_forward(h, 0, FAKE, 1, FAKE, None))
        assert rc == E.E_STATE and "no weights" in msg
        # the table must cover every hashed id of the layer: max(offset+prime) =
        # 47*101 + 101 = 4848 rows for layer 1
        tab = E.TableC(E.FMT_Q2K, 256, 0, 0, 4847, FAKE, None)
        rc, msg = rc_msg(L.engram_ctx_add_layer(h, 1, ctypes.byref(tab), FAKE, FAKE))
        assert rc == E.E_RANGE and "reaches row 4847" in msg
        tab = E.TableC(E.FMT_Q2K, 256, 0, 0, 4848, FAKE, None)
        assert L.engram_ctx_add_layer(h, 1, ctypes.byref(tab), FAKE, FAKE) == E.OK
        assert L.engram_ctx_add_layer(h, 2, ctypes.byref(tab), FAKE, FAKE) == E.E_ARG
        tab128 = E.TableC(E.FMT_E4M3, 128, 128, 0, 5000, FAKE, FAKE)
        assert L.engram_ctx_add_layer(h, 0, ctypes.byref(tab128), FAKE, FAKE) == E.E_ARG
        tab0 = E.TableC(E.FMT_Q2K, 256, 0, 0, 2424, FAKE, None)
        assert L.engram_ctx_add_layer(h, 0, ctypes.byref(tab0), FAKE, FAKE) == E.OK
        # layer 1 before layer 0 opened a step
        rc, msg = rc_msg(L.engram_forward(h, 1, None, 1, FAKE, None))
        assert rc == E.E_STATE and "before layer 0" in msg
        # too many tokens, too many positions, bad arguments
        assert L.engram_forward(h, 0, FAKE, 65, FAKE, None) == E.E_RANGE
        assert L.engram_forward(h, 0, FAKE, 0, FAKE, None) == E.E_ARG
        assert L.engram_forward(h, 0, None, 1, FAKE, None) == E.E_ARG
        assert L.engram_forward(h, 0, FAKE, 1, FAKE + 4, None) == E.E_ARG
        assert L.engram_forward(h, 3, FAKE, 1, FAKE, None) == E.E_ARG
        # Q2_K wkv: an unregistered layer, misaligned blocks; NULL drops them
        assert L.engram_ctx_set_wkv_q2k(h, 1, FAKE) == E.OK
        rc, msg = rc_msg(L.engram_ctx_set_wkv_q2k(h, 2, FAKE))
        assert rc == E.E_ARG
        assert L.engram_ctx_set_wkv_q2k(h, 0, FAKE + 2) == E.E_ARG
        assert L.engram_ctx_set_wkv_q2k(h, 0, None) == E.OK
        # a valid call before the first engram_reset (nothing is launched)
        rc, msg = rc_msg(L.engram_forward(h, 0, FAKE, 1, FAKE, None))
        assert rc == E.E_STATE and "engram_reset" in msg
        # graph mode likewise needs the reset (the device position starts there)
        rc, msg = rc_msg(L.engram_ctx_set_graph_mode(h, 1, None))
        assert rc == E.E_STATE and "engram_reset" in msg
        assert L.engram_ctx_set_graph_mode(None, 1, None) == E.E_ARG
        # resuming: the position must lie in 0..max_seq (checked before any launch)
        rc, msg = rc_msg(L.engram_ctx_set_position(h, 513, None))
        assert rc == E.E_RANGE and "outside 0..512" in msg
        assert L.engram_ctx_set_position(h, -1, None) == E.E_RANGE
        assert L.engram_ctx_set_position(None, 0, None) == E.E_ARG
        assert L.engram_position(h) == 0
        # timing with nothing recorded makes no runtime call
        assert L.engram_ctx_set_timing(h, 1) == E.OK
        ms = (ctypes.c_double * 4)()
        cnt = (ctypes.c_int64 * 4)()
        assert L.engram_ctx_timing(h, ms, cnt) == E.OK and list(cnt) == [0, 0, 0, 0]
    finally:
        L.engram_ctx_destroy(h)
    L.engram_ctx_destroy(None)
    assert L.engram_position(None) == -1


def test_position_limit(L):
    cfg, keep = make_cfg(max_tokens=64, max_seq=16)
    n = L.engram_workspace_bytes(ctypes.byref(cfg))
    h = ctypes.c_void_p()
    assert L.engram_ctx_create(ctypes.byref(cfg), FAKE, n, ctypes.byref(h)) == E.OK
    try:
        tab = E.TableC(E.FMT_Q2K, 256, 0, 0, 1 << 20, FAKE, None)
        assert L.engram_ctx_add_layer(h, 0, ctypes.byref(tab), FAKE, FAKE) == E.OK
        rc, msg = rc_msg(L.engram_forward(h, 0, FAKE, 17, FAKE, None))
        assert rc == E.E_RANGE and "16 positions, 17 needed" in msg
    finally:
        L.engram_ctx_destroy(h)


def test_binding_without_library(monkeypatch, tmp_path):
    """The binding has no fallback: a missing library raises."""
    monkeypatch.setattr(E, "_lib", None)
    monkeypatch.setattr(E, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        E.lib()


def test_binding_refuses_short_buffers(monkeypatch):
    """The C entry points cannot see a buffer's size; the binding refuses a
    tensor that a call of the given sizes would read or write past the end of
    its storage (or a strided view where rows must be dense) before the
    library is reached."""
    torch = pytest.importorskip("torch")

    def unreachable():
        raise AssertionError("the library was reached")
    monkeypatch.setattr(E, "lib", unreachable)
    i16 = lambda *s: torch.zeros(*s, dtype=torch.int16)

    def refused(f, *args, what):
        with pytest.raises(E.EngramError, match=what) as e:
            f(*args, stream=0)
        assert e.value.code == E.E_ARG

    refused(E.project, i16(4, 64), i16(32, 32), i16(4, 32), what="w: the call needs 4096 bytes")
    refused(E.project, i16(4, 64), i16(32, 64), i16(4, 16), what="y: the call needs 256 bytes")
    refused(E.project, i16(64, 4).t(), i16(32, 64), i16(4, 32), what="x: a contiguous tensor")
    refused(E.project_q2k, i16(1, 512), torch.zeros(16, 1, 84, dtype=torch.uint8), i16(1, 16),
            what="wkv_q2k: the call needs 2688 bytes")
    refused(E.dequant_q2k, torch.zeros(3 * 84, dtype=torch.uint8), i16(2 * 256), what="out")
    refused(E.gate_apply, torch.zeros(2, 4, 256), i16(2, 256 * 4), torch.zeros(4, 256), 1e-6,
            what="kv: the call needs 5120 bytes")
    refused(E.qk_product, i16(4, 256), i16(4, 256), torch.zeros(4, 128),
            what="qk: the call needs 4096 bytes")
    refused(E.qk_product, i16(4, 256), i16(2, 256), torch.zeros(4, 256),
            what="k: the call needs 2048 bytes")
    refused(E.stream_read, torch.zeros(4096, dtype=torch.uint8),
            torch.zeros(100, dtype=torch.int32), what="sink")

    tabs = E.HashTables(torch.zeros(16, dtype=torch.int64), 0, np.ones((2, 3), np.int64),
                        np.full((2, 4), 7, np.int64), np.zeros((2, 4), np.int64))
    ids = torch.zeros(5, dtype=torch.int32)
    hist = torch.zeros(16, dtype=torch.int64)
    refused(E.hash, tabs, ids, 0, hist, torch.zeros(5, 2, 3, dtype=torch.int64),
            what="row_ids: the call needs 320 bytes")
    # a strided id view reaching every id passes the check; one that stops short does not
    table = E.Table.__new__(E.Table)          # device table stand-in (no host mapping)
    table.c = E.TableC(E.FMT_Q2K, 256, 0, 0, 64, FAKE, None)
    ids2 = torch.zeros(5, 8, dtype=torch.int64)
    refused(E.gather_dequant, table, ids2[1:, 4:], 5, 4, 8, i16(5, 4 * 256),
            what="row_ids: the call needs 288 bytes, its storage holds 224")
    with pytest.raises(AssertionError, match="library was reached"):
        E.gather_dequant(table, ids2[:, 4:], 5, 4, 8, i16(5, 4 * 256), stream=0)


def test_layer_static_refusals(L):
    """The entry point that allocates nothing refuses, before any runtime
    call, sizes its static scratch cannot hold and the arguments
    engram_forward refuses."""
    c, keep = tables_c()
    # 2 layers x 101-row primes at offsets up to 47*101: 4848 rows needed
    tab = E.TableC(E.FMT_Q2K, 256, 0, 0, 5000, FAKE, None)
    sc = E.STATIC_SCRATCH_BYTES
    assert "#define ENGRAM_STATIC_SCRATCH_BYTES (32 << 20)" in open(HEADER).read()
    assert sc == 32 << 20

    def call(T=4, layer=0, start=0, max_seq=4096, table=tab, hc=4, dim=4096, ids=FAKE,
             wkv=FAKE, h=FAKE):
        return rc_msg(L.engram_layer_static(ctypes.byref(c), layer, ctypes.byref(table), wkv,
                                            FAKE, hc, dim, 1e-6, ids, T, start, FAKE, max_seq,
                                            h, None, None))

    # K = 24*256, N = 4096*5: 626 tokens need more than the 32 MiB scratch
    rc, msg = call(T=626)
    assert rc == E.E_RANGE and "scratch" in msg
    assert call(layer=2)[0] == E.E_ARG
    rc, msg = call(T=10, start=4090)
    assert rc == E.E_RANGE and "4096 positions" in msg
    assert call(T=2, start=(1 << 63) - 1, max_seq=(1 << 63) - 1)[0] == E.E_RANGE
    small = E.TableC(E.FMT_Q2K, 256, 0, 0, 100, FAKE, None)
    rc, msg = call(table=small)
    assert rc == E.E_RANGE and "rows" in msg
    assert call(hc=5)[0] == E.E_UNSUPPORTED
    assert call(ids=None)[0] == E.E_ARG
    assert call(wkv=None)[0] == E.E_ARG
    assert call(h=FAKE + 4)[0] == E.E_ARG
    assert call(T=0, ids=None, h=None)[0] == E.OK
