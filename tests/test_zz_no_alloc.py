"""The entry point that allocates nothing (engram_layer_static): its row
ids, rows and kv sit in the library's static device scratch.  Called through
the C ABI and checked against engram_forward (the stateful entry point the
same kernels serve) on the same inputs, bit for bit: two calls in a row on
one sequence, the second smaller than the first (a prompt, then single-token
steps), on every layer; the highway also against the oracle gate of the
stateful path's kv, and sizes past the scratch refused."""
import ctypes

import numpy as np
import pytest

import synth
from synth import generate as G
from _gpu_util import Device, log, relerr

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def E():
    import gram_hashed_embedding_engram_amd as E
    E.lib()
    return E


def cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("name,calls", [(synth.DECODE_Q2K.name, (32, 1, 1)),
                                        (synth.TINY_E4M3.name, (64, 7, 1)),
                                        (synth.ODD_Q2K.name, (8, 3, 1)),
                                        (synth.ODD_E4M3.name, (5, 1))])
def test_layer_static_matches_forward(E, name, calls):
    import oracle
    dev = Device(name)
    w = dev.w
    n = sum(calls)
    log(f"layer_static vs forward: {name}, calls {calls}")
    ids = G.token_ids(w, n)
    h_all = G.highway(w, n)
    d_ids = cuda(ids.astype(np.int32))
    ctx = dev.context(max_tokens=max(calls), max_seq=n)
    hist = torch.zeros(n, dtype=torch.int64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pos = 0
    for T in calls:
        for layer in range(w.n_layers):
            h0 = h_all[pos:pos + T]
            want = cuda(h0)
            ctx.forward(layer, d_ids[pos:pos + T] if layer == 0 else None, T, want)
            _, _, kv = ctx.views(T)
            kv = kv.cpu().numpy().view(np.uint16)
            got = cuda(h0)
            E.layer_static(dev.tables, layer, dev.tab[layer], dev.wkv[layer], dev.qk[layer],
                           w.eps, d_ids[pos:pos + T], pos, hist, got, err)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(got.cpu().numpy().view(np.uint32),
                                          want.cpu().numpy().view(np.uint32),
                                          err_msg=f"call at {pos} (T {T}) layer {layer}")
            L = dev.layers[layer]
            e_h = relerr(got.cpu().numpy(), oracle.gate_and_add(h0, kv, L["q"], L["k"], w.eps))
            assert e_h <= 2e-3, f"call at {pos} layer {layer}: highway relerr {e_h:.2e}"
        pos += T
    ctx.check()
    assert int(err.item()) == 0
    # the sequence's history equals the stateful context's
    torch.testing.assert_close(hist, ctx.history()[0], rtol=0, atol=0)


def test_layer_static_refuses_past_scratch(E):
    dev = Device(synth.DECODE_Q2K.name)
    w = dev.w
    T = 626            # one token more than the scratch holds at this geometry
    d_ids = torch.zeros(T, dtype=torch.int32, device="cuda")
    hist = torch.zeros(T, dtype=torch.int64, device="cuda")
    h = torch.zeros(T, w.hc, w.dim, dtype=torch.float32, device="cuda")
    with pytest.raises(E.EngramError) as ei:
        E.layer_static(dev.tables, 0, dev.tab[0], dev.wkv[0], dev.qk[0], w.eps, d_ids, 0, hist, h)
    assert ei.value.code == E.E_RANGE and "scratch" in str(ei.value)
    # 625 tokens fit
    E.layer_static(dev.tables, 0, dev.tab[0], dev.wkv[0], dev.qk[0], w.eps, d_ids[:625], 0,
                   hist, h[:625])
    torch.cuda.synchronize()
