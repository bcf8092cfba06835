"""GPU parity of the fused, stateful engram_forward on the five synthetic
workloads, the decode workload with Q2_K wkv and small odd-column edge cases
(run on an MI355X).

The chain is checked stage by stage on the GPU's own intermediates: hash ids
(bit for bit against the oracle hasher fed the same token stream), rows (bit
for bit against the oracle gather of the oracle ids), kv (relative error
<= 1e-2 against the oracle projection of the rows), highway (relative error
<= 2e-3 against the oracle gate applied to the GPU's kv).  Large workloads
are checked on all hash ids and rows and on sampled tokens / output columns
for kv.
"""
import numpy as np
import pytest

import oracle
import synth
from synth import generate as G
from _gpu_util import (Device, log, relerr, widen, to_np_u16, tile_strata, assert_tiles_covered,
                       GEMM_TILE_M, GEMM_TILE_N)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def E():
    import gram_hashed_embedding_engram_amd as E
    E.lib()
    return E


def cuda(a):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def check_call(dev, ctx, layer, ids_np, hasher_out, h_before, h_after, T, sample_tokens=None,
               sample_cols=None, label=""):
    """Compare one forward call's intermediates and output with the oracle
    (T = all tokens of the call, batch * tokens per sequence): every row id and
    row bit for bit, kv on the sampled tokens (all outputs) and the sampled
    outputs (all tokens), or on everything, and the highway of every token
    against the oracle gate of the GPU's kv."""
    w = dev.w
    rid, rows, kv = ctx.views(T // ctx.batch)
    rid = rid.cpu().numpy()
    np.testing.assert_array_equal(rid, hasher_out, err_msg=f"{label} hash ids")
    rows = to_np_u16(rows)
    want_rows = dev.oracle_rows(layer, hasher_out[:, layer, :]).reshape(T, -1)
    np.testing.assert_array_equal(rows, want_rows, err_msg=f"{label} rows")
    kv = to_np_u16(kv)
    toks = np.arange(T) if sample_tokens is None else sample_tokens
    want_kv = oracle.linear_bf16(rows[toks], dev.oracle_wkv(layer))
    e_kv = relerr(widen(kv[toks]), widen(want_kv))
    assert e_kv <= 1e-2, f"{label} kv relerr {e_kv:.2e}"
    if sample_cols is not None:
        want_c = oracle.linear_bf16(rows, dev.oracle_wkv(layer)[sample_cols])
        e_c = relerr(widen(kv[:, sample_cols]), widen(want_c))
        assert e_c <= 1e-2, f"{label} kv cols relerr {e_c:.2e}"
    # the gate over every token (cheap on the host), fed the GPU's own kv
    L = dev.layers[layer]
    want_h = oracle.gate_and_add(h_before, kv, L["q"], L["k"], w.eps)
    e_h = relerr(h_after, want_h)
    assert e_h <= 2e-3, f"{label} highway relerr {e_h:.2e}"
    return e_kv, e_h, kv


def test_forward_tiny(E):
    w = synth.TINY_E4M3
    log("forward: tiny e4m3 T=64")
    dev = Device(w.name)
    ids = G.token_ids(w)
    h0 = G.highway(w, w.prompt)
    ctx = dev.context(max_tokens=64, max_seq=64)
    d_h = torch.from_numpy(h0).cuda()
    ctx.forward(0, cuda(ids.astype(np.int32)), 64, d_h)
    ctx.check()
    assert ctx.position == 64
    h1 = d_h.cpu().numpy()
    want_ids = dev.oracle_hasher(64).hash(ids, 0)
    e_kv, e_h, kv = check_call(dev, ctx, 0, ids, want_ids, h0, h1, 64, label="tiny")
    # the fully oracle chain (diagnostic: differs from the GPU's by kv rounding)
    rows = dev.oracle_rows(0, want_ids[:, 0, :]).reshape(64, -1)
    kv_o = oracle.linear_bf16(rows, dev.oracle_wkv(0))
    h_o = oracle.gate_and_add(h0, kv_o, dev.layers[0]["q"], dev.layers[0]["k"], w.eps)
    log(f"  kv {e_kv:.2e}  highway {e_h:.2e}  full-oracle highway {relerr(h1, h_o):.2e}"
        f"  kv bits differing {(kv != kv_o).mean():.2e}")
    # the rows themselves: e4m3 times a power of two is exact in bf16
    assert relerr(h1, h_o) < 2e-2


def test_forward_decode_workload(E):
    """32-token prompt, then 256 single-token steps over both layers."""
    w = synth.DECODE_Q2K
    log("forward: decode Q2_K, prompt 32 + 256 steps, 2 layers")
    dev = Device(w.name)
    ids = G.token_ids(w)
    max_seq = w.total_tokens
    ctx = dev.context(max_tokens=32, max_seq=max_seq)
    hasher = dev.oracle_hasher(max_seq)
    d_ids = cuda(ids.astype(np.int32))
    prompt_h = G.highway(w, w.prompt)
    step_h = G.highway(w, w.decode_steps, decode=True)
    worst = [0.0, 0.0]
    pos = 0
    for step in range(1 + w.decode_steps):
        T = w.prompt if step == 0 else 1
        h0 = prompt_h if step == 0 else step_h[step - 1:step]
        want_ids = hasher.hash(ids[pos:pos + T], pos)
        for layer in range(2):
            d_h = torch.from_numpy(h0).cuda()
            ctx.forward(layer, d_ids[pos:pos + T] if layer == 0 else None, T, d_h)
            h1 = d_h.cpu().numpy()
            e_kv, e_h, _ = check_call(dev, ctx, layer, ids[pos:pos + T], want_ids, h0, h1, T,
                                      label=f"step {step} layer {layer}")
            worst = [max(worst[0], e_kv), max(worst[1], e_h)]
        pos += T
        assert ctx.position == pos
    ctx.check()
    log(f"  worst kv relerr {worst[0]:.2e}, highway {worst[1]:.2e}")


@pytest.mark.parametrize("name", [synth.ODD_Q2K.name, synth.ODD_E4M3.name,
                                  synth.ODD_WKVQ2K.name, synth.ODD_E4M3_WKVQ2K.name,
                                  synth.MAX_SLOTS_Q2K.name, synth.MAX_NGRAM_E4M3.name,
                                  synth.HC1_Q2K.name, synth.HC3_E4M3.name,
                                  synth.HC2_WKVQ2K.name])
def test_forward_edge_geometry(E, name):
    """Edge-case hash geometries: an odd number of columns (5: K 1280, an
    odd number of 1 KiB loads a row, a partial last sub-block round), the
    most hash slots (4 layers x 32 columns = 128, K 8192) and the longest
    n-gram (8, 4 layers x 28 columns).  A prompt, then single-token steps
    through the one-launch decode kernels, every layer, every call against
    the oracle."""
    dev = Device(name)
    w = dev.w
    log(f"forward: {name}, prompt {w.prompt} + {w.decode_steps} steps")
    ids = G.token_ids(w)
    max_seq = w.total_tokens
    ctx = dev.context(max_tokens=w.prompt, max_seq=max_seq)
    hasher = dev.oracle_hasher(max_seq)
    d_ids = cuda(ids.astype(np.int32))
    prompt_h = G.highway(w, w.prompt)
    step_h = G.highway(w, w.decode_steps, decode=True)
    pos = 0
    for step in range(1 + w.decode_steps):
        T = w.prompt if step == 0 else 1
        h0 = prompt_h if step == 0 else step_h[step - 1:step]
        want_ids = hasher.hash(ids[pos:pos + T], pos)
        for layer in range(w.n_layers):
            d_h = torch.from_numpy(h0).cuda()
            ctx.forward(layer, d_ids[pos:pos + T] if layer == 0 else None, T, d_h)
            check_call(dev, ctx, layer, ids[pos:pos + T], want_ids, h0, d_h.cpu().numpy(), T,
                       label=f"step {step} layer {layer}")
        pos += T
    ctx.check()


def test_forward_decode_wkv_q2k(E):
    """The decode workload with wkv shipped as Q2_K blocks: the 32-token prompt
    runs the GEMM over the library's bf16 expansion, every single-token step
    projects from the blocks; kv against the oracle projection over the
    oracle's own expansion."""
    w = synth.DECODE_WKVQ2K
    steps = 64
    log(f"forward: decode Q2_K with Q2_K wkv, prompt 32 + {steps} steps, 2 layers")
    dev = Device(w.name)
    ids = G.token_ids(w)
    max_seq = w.prompt + steps
    ctx = dev.context(max_tokens=32, max_seq=max_seq)
    hasher = dev.oracle_hasher(max_seq)
    d_ids = cuda(ids.astype(np.int32))
    prompt_h = G.highway(w, w.prompt)
    step_h = G.highway(w, steps, decode=True)
    worst = [0.0, 0.0]
    pos = 0
    for step in range(1 + steps):
        T = w.prompt if step == 0 else 1
        h0 = prompt_h if step == 0 else step_h[step - 1:step]
        want_ids = hasher.hash(ids[pos:pos + T], pos)
        for layer in range(2):
            d_h = torch.from_numpy(h0).cuda()
            ctx.forward(layer, d_ids[pos:pos + T] if layer == 0 else None, T, d_h)
            h1 = d_h.cpu().numpy()
            e_kv, e_h, _ = check_call(dev, ctx, layer, ids[pos:pos + T], want_ids, h0, h1, T,
                                      label=f"step {step} layer {layer}")
            worst = [max(worst[0], e_kv), max(worst[1], e_h)]
        pos += T
    ctx.check()
    log(f"  worst kv relerr {worst[0]:.2e}, highway {worst[1]:.2e}")


@pytest.mark.parametrize("B,prompt,steps", [(4, 8, 16), (6, 4, 4)])
def test_forward_batched_sequences(E, B, prompt, steps):
    """B sequences decoded together (one token of each per step through one
    pass over each layer's weights): every token's ids, rows, kv and highway
    against the oracle run on that sequence alone.  B = 4 single-token steps
    take the GEMV, B = 6 the GEMM."""
    w = synth.DECODE_Q2K
    log(f"forward: {B} sequences, prompt {prompt} + {steps} steps, 2 layers")
    dev = Device(w.name)
    rng = np.random.default_rng(B)
    n = prompt + steps
    ids = rng.integers(0, w.vocab, size=(B, n)).astype(np.int32)
    ctx = dev.context(max_tokens=prompt, max_seq=n, batch=B)
    hashers = [dev.oracle_hasher(n) for _ in range(B)]
    h_all = rng.standard_normal((B, n, w.hc, w.dim)).astype(np.float32)
    pos = 0
    worst = [0.0, 0.0]
    for step in range(1 + steps):
        T = prompt if step == 0 else 1
        want_ids = np.concatenate([hashers[b].hash(ids[b, pos:pos + T], pos) for b in range(B)])
        h0 = np.ascontiguousarray(h_all[:, pos:pos + T]).reshape(B * T, w.hc, w.dim)
        d_ids = cuda(np.ascontiguousarray(ids[:, pos:pos + T]))
        for layer in range(2):
            d_h = torch.from_numpy(h0).cuda()
            ctx.forward(layer, d_ids if layer == 0 else None, T, d_h)
            h1 = d_h.cpu().numpy()
            e_kv, e_h, _ = check_call(dev, ctx, layer, None, want_ids, h0, h1, B * T,
                                      label=f"B={B} step {step} layer {layer}")
            worst = [max(worst[0], e_kv), max(worst[1], e_h)]
        pos += T
        assert ctx.position == pos
    ctx.check()
    log(f"  worst kv relerr {worst[0]:.2e}, highway {worst[1]:.2e}")


def test_forward_prefill_workload(E):
    """T = 4096 Zipf tokens through both layers with one hash pass."""
    w = synth.PREFILL_Q2K
    log("forward: prefill Q2_K T=4096, 2 layers")
    dev = Device(w.name)
    ids = G.token_ids(w)
    T = w.prompt
    h0 = G.highway(w, T)
    ctx = dev.context(max_tokens=T, max_seq=T)
    want_ids = dev.oracle_hasher(T).hash(ids, 0)
    rng = np.random.default_rng(1)
    toks = tile_strata(T, GEMM_TILE_M, rng)
    cols = tile_strata(w.N, GEMM_TILE_N, rng)
    assert_tiles_covered(toks, cols, T, w.N)
    d_ids = cuda(ids.astype(np.int32))
    for layer in range(2):
        d_h = torch.from_numpy(h0).cuda()
        ctx.forward(layer, d_ids if layer == 0 else None, T, d_h)
        h1 = d_h.cpu().numpy()
        e_kv, e_h, _ = check_call(dev, ctx, layer, ids, want_ids, h0, h1, T, toks, cols,
                                  label=f"prefill layer {layer}")
        log(f"  layer {layer}: kv {e_kv:.2e} highway {e_h:.2e}")
    ctx.check()


def test_forward_split_workload(E):
    """e4m3 tables: 8192 Zipf tokens in chunks of 2048, then 128 decode steps.
    Each call's hash ids equal the single-pass hash of the whole sequence."""
    w = synth.SPLIT_E4M3
    log("forward: split e4m3, 4x2048 + 128x1, 2 layers")
    dev = Device(w.name)
    ids = G.token_ids(w)
    n = ids.size
    single = dev.oracle_hasher(n).hash(ids, 0)
    ctx = dev.context(max_tokens=w.chunk, max_seq=n)
    d_ids = cuda(ids.astype(np.int32))
    prompt_h = G.highway(w, w.prompt)
    step_h = G.highway(w, w.decode_steps, decode=True)
    bounds = list(range(0, w.prompt + 1, w.chunk)) + list(range(w.prompt + 1, n + 1))
    rng = np.random.default_rng(3)
    for ci, (a, b) in enumerate(zip(bounds[:-1], bounds[1:])):
        T = b - a
        h0 = prompt_h[a:b] if a < w.prompt else step_h[a - w.prompt:b - w.prompt]
        full_check = T > 1 or ci % 16 == 0
        for layer in range(2):
            d_h = torch.from_numpy(h0).cuda()
            ctx.forward(layer, d_ids[a:b] if layer == 0 else None, T, d_h)
            if full_check:
                toks = tile_strata(T, GEMM_TILE_M, rng)
                cols = tile_strata(w.N, GEMM_TILE_N, rng) if T > 1 else None
                if T > 1:
                    assert_tiles_covered(toks, cols, T, w.N)
                check_call(dev, ctx, layer, ids[a:b], single[a:b], h0, d_h.cpu().numpy(), T,
                           toks, cols, label=f"split call {ci} layer {layer}")
            else:
                rid = ctx.views(T)[0].cpu().numpy()
                np.testing.assert_array_equal(rid, single[a:b])
    assert ctx.position == n
    ctx.check()


def test_forward_gather_stress(E):
    """One Q2_K layer over ~71M rows (5.9 GB), T = 16384 uniform tokens."""
    w = synth.GATHER_Q2K
    log("forward: gather stress Q2_K, 71M-row table, T=16384")
    dev = Device(w.name)
    ids = G.token_ids(w)
    T = w.prompt
    h0 = G.highway(w, T)
    ctx = dev.context(max_tokens=T, max_seq=T)
    d_h = torch.from_numpy(h0).cuda()
    ctx.forward(0, cuda(ids.astype(np.int32)), T, d_h)
    ctx.check()
    want_ids = dev.oracle_hasher(T).hash(ids, 0)
    rng = np.random.default_rng(4)
    toks = tile_strata(T, GEMM_TILE_M, rng)
    cols = tile_strata(w.N, GEMM_TILE_N, rng)
    assert_tiles_covered(toks, cols, T, w.N)
    e_kv, e_h, _ = check_call(dev, ctx, 0, ids, want_ids, h0, d_h.cpu().numpy(), T, toks, cols,
                              label="gather stress")
    log(f"  kv {e_kv:.2e} highway {e_h:.2e}")


def test_forward_deterministic_and_device_error(E):
    w = synth.TINY_E4M3
    dev = Device(w.name)
    ids = G.token_ids(w)
    h0 = G.highway(w, 64)
    outs = []
    for _ in range(2):
        ctx = dev.context(max_tokens=64, max_seq=128)
        d_h = torch.from_numpy(h0).cuda()
        ctx.forward(0, cuda(ids.astype(np.int32)), 64, d_h)
        outs.append(d_h.cpu().numpy().view(np.uint32))
        ctx.check()
    np.testing.assert_array_equal(outs[0], outs[1])
    bad = ids.copy()
    bad[5] = w.vocab + 3
    ctx = dev.context(max_tokens=64, max_seq=128)
    d_h = torch.from_numpy(h0).cuda()
    ctx.forward(0, cuda(bad.astype(np.int32)), 64, d_h)
    with pytest.raises(E.EngramError) as ei:
        ctx.check()
    assert ei.value.code == E.E_DEVICE
    ctx.reset()
    ctx.check()


def run_steps(dev, ctx, ids, steps, prompt, h_prompt, h_steps):
    """Prompt then single-token steps; returns per call (row ids, rows, kv, h)."""
    out = []
    d_ids = cuda(ids.astype(np.int32))
    pos = 0
    for step in range(1 + steps):
        T = prompt if step == 0 else 1
        h0 = h_prompt if step == 0 else h_steps[step - 1:step]
        for layer in range(dev.w.n_layers):
            d_h = torch.from_numpy(np.ascontiguousarray(h0)).cuda()
            ctx.forward(layer, d_ids[pos:pos + T] if layer == 0 else None, T, d_h)
            rid, rows, kv = ctx.views(T)
            out.append((rid.cpu().numpy(), to_np_u16(rows), to_np_u16(kv),
                        d_h.cpu().numpy().view(np.uint32)))
        pos += T
    return out


@pytest.mark.parametrize("name", [synth.DECODE_Q2K.name, synth.TINY_E4M3.name,
                                  synth.DECODE_WKVQ2K.name, synth.ODD_Q2K.name,
                                  synth.ODD_E4M3.name, synth.ODD_WKVQ2K.name,
                                  synth.ODD_E4M3_WKVQ2K.name, synth.MAX_SLOTS_Q2K.name,
                                  synth.MAX_NGRAM_E4M3.name, synth.HC1_Q2K.name,
                                  synth.HC3_E4M3.name, synth.HC2_WKVQ2K.name])
def test_fused_decode_matches_staged(E, name):
    """The one-launch decode layer (hash + gather + projection) leaves exactly
    what the staged kernels leave: row ids, rows, kv and highway, bit for bit."""
    dev = Device(name)
    w = dev.w
    log(f"fused vs staged decode: {name}")
    prompt, steps = 8, 24
    ids = G.token_ids(w, prompt + steps)
    hp = G.highway(w, prompt)
    hs = G.highway(w, steps, decode=True) if w.decode_steps else G.highway(w, steps)
    res = []
    for fused in (True, False):
        ctx = dev.context(max_tokens=prompt, max_seq=prompt + steps)
        ctx.set_fused_decode(fused)
        res.append(run_steps(dev, ctx, ids, steps, prompt, hp, hs))
        ctx.check()
    for i, (a, b) in enumerate(zip(*res)):
        for x, y, what in zip(a, b, ("row ids", "rows", "kv", "highway")):
            np.testing.assert_array_equal(x, y, err_msg=f"call {i}: {what}")
    # and the hash of the steps equals the oracle's single pass
    want = dev.oracle_hasher(prompt + steps).hash(ids, 0)
    calls = res[0][::w.n_layers]
    np.testing.assert_array_equal(calls[-1][0], want[-1:])


@pytest.mark.parametrize("name,B", [(synth.DECODE_Q2K.name, 1), (synth.TINY_E4M3.name, 1),
                                    (synth.ODD_E4M3.name, 1), (synth.DECODE_Q2K.name, 3)])
def test_host_tables_match_device_tables(E, name, B):
    """Tables in pinned host memory, read by the kernels across the host link
    (the atlascybernetics engram_v41 page, EngramRowReader: rows fetched from
    wherever the table lives): the prompt and every decode step, one launch or
    staged, are checked against the oracle (ids and rows bit for bit, kv and
    highway within tolerance) and leave exactly what device-resident tables
    leave -- row ids, rows, kv and highway, bit for bit."""
    w = synth.WORKLOADS[name]
    prompt, steps = 8, 12
    log(f"host vs device tables: {name}, B={B}")
    ids = G.token_ids(w, B * (prompt + steps)).reshape(B, prompt + steps)
    hp = G.highway(w, B * prompt).reshape(B, prompt, w.hc, w.dim)
    hs = G.highway(w, B * steps).reshape(steps, B, w.hc, w.dim)
    res = []
    for host in (False, True):
        dev = Device(name, host_tables=host)
        assert dev.tab[0].data.is_cuda != host
        for fused in (True, False):
            ctx = dev.context(max_tokens=prompt, max_seq=prompt + steps, batch=B)
            ctx.set_fused_decode(fused)
            hashers = [dev.oracle_hasher(prompt + steps) for _ in range(B)]
            d_ids = cuda(ids.astype(np.int32))
            out = []
            for step in range(1 + steps):
                T = prompt if step == 0 else 1
                p0 = 0 if step == 0 else prompt + step - 1
                h0 = hp if step == 0 else hs[step - 1][:, None]
                want_ids = np.concatenate([hashers[b].hash(ids[b, p0:p0 + T], p0)
                                           for b in range(B)])
                for layer in range(w.n_layers):
                    d_h = torch.from_numpy(np.ascontiguousarray(h0)).cuda()
                    ctx.forward(layer, d_ids[:, p0:p0 + T].contiguous() if layer == 0 else None,
                                T, d_h)
                    if host:
                        # the host-table path against the oracle itself
                        check_call(dev, ctx, layer, None, want_ids,
                                   np.ascontiguousarray(h0).reshape(B * T, w.hc, w.dim),
                                   d_h.cpu().numpy().reshape(B * T, w.hc, w.dim), B * T,
                                   label=f"host tables fused={fused} step {step} layer {layer}")
                    rid, rows, kv = ctx.views(T)
                    out.append((rid.cpu().numpy(), to_np_u16(rows), to_np_u16(kv),
                                d_h.cpu().numpy().view(np.uint32)))
            ctx.check()
            res.append(out)
        del dev
    for r in res[1:]:
        for i, (a, b) in enumerate(zip(res[0], r)):
            for x, y, what in zip(a, b, ("row ids", "rows", "kv", "highway")):
                np.testing.assert_array_equal(x, y, err_msg=f"call {i}: {what}")


def decode_steps_eager(dev, B, ids, hp, hs, prompt, steps):
    """Reference: the prompt, then single-token steps through the one-launch
    kernels, eagerly; per step the row ids, the last layer's rows and kv, and
    every layer's highway (each layer gated from the step's fresh highway)."""
    w = dev.w
    ctx = dev.context(max_tokens=prompt, max_seq=prompt + steps, batch=B)
    d_ids = cuda(ids.astype(np.int32))
    for layer in range(w.n_layers):
        ctx.forward(layer, d_ids[:, :prompt].contiguous() if layer == 0 else None, prompt,
                    torch.from_numpy(np.ascontiguousarray(hp)).cuda())
    out = []
    for step in range(steps):
        hl = []
        for layer in range(w.n_layers):
            d_h = torch.from_numpy(np.ascontiguousarray(hs[step][:, None])).cuda()
            ctx.forward(layer, d_ids[:, prompt + step:prompt + step + 1].contiguous()
                        if layer == 0 else None, 1, d_h)
            hl.append(d_h.cpu().numpy().view(np.uint32))
        rid, rows, kv = ctx.views(1)
        out.append((rid.cpu().numpy(), to_np_u16(rows), to_np_u16(kv), hl))
    ctx.check()
    return out


@pytest.mark.parametrize("name,B", [(synth.DECODE_Q2K.name, 1), (synth.ODD_E4M3.name, 1),
                                    (synth.DECODE_WKVQ2K.name, 1), (synth.DECODE_Q2K.name, 3)])
def test_graph_replay_matches_eager(E, name, B):
    """A decode step captured once into a hipGraph in graph mode (the kernels
    read the step's position from the device; the last layer's gate advances
    it) and replayed step after step, with the token and highway buffers
    refilled eagerly between replays, leaves exactly what eager steps leave:
    row ids, rows, kv and every layer's highway, bit for bit (the pages' graph
    oracle mode).  A replay past max_seq is reported, and the device position
    comes back to the host when graph mode ends."""
    dev = Device(name)
    w = dev.w
    prompt, steps = 8, 12
    log(f"graph replay vs eager: {name}, B={B}")
    ids = G.token_ids(w, B * (prompt + steps)).reshape(B, prompt + steps)
    hp = G.highway(w, B * prompt).reshape(B, prompt, w.hc, w.dim)
    hs = G.highway(w, B * steps).reshape(steps, B, w.hc, w.dim)
    want = decode_steps_eager(dev, B, ids, hp, hs, prompt, steps)

    ctx = dev.context(max_tokens=prompt, max_seq=prompt + steps, batch=B)
    d_ids = cuda(ids.astype(np.int32))
    for layer in range(w.n_layers):
        ctx.forward(layer, d_ids[:, :prompt].contiguous() if layer == 0 else None, prompt,
                    torch.from_numpy(np.ascontiguousarray(hp)).cuda())
    ctx.set_graph_mode(True)
    with pytest.raises(E.EngramError) as ei:          # many tokens: not in graph mode
        ctx.forward(0, d_ids[:, :2].contiguous(), 2, torch.zeros(B, 2, w.hc, w.dim).cuda())
    assert ei.value.code == E.E_STATE
    for refused in (lambda: ctx.set_timing(True), lambda: ctx.set_fused_decode(False)):
        with pytest.raises(E.EngramError) as ei:      # nothing a capture could not replay
            refused()
        assert ei.value.code == E.E_STATE
    tok = torch.zeros(B, 1, dtype=torch.int32, device="cuda")
    hbuf = [torch.zeros(B, 1, w.hc, w.dim, dtype=torch.float32, device="cuda")
            for _ in range(w.n_layers)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for layer in range(w.n_layers):
            ctx.forward(layer, tok if layer == 0 else None, 1, hbuf[layer])
    for step in range(steps):
        tok.copy_(d_ids[:, prompt + step:prompt + step + 1])
        h0 = torch.from_numpy(np.ascontiguousarray(hs[step][:, None])).cuda()
        for hb in hbuf:
            hb.copy_(h0)
        g.replay()
        torch.cuda.synchronize()
        rid, rows, kv = ctx.views(1)
        wr, wrows, wkv, wh = want[step]
        np.testing.assert_array_equal(rid.cpu().numpy(), wr, err_msg=f"step {step} row ids")
        np.testing.assert_array_equal(to_np_u16(rows), wrows, err_msg=f"step {step} rows")
        np.testing.assert_array_equal(to_np_u16(kv), wkv, err_msg=f"step {step} kv")
        for layer in range(w.n_layers):
            np.testing.assert_array_equal(hbuf[layer].cpu().numpy().view(np.uint32), wh[layer],
                                          err_msg=f"step {step} layer {layer} highway")
    ctx.check()
    # one replay past max_seq: reported on the device, position held at
    # max_seq, and no gate touches the highway
    h_keep = [torch.full_like(hb, 0.75) for hb in hbuf]
    for hb, hk in zip(hbuf, h_keep):
        hb.copy_(hk)
    g.replay()
    with pytest.raises(E.EngramError) as ei:
        ctx.check()
    assert ei.value.code == E.E_DEVICE and "max_seq" in str(ei.value)
    for layer, (hb, hk) in enumerate(zip(hbuf, h_keep)):
        assert torch.equal(hb, hk), f"layer {layer}: a refused step gated the highway"
    ctx.set_graph_mode(False)
    assert ctx.position == prompt + steps
    del g


@pytest.mark.parametrize("name,B", [(synth.DECODE_Q2K.name, 1), (synth.ODD_E4M3.name, 1),
                                    (synth.DECODE_WKVQ2K.name, 1), (synth.DECODE_Q2K.name, 3),
                                    (synth.ODD_Q2K.name, 2), (synth.MAX_SLOTS_Q2K.name, 1),
                                    (synth.HC1_Q2K.name, 1), (synth.HC3_E4M3.name, 3)])
def test_graph_replay_matches_oracle(E, name, B):
    """Replayed decode steps against the oracle itself (atlascybernetics
    "deepseek_v41_layer.rs", GraphMode): each layer's step is captured into a
    hipGraph of its own in graph mode, and every replay of every layer is
    checked like an eager call -- row ids and rows bit for bit against the
    oracle hasher and gather, kv within 1e-2 of the oracle projection, the
    highway within 2e-3 of the oracle gate of the GPU's kv."""
    dev = Device(name)
    w = dev.w
    prompt, steps = 6, 10
    log(f"graph replay vs oracle: {name}, B={B}")
    ids = G.token_ids(w, B * (prompt + steps)).reshape(B, prompt + steps)
    hp = G.highway(w, B * prompt).reshape(B * prompt, w.hc, w.dim)
    hs = G.highway(w, B * steps).reshape(steps, B, 1, w.hc, w.dim)
    hashers = [dev.oracle_hasher(prompt + steps) for _ in range(B)]
    ctx = dev.context(max_tokens=prompt, max_seq=prompt + steps, batch=B)
    d_ids = cuda(ids.astype(np.int32))
    want_ids = np.concatenate([hashers[b].hash(ids[b, :prompt], 0) for b in range(B)])
    for layer in range(w.n_layers):
        d_h = torch.from_numpy(hp).cuda()
        ctx.forward(layer, d_ids[:, :prompt].contiguous() if layer == 0 else None, prompt, d_h)
        check_call(dev, ctx, layer, None, want_ids, hp, d_h.cpu().numpy(), B * prompt,
                   label=f"prompt layer {layer}")
    ctx.set_graph_mode(True)
    tok = torch.zeros(B, 1, dtype=torch.int32, device="cuda")
    hbuf = [torch.zeros(B, 1, w.hc, w.dim, dtype=torch.float32, device="cuda")
            for _ in range(w.n_layers)]
    torch.cuda.synchronize()
    graphs = []
    for layer in range(w.n_layers):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            ctx.forward(layer, tok if layer == 0 else None, 1, hbuf[layer])
        graphs.append(g)
    worst = [0.0, 0.0]
    for step in range(steps):
        p = prompt + step
        tok.copy_(d_ids[:, p:p + 1])
        want_ids = np.concatenate([hashers[b].hash(ids[b, p:p + 1], p) for b in range(B)])
        h0 = np.ascontiguousarray(hs[step]).reshape(B, w.hc, w.dim)
        for layer in range(w.n_layers):
            hbuf[layer].copy_(torch.from_numpy(h0).reshape(B, 1, w.hc, w.dim))
            graphs[layer].replay()
            torch.cuda.synchronize()
            e_kv, e_h, _ = check_call(dev, ctx, layer, None, want_ids, h0,
                                      hbuf[layer].cpu().numpy().reshape(B, w.hc, w.dim), B,
                                      label=f"replay step {step} layer {layer}")
            worst = [max(worst[0], e_kv), max(worst[1], e_h)]
    ctx.check()
    ctx.set_graph_mode(False)
    assert ctx.position == prompt + steps
    log(f"  worst kv relerr {worst[0]:.2e}, highway {worst[1]:.2e}")
    del graphs


@pytest.mark.parametrize("name,B,fused", [(synth.DECODE_Q2K.name, 1, True),
                                          (synth.ODD_E4M3.name, 2, True),
                                          (synth.TINY_E4M3.name, 1, False)])
def test_resume_from_restored_history(E, name, B, fused):
    """A sequence resumed in a fresh context -- its history rows copied in
    from the first context's workspace, the position set -- continues exactly
    as the uninterrupted context: row ids, rows, kv and highway, bit for bit."""
    dev = Device(name)
    w = dev.w
    prompt, before, after = 8, 5, 7
    total = prompt + before + after
    log(f"resume: {name}, B={B}, fused={fused}")
    ids = G.token_ids(w, B * total).reshape(B, total)
    hp = G.highway(w, B * prompt).reshape(B, prompt, w.hc, w.dim)
    hs = G.highway(w, B * (before + after)).reshape(before + after, B, w.hc, w.dim)
    d_ids = cuda(ids.astype(np.int32))

    def step(ctx, p, h0):
        T = h0.shape[1]
        out = []
        for layer in range(w.n_layers):
            d_h = torch.from_numpy(np.ascontiguousarray(h0)).cuda()
            ctx.forward(layer, d_ids[:, p:p + T].contiguous() if layer == 0 else None, T, d_h)
            rid, rows, kv = ctx.views(T)
            out.append((rid.cpu().numpy(), to_np_u16(rows), to_np_u16(kv),
                        d_h.cpu().numpy().view(np.uint32)))
        return out

    a = dev.context(max_tokens=prompt, max_seq=total, batch=B)
    a.set_fused_decode(fused)
    step(a, 0, hp)
    for k in range(before):
        step(a, prompt + k, hs[k][:, None])
    pos = prompt + before
    assert a.position == pos
    saved = a.history().clone()
    b = dev.context(max_tokens=prompt, max_seq=total, batch=B)
    b.set_fused_decode(fused)
    b.history().copy_(saved)
    b.set_position(pos)
    assert b.position == pos
    for k in range(before, before + after):
        got = step(b, prompt + k, hs[k][:, None])
        want = step(a, prompt + k, hs[k][:, None])
        for i, (x, y) in enumerate(zip(got, want)):
            for u, v, what in zip(x, y, ("row ids", "rows", "kv", "highway")):
                np.testing.assert_array_equal(u, v, err_msg=f"step {k} layer {i}: {what}")
    a.check()
    b.check()
    torch.testing.assert_close(b.history(), a.history(), rtol=0, atol=0)


def test_map_host_refuses_unpinned_memory(E):
    """Only pinned host memory is mapped for the device; pageable memory is
    refused with E_ARG before any kernel could read it."""
    pinned = torch.zeros(4096, dtype=torch.uint8).pin_memory()
    assert E.map_host(pinned)
    with pytest.raises(E.EngramError) as ei:
        E.map_host(torch.zeros(4096, dtype=torch.uint8))
    assert ei.value.code == E.E_ARG


@pytest.mark.parametrize("name", [synth.DECODE_WKVQ2K.name, synth.ODD_WKVQ2K.name,
                                  synth.ODD_E4M3_WKVQ2K.name, synth.HC2_WKVQ2K.name])
def test_wkv_q2k_forward_matches_bf16_expansion(E, name):
    """Workloads with Q2_K wkv: every step through the kernels over the
    blocks (one launch or staged) leaves exactly what the bf16 kernels over
    the expanded wkv leave (row ids, rows, kv, highway) -- the pages'
    byte-identical results."""
    dev = Device(name)
    w = dev.w
    prompt, steps = 8, 24
    log(f"Q2_K wkv vs bf16 expansion: {w.name}, prompt {prompt} + {steps} steps")
    ids = G.token_ids(w, prompt + steps)
    hp = G.highway(w, prompt)
    hs = G.highway(w, steps, decode=True)
    res = []
    for blocks in (True, False):
        for fused in (True, False):
            ctx = dev.context(max_tokens=prompt, max_seq=prompt + steps)
            if not blocks:
                for l in range(w.n_layers):
                    ctx.set_wkv_q2k(l, None)
            ctx.set_fused_decode(fused)
            res.append(run_steps(dev, ctx, ids, steps, prompt, hp, hs))
            ctx.check()
    for r in res[1:]:
        for i, (a, b) in enumerate(zip(res[0], r)):
            for x, y, what in zip(a, b, ("row ids", "rows", "kv", "highway")):
                np.testing.assert_array_equal(x, y, err_msg=f"call {i}: {what}")


@pytest.mark.parametrize("name,B", [(synth.DECODE_Q2K.name, 2), (synth.DECODE_Q2K.name, 3),
                                    (synth.DECODE_Q2K.name, 4), (synth.ODD_Q2K.name, 3),
                                    (synth.ODD_E4M3.name, 4), (synth.MAX_SLOTS_Q2K.name, 3),
                                    (synth.MAX_NGRAM_E4M3.name, 2), (synth.HC1_Q2K.name, 4),
                                    (synth.HC3_E4M3.name, 3)])
def test_fused_batched_decode_matches_staged(E, name, B):
    """B sequences' decode steps through the one-launch several-sequence
    kernel leave exactly what the staged kernels leave (row ids, rows, kv,
    highway, bit for bit), and each sequence's kv equals a one-sequence run's
    (the projection adds in the one-token order)."""
    dev = Device(name)
    w = dev.w
    prompt, steps = 4, 12
    log(f"fused vs staged batched decode: {name}, B={B}")
    ids = G.token_ids(w, B * (prompt + steps)).reshape(B, prompt + steps)
    hp = G.highway(w, B * prompt).reshape(B, prompt, w.hc, w.dim)
    hs = G.highway(w, B * steps).reshape(steps, B, w.hc, w.dim)
    res = []
    for fused in (True, False):
        ctx = dev.context(max_tokens=prompt, max_seq=prompt + steps, batch=B)
        ctx.set_fused_decode(fused)
        d_ids = cuda(ids.astype(np.int32))
        out = []
        for step in range(1 + steps):
            T = prompt if step == 0 else 1
            p0 = 0 if step == 0 else prompt + step - 1
            h0 = hp if step == 0 else hs[step - 1][:, None]
            for layer in range(w.n_layers):
                d_h = torch.from_numpy(np.ascontiguousarray(h0)).cuda()
                ctx.forward(layer, d_ids[:, p0:p0 + T].contiguous() if layer == 0 else None, T, d_h)
                rid, rows, kv = ctx.views(T)
                out.append((rid.cpu().numpy(), to_np_u16(rows), to_np_u16(kv),
                            d_h.cpu().numpy().view(np.uint32)))
        ctx.check()
        res.append(out)
    for i, (a, b) in enumerate(zip(*res)):
        for x, y, what in zip(a, b, ("row ids", "rows", "kv", "highway")):
            np.testing.assert_array_equal(x, y, err_msg=f"call {i}: {what}")
    # one sequence alone (batch 1) gives the same kv for that sequence
    ctx = dev.context(max_tokens=prompt, max_seq=prompt + steps)
    d_ids = cuda(ids[B - 1].astype(np.int32))
    k = 0
    for step in range(1 + steps):
        T = prompt if step == 0 else 1
        p0 = 0 if step == 0 else prompt + step - 1
        h0 = hp[B - 1] if step == 0 else hs[step - 1][B - 1:B]
        for layer in range(w.n_layers):
            d_h = torch.from_numpy(np.ascontiguousarray(h0)).cuda()
            ctx.forward(layer, d_ids[p0:p0 + T] if layer == 0 else None, T, d_h)
            if step > 0:
                _, _, kv1 = ctx.views(T)
                np.testing.assert_array_equal(to_np_u16(kv1)[0], res[0][k][2][B - 1],
                                              err_msg=f"step {step} layer {layer}")
            k += 1
    ctx.check()


def test_fused_decode_bad_token(E):
    w = synth.TINY_E4M3
    dev = Device(w.name)
    ids = G.token_ids(w, 12).copy()
    unmapped = int(np.nonzero(dev.ht["token_map"] == -1)[0][0])
    bad = ids.copy()
    bad[9] = w.vocab + 7
    subst = ids.copy()
    subst[9] = unmapped
    ctx = dev.context(max_tokens=8, max_seq=12)
    hp, hs = G.highway(w, 8), G.highway(w, 4)
    out = run_steps(dev, ctx, bad, 4, 8, hp, hs)
    with pytest.raises(E.EngramError) as ei:
        ctx.check()
    assert ei.value.code == E.E_DEVICE
    want = dev.oracle_hasher(12).hash(subst, 0)
    for step in range(1, 5):
        np.testing.assert_array_equal(out[step][0], want[7 + step:8 + step])
