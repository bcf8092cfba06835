"""Engram hot-path benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

Headline: the decode workload (two Q2_K engram layers, 32-token prompt, then
single-token steps; wkv [20480, 6144] bf16 per layer).  One step = one token
through both layers via engram_forward: per layer one fused kernel (hash,
gather + dequant of the token's 24 rows, projection) and the gate.  `value` =
engram tokens/s per layer = steps * layers / seconds, inputs resident in HBM.
The same steps through the staged kernels (hash, gather, GEMV, gate) are
reported under "decode_staged".

Also measured in the same run: the decode workload with wkv as Q2_K blocks
("decode_wkv_q2k"), several sequences decoded together ("decode_batched"),
the prefill workload (T = 4096 Zipf tokens, both layers, one hash pass;
projection on the MFMA GEMM) under "prefill" with its own roofline, the
large-table gather workload (5.9 GB Q2_K table, T = 16384 uniform tokens;
gather + dequant GB/s apart from the GEMM) under "gather_stress", and the
e4m3 prefill/decode split (four 2048-token calls, then 128 single-token
steps) under "split_e4m3".

Per-kernel durations come from HIP events the runtime records with each
kernel dispatch (engram_ctx_set_timing) during a second pass over the same
steps; the plain pass gives `value`.  The roofline uses the projection
kernel: algorithmic bytes (decode) or flops (prefill GEMM) per launch divided
by its average event-timed duration.  `traffic` is read from the committed
rocprofv3 counter summary when it matches the current kernel source, else
null.

The oracle (plain C on the host cores) is timed on bounded samples of the
same workloads: the decode workload's first single-token steps (its own
token stream and per-step highways) for `cpu_baseline`, and the prefill
workload's first tokens for `prefill.cpu_baseline`.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
PROFILE_DIR = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "gram_hashed_embedding_engram_amd", "csrc")


def run_leg(name, fn):
    """One secondary leg of the run: its result, or -- if it raises -- an
    error entry, so that one failing leg (or the CPU baseline) does not take
    the measured ones and the line with them.  The traceback goes to stderr."""
    import traceback
    try:
        return fn()
    except Exception as e:           # the error is reported in the line and on stderr
        traceback.print_exc()
        log(f"{name}: failed: {type(e).__name__}: {e}")
        return {"error": f"{type(e).__name__}: {e}"}


def failed(r):
    return isinstance(r, dict) and "error" in r


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest(name):
    """First 16 hex digits of the SHA-256 of a kernel source followed by the
    library headers it includes (recursively, each once, in include order),
    with // comments and blank lines removed (a comment edit does not change
    the kernel)."""
    h = hashlib.sha256()
    seen = []

    def add(f):
        if f in seen:
            return
        seen.append(f)
        with open(os.path.join(CSRC, f)) as fh:
            for line in fh:
                m = re.match(r'\s*#include "([^"]+)"', line)
                if m and os.path.exists(os.path.join(CSRC, m.group(1))):
                    add(m.group(1))
                code = re.sub(r"//.*", "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")

    add(name)
    return h.hexdigest()[:16]


def counter_traffic(summary, kernel_src):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current source of the kernel."""
    path = os.path.join(PROFILE_DIR, summary)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_sha256_16:\s*([0-9a-f]{16})", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != source_digest(kernel_src):
        return None
    return float(t.group(1))


# VALU issue peak: 1024 SIMDs, one wave64 vector instruction every 4 cycles a
# SIMD (16 lanes a cycle), 2.4 GHz
VALU_PEAK_WAVE_INSTR = 1024 * 2.4e9 / 4


def counter_value(summary, kernel_src, key):
    """A per-launch figure (key: value) from a committed counter summary, if
    it was taken on the current source of the kernel."""
    path = os.path.join(PROFILE_DIR, summary)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_sha256_16:\s*([0-9a-f]{16})", text)
    t = re.search(key + r":\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != source_digest(kernel_src):
        return None
    return float(t.group(1))


def device_inputs(w, torch, E, G):
    ht = G.hash_tables(w)
    tm = torch.from_numpy(ht["token_map"]).cuda()
    tables = E.HashTables(tm, ht["pad_id"], ht["multipliers"], ht["primes"], ht["offsets"])
    layers = []
    host = []
    for l in range(w.n_layers):
        L = G.layer_inputs(w, ht, l)
        data = torch.from_numpy(L["table"]).cuda()
        scales = None if L["scales"] is None else torch.from_numpy(L["scales"]).cuda()
        tab = E.Table(data, scales, head_dim=w.head_dim, scale_block=w.scale_block)
        wkv = torch.from_numpy(L["wkv"].view(np.int16)).cuda()
        qk = torch.empty(w.hc, w.dim, dtype=torch.float32, device="cuda")
        E.qk_product(torch.from_numpy(L["q"].view(np.int16)).cuda(),
                     torch.from_numpy(L["k"].view(np.int16)).cuda(), qk)
        layers.append((tab, wkv, qk))
        host.append(L)
    torch.cuda.synchronize()
    return ht, tm, tables, layers, host


def host_table_inputs(w, inputs, torch, E):
    """The same inputs with every layer's table (and e4m3 scales) moved to
    pinned host memory, read by the kernels across the host link; wkv, qk
    and the hash tables stay on the device."""
    ht, tm, tables, layers, host = inputs
    out = []
    for (tab, *rest), L in zip(layers, host):
        data = torch.from_numpy(L["table"]).pin_memory()
        scales = None if L["scales"] is None else torch.from_numpy(L["scales"]).pin_memory()
        out.append((E.Table(data, scales, head_dim=w.head_dim, scale_block=w.scale_block),
                    *rest))
    return ht, tm, tables, out, host


def make_ctx(E, w, tables, layers, max_tokens, max_seq, batch=1):
    ctx = E.Context(tables, w.hc, w.dim, w.head_dim, w.eps, max_tokens, max_seq, batch=batch)
    for l, layer in enumerate(layers):
        tab, wkv, qk = layer[:3]
        ctx.add_layer(l, tab, wkv, qk)
        if len(layer) > 3:
            ctx.set_wkv_q2k(l, layer[3])
    ctx.reset()
    return ctx


def wkv_q2k_inputs(w, inputs, torch, E, G):
    """The decode inputs with each layer's wkv shipped as Q2_K blocks: the
    blocks on the device, and their bf16 expansion (the library's dequant)
    for the many-token prompt."""
    ht, tm, tables, layers, host = inputs
    out = []
    for l, (tab, _, qk) in enumerate(layers):
        blocks = torch.from_numpy(G.wkv_q2k(w, l)).cuda()
        wkv = torch.empty(w.N, w.K, dtype=torch.int16, device="cuda")
        E.dequant_q2k(blocks, wkv)
        out.append((tab, wkv, qk, blocks))
    torch.cuda.synchronize()
    return ht, tm, tables, out, host


def decode_q2kw_bytes(w):
    """Algorithmic bytes of one decode launch with wkv as Q2_K blocks: the
    blocks (84 B per 256 weights) instead of the bf16 wkv, the rest as in
    decode_bytes."""
    return decode_bytes(w) - w.N * w.K * 2 + w.N * (w.K // 256) * 84


def decode_bytes(w):
    """Algorithmic bytes of one fused decode launch (one token, one layer):
    wkv read once, the token's cols Q2_K blocks, kv written, the dequantised
    rows and the step's row ids written back, the token id, its token-map
    entry and max_ngram-1 history entries read, one history entry written."""
    return (w.N * w.K * 2 + w.cols * 84 + w.N * 2 + w.K * 2 + w.n_layers * w.cols * 8
            + 4 + 8 + 8 * w.max_ngram)


def bench_decode(args, torch, E, G, synth, fused=True, inputs=None, w=None):
    w = synth.DECODE_Q2K if w is None else w
    if inputs is None:
        log(f"decode: generating {w.name}")
        inputs = device_inputs(w, torch, E, G)
    ht, tm, tables, layers, host = inputs
    n_tok = w.prompt + 2 * (args.warmup + args.steps)
    ids = G.token_ids(w, n_tok)
    d_ids = torch.from_numpy(ids.astype(np.int32)).cuda()
    hw = torch.from_numpy(G.highway(w, w.decode_steps, decode=True)).cuda()
    prompt_h = torch.from_numpy(G.highway(w, w.prompt)).cuda()
    ctx = make_ctx(E, w, tables, layers, w.prompt, n_tok)
    ctx.set_fused_decode(fused)
    stream = torch.cuda.current_stream()
    nl = w.n_layers
    for l in range(nl):
        ctx.forward(l, d_ids[:w.prompt], w.prompt, prompt_h)
    pos = w.prompt

    def step(i):
        nonlocal pos
        h = hw[i % w.decode_steps:i % w.decode_steps + 1]
        for l in range(nl):
            ctx.forward(l, d_ids[pos:pos + 1], 1, h)
        pos += 1

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    host_ms = (time.perf_counter() - t0) * 1e3
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    # second pass over the same number of steps with per-stage events
    ctx.set_timing(True)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    stages = ctx.timing()
    ctx.set_timing(False)
    ctx.check()
    proj_ms, proj_n = stages["project"]
    res = dict(
        fused=fused,
        ms_per_step=ms / args.steps,
        host_ms_per_step=host_ms / args.steps,
        value=args.steps * nl / (ms / 1e3),
        proj_avg_ms=proj_ms / proj_n,
        proj_bytes=(decode_q2kw_bytes(w) if w.wkv_fmt == "q2k" else decode_bytes(w)) if fused
        else w.N * w.K * 2 + w.K * 2 + w.N * 2,
        stages={k: v[0] / max(1, v[1]) for k, v in stages.items() if v[1]},
        host=host, ht=ht, ids=ids,
    )
    if not fused:
        g_ms, g_n = stages["gather"]
        res["gather_GBps"] = w.cols * (84 + 512 + 8) / (g_ms / g_n / 1e3) / 1e9
    del ctx
    return res


def bench_decode_graph(args, torch, E, G, synth, inputs):
    """The decode workload's steps replayed from a hipGraph: after the prompt,
    graph mode moves the position to the device and one step (both layers'
    one-launch decode kernel and gate) is captured once; each timed step
    writes the next token id into the captured id buffer (a device copy) and
    replays the graph.  The highway buffer is the captured one, gated in place
    step after step."""
    w = synth.DECODE_Q2K
    ht, tm, tables, layers, host = inputs
    n_tok = w.prompt + 2 * args.warmup + args.steps + 1
    ids = G.token_ids(w, n_tok)
    d_ids = torch.from_numpy(ids.astype(np.int32)).cuda()
    prompt_h = torch.from_numpy(G.highway(w, w.prompt)).cuda()
    h = torch.from_numpy(G.highway(w, 1, decode=True)).cuda()
    ctx = make_ctx(E, w, tables, layers, w.prompt, n_tok)
    for l in range(w.n_layers):
        ctx.forward(l, d_ids[:w.prompt], w.prompt, prompt_h)
    ctx.set_graph_mode(True)
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for l in range(w.n_layers):
            ctx.forward(l, tok if l == 0 else None, 1, h)
    stream = torch.cuda.current_stream()
    pos = w.prompt

    def step(copy):
        nonlocal pos
        if copy:
            tok.copy_(d_ids[pos:pos + 1])
        g.replay()
        pos += 1

    def timed(copy, n):
        for _ in range(args.warmup):
            step(copy)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        t0 = time.perf_counter()
        for _ in range(n):
            step(copy)
        host = (time.perf_counter() - t0) * 1e3 / n
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / n, host

    half = args.steps // 2
    ms_copy, host_copy = timed(True, half)
    ms_replay, host_replay = timed(False, args.steps - half)
    ctx.check()
    ctx.set_graph_mode(False)
    assert ctx.position == pos, (ctx.position, pos)
    del g, ctx
    return dict(ms_per_step=ms_copy, value=w.n_layers / (ms_copy / 1e3),
                host_ms_per_step=host_copy, replay_only_ms_per_step=ms_replay,
                replay_only_host_ms_per_step=host_replay,
                unit="engram tokens/s per layer",
                how="one captured step (both layers) replayed per token, after a device copy "
                    "of the token id into the captured buffer (replay_only: the same buffer "
                    "content replayed, no copy)")


def bench_decode_batched(args, torch, E, G, synth, inputs, B):
    """B sequences decoded together on the decode workload's tables and
    weights: a prompt of w.prompt tokens each, then single-token steps, every
    step one pass over each layer's weights for B tokens.  Token ids: the
    decode workload's stream cut into B sequences."""
    w = synth.DECODE_Q2K
    ht, tm, tables, layers, host = inputs
    n_tok = w.prompt + 2 * (args.warmup + args.steps)
    ids = G.token_ids(w, n_tok * B).reshape(B, n_tok)
    d_ids = torch.from_numpy(ids.astype(np.int32)).cuda()
    hw = torch.from_numpy(G.highway(w, w.decode_steps, decode=True)).cuda()
    prompt_h = torch.from_numpy(G.highway(w, B * w.prompt)).cuda()
    ctx = make_ctx(E, w, tables, layers, w.prompt, n_tok, batch=B)
    stream = torch.cuda.current_stream()
    nl = w.n_layers
    for l in range(nl):
        ctx.forward(l, d_ids[:, :w.prompt].contiguous(), w.prompt, prompt_h)
    pos = w.prompt
    steps_h = [hw[(i * B) % (w.decode_steps - B):(i * B) % (w.decode_steps - B) + B]
               for i in range(max(args.steps, args.warmup))]
    step_ids = [d_ids[:, p:p + 1].contiguous() for p in range(n_tok)]

    def step(i):
        nonlocal pos
        for l in range(nl):
            ctx.forward(l, step_ids[pos], 1, steps_h[i])
        pos += 1

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    ctx.set_timing(True)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    stages = ctx.timing()
    ctx.check()
    del ctx
    return dict(sequences=B, ms_per_step=ms / args.steps,
                value=args.steps * B * nl / (ms / 1e3), unit="engram tokens/s per layer",
                stages_ms_per_layer_step={k: v[0] / max(1, v[1]) for k, v in stages.items()
                                          if v[1]})


def bench_prefill(args, torch, E, G, synth):
    w = synth.PREFILL_Q2K
    log(f"prefill: generating {w.name}")
    ht, tm, tables, layers, host = device_inputs(w, torch, E, G)
    T = w.prompt
    reps = args.prefill_steps
    warm = 3
    ids = G.token_ids(w)
    d_ids = torch.from_numpy(ids.astype(np.int32)).cuda()
    h = torch.from_numpy(G.highway(w, T)).cuda()
    ctx = make_ctx(E, w, tables, layers, T, T * (warm + 2 * reps))
    stream = torch.cuda.current_stream()

    def step():
        for l in range(w.n_layers):
            ctx.forward(l, d_ids, T, h)

    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    # an event between consecutive steps (one record per ~2 ms step) for the
    # per-step median beside the whole region's mean
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for i in range(reps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[reps])
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))
    ctx.set_timing(True)
    for _ in range(reps):
        step()
    torch.cuda.synchronize()
    stages = ctx.timing()
    ctx.check()
    flops = 2.0 * T * w.K * w.N
    gemm_ms = stages["project"][0] / stages["project"][1]
    gather_ms = stages["gather"][0] / stages["gather"][1]
    gate_ms = stages["gate"][0] / stages["gate"][1]
    tflops = flops / (gemm_ms / 1e3) / 1e12
    gate_bytes = T * w.hc * w.dim * 8 + T * w.N * 2
    return dict(
        workload=w.name, T=T, layers=w.n_layers, steps=reps, warmup=warm,
        ms_per_step=ms / reps,
        median_ms_per_step=per_step[reps // 2],
        value=reps * T * w.n_layers / (ms / 1e3),
        unit="engram tokens/s per layer",
        stages_ms={k: v[0] / max(1, v[1]) for k, v in stages.items()},
        roofline=dict(bound="mfma", achieved=tflops, peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                      frac=tflops / BF16_PEAK_TFLOPS,
                      traffic=counter_traffic("gemm_prefill_T4096_counters.md", "gemm.hip")),
        gather_GBps=T * w.cols * (84 + 512 + 8) / (gather_ms / 1e3) / 1e9,
        gate_GBps=gate_bytes / (gate_ms / 1e3) / 1e9,
        ht=ht, host=host,
    )


def bench_tiny(args, torch, E, G, synth, reps=50):
    """The small e4m3 workload (one layer, T 64, K 1024, N 1280): whole
    forwards, a correctness-sized configuration, so a rate without a roofline
    (launch latency bounds it)."""
    w = synth.TINY_E4M3
    ht, tm, tables, layers, host = device_inputs(w, torch, E, G)
    T = w.prompt
    d_ids = torch.from_numpy(G.token_ids(w).astype(np.int32)).cuda()
    h = torch.from_numpy(G.highway(w, T)).cuda()
    ctx = make_ctx(E, w, tables, layers, T, T * (reps + 3))
    stream = torch.cuda.current_stream()

    def forward():                    # the same 64 tokens again, at the next positions
        for l in range(w.n_layers):
            ctx.forward(l, d_ids, T, h)

    for _ in range(3):
        forward()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        forward()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    ctx.check()
    del ctx
    return dict(workload=w.name, T=T, layers=w.n_layers, forwards=reps, ms_per_forward=ms,
                value=T * w.n_layers / (ms / 1e3), unit="engram tokens/s per layer",
                note="correctness-sized: launch latency bounds it, no roofline claim")


def bench_gather_stress(args, torch, E, G, synth):
    """The large-table workload (one Q2_K layer of ~71 M rows, 5.9 GB; T
    16384 uniform tokens, so every row read is a random 84-byte block):
    whole forwards, with the gather + dequant rate reported apart from the
    projection GEMM."""
    w = synth.GATHER_Q2K
    log(f"gather stress: generating {w.name}")
    inputs = device_inputs(w, torch, E, G)
    ht, tm, tables, layers, host = inputs
    T = w.prompt
    reps, warm = args.stress_steps, 1
    ids = G.token_ids(w)
    d_ids = torch.from_numpy(ids.astype(np.int32)).cuda()
    h = torch.from_numpy(G.highway(w, T)).cuda()
    stream = torch.cuda.current_stream()

    def run(layers):
        ctx = make_ctx(E, w, tables, layers, T, T * (warm + 2 * reps))

        def step():
            for l in range(w.n_layers):
                ctx.forward(l, d_ids, T, h)

        for _ in range(warm):
            step()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(reps):
            step()
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end)
        ctx.set_timing(True)
        for _ in range(reps):
            step()
        torch.cuda.synchronize()
        stages = ctx.timing()
        ctx.check()
        del ctx
        return ms, {k: v[0] / max(1, v[1]) for k, v in stages.items()}

    gather_bytes = T * w.cols * (8 + 84 + w.head_dim * 2)
    ms, avg = run(layers)
    gbps = gather_bytes / (avg["gather"] / 1e3) / 1e9
    tflops = 2.0 * T * w.K * w.N / (avg["project"] / 1e3) / 1e12
    rows = int(ht["offsets"][0][-1] + ht["primes"][0][-1])
    res = dict(
        workload=w.name, T=T, layers=w.n_layers, table_rows=rows, table_bytes=rows * 84,
        ms_per_step=ms / reps, value=reps * T * w.n_layers / (ms / 1e3),
        unit="engram tokens/s per layer", stages_ms=avg,
        gather=dict(bound="hbm", kernel="gather_q2k_kernel (random 84-byte rows -> bf16)",
                    bytes_per_launch=gather_bytes, avg_launch_ms=avg["gather"],
                    achieved=gbps, peak=HBM_PEAK_GBPS, unit="GB/s", frac=gbps / HBM_PEAK_GBPS,
                    traffic=counter_traffic("gather_stress_counters.md", "gather.hip")),
        project=dict(bound="mfma", achieved=tflops, peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                     frac=tflops / BF16_PEAK_TFLOPS))
    if args.host_tables:
        # the same forwards with the 5.9 GB table in pinned host memory: the
        # gather's 84-byte row reads cross the host link
        del layers
        hinputs = host_table_inputs(w, inputs, torch, E)
        del inputs
        torch.cuda.empty_cache()
        ms_h, avg_h = run(hinputs[3])
        res["host_table"] = dict(
            ms_per_step=ms_h / reps, value=reps * T * w.n_layers / (ms_h / 1e3),
            stages_ms=avg_h, gather_table_GBps=T * w.cols * 84 / (avg_h["gather"] / 1e3) / 1e9,
            gather_GBps=gather_bytes / (avg_h["gather"] / 1e3) / 1e9)
    return res


def bench_split(args, torch, E, G, synth):
    """The e4m3 prefill/decode split: 8192 Zipf tokens as four 2048-token
    calls, then 128 single-token steps, both layers, the look-back carried
    across every call.  A pass starts from a reset history; tokens/s per
    layer reported for each phase."""
    w = synth.SPLIT_E4M3
    log(f"split: generating {w.name}")
    ht, tm, tables, layers, host = device_inputs(w, torch, E, G)
    del host
    ids = G.token_ids(w)
    d_ids = torch.from_numpy(ids.astype(np.int32)).cuda()
    chunks = [d_ids[c:c + w.chunk] for c in range(0, w.prompt, w.chunk)]
    steps = [d_ids[w.prompt + i:w.prompt + i + 1] for i in range(w.decode_steps)]
    hp = torch.from_numpy(G.highway(w, w.chunk)).cuda()
    hd = torch.from_numpy(G.highway(w, w.decode_steps, decode=True)).cuda()
    ctx = make_ctx(E, w, tables, layers, w.chunk, w.prompt + w.decode_steps)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    pre_ms = dec_ms = 0.0
    for p in range(1 + args.split_passes):
        ctx.reset()
        torch.cuda.synchronize()
        ev[0].record(stream)
        for c in chunks:
            for l in range(w.n_layers):
                ctx.forward(l, c, w.chunk, hp)
        ev[1].record(stream)
        for i, t in enumerate(steps):
            for l in range(w.n_layers):
                ctx.forward(l, t, 1, hd[i:i + 1])
        ev[2].record(stream)
        torch.cuda.synchronize()
        if p:
            pre_ms += ev[0].elapsed_time(ev[1])
            dec_ms += ev[1].elapsed_time(ev[2])
    ctx.check()
    del ctx
    n = args.split_passes
    return dict(
        workload=w.name, layers=w.n_layers, prompt=w.prompt, chunk=w.chunk,
        decode_steps=w.decode_steps, passes=n,
        prefill=dict(ms_per_chunk=pre_ms / (n * len(chunks)),
                     value=n * w.prompt * w.n_layers / (pre_ms / 1e3),
                     unit="engram tokens/s per layer"),
        decode=dict(ms_per_step=dec_ms / (n * w.decode_steps),
                    value=n * w.decode_steps * w.n_layers / (dec_ms / 1e3),
                    unit="engram tokens/s per layer"))


def read_ceiling(torch, E, synth, reps=30):
    """The device's practical read-stream rate: engram_stream_read over one
    layer's wkv bytes at the decode shape, three buffers in turn (768 MB,
    past the 256 MB last-level cache), so every launch reads HBM."""
    w = synth.DECODE_Q2K
    nbytes = w.N * w.K * 2
    bufs = [torch.full((nbytes // 4,), i + 1, dtype=torch.int32, device="cuda")
            for i in range(3)]
    sink = torch.zeros(E.STREAM_SINK_WORDS, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    for i in range(3):
        E.stream_read(bufs[i], sink, stream)
    torch.cuda.synchronize()
    # the launches straight through the C ABI, so host overhead stays far
    # below a launch's duration
    fn, s_ptr, k_ptr = E.lib().engram_stream_read, stream.cuda_stream, sink.data_ptr()
    ptrs = [b.data_ptr() for b in bufs]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(reps):
        fn(ptrs[i % 3], nbytes, k_ptr, s_ptr)
    end.record(stream)
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / reps
    del bufs
    return dict(kernel="stream_read_kernel (12 KiB rows, 1 KiB non-temporal loads, "
                       "no arithmetic)", bytes_per_launch=nbytes, avg_launch_us=us,
                GBps=nbytes / (us / 1e6) / 1e9, frac_of_peak=nbytes / (us / 1e6) / 1e9 /
                HBM_PEAK_GBPS)


def oracle_threads():
    """Host threads for the oracle: the CPUs this process may run on, capped
    by OMP_NUM_THREADS when set (the share of a shared host)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def layer_rows(oracle, w, L, rid):
    """The oracle's gather of one layer's rows for row ids [T, cols]."""
    return oracle.gather(L["table"], L["scales"], rid, w.head_dim, w.scale_block).reshape(
        rid.shape[0], -1)


def layer_wkv(oracle, L):
    return L["wkv"] if L.get("wkv_q2k") is None else oracle.expand_q2k_matrix(L["wkv_q2k"])


def cpu_baseline(w, ht, host, budget_s, max_steps=256, threads=None):
    """The oracle on the host cores over the workload's decode: its prompt,
    then single-token steps through every layer (hash, gather + dequant,
    projection, gate of that step's own highway), until budget_s seconds of
    steps have run or max_steps are done.  The token stream (prompt +
    max_steps ids) and the per-step highways are the workload's own, drawn
    here, so the sample does not depend on how many steps the GPU legs ran."""
    import oracle
    from synth import generate as G
    threads = threads or oracle_threads()
    ids = G.token_ids(w, w.prompt + max_steps)
    hw = G.highway(w, max_steps, decode=True)
    wkv = [layer_wkv(oracle, L) for L in host]
    hasher = oracle.Hasher(ht["token_map"], ht["pad_id"], ht["multipliers"], ht["primes"],
                           ht["offsets"], ids.size)
    hasher.hash(ids[:w.prompt], 0)
    pos, steps, el = w.prompt, 0, 0.0
    t0 = time.perf_counter()
    while steps < max_steps and (steps == 0 or el < budget_s):
        rid = hasher.hash(ids[pos:pos + 1], pos)
        h = hw[steps:steps + 1]
        for l in range(w.n_layers):
            L = host[l]
            rows = layer_rows(oracle, w, L, rid[:, l, :])
            kv = oracle.linear_bf16(rows, wkv[l], nthreads=threads)
            h = oracle.gate_and_add(h, kv, L["q"], L["k"], w.eps, nthreads=1)
        pos += 1
        steps += 1
        el = time.perf_counter() - t0
    return dict(value=steps * w.n_layers / el, unit="engram tokens/s per layer", cores=threads,
                kind="oracle", steps=steps, seconds=el,
                sample=f"the first {steps} single-token decode steps of {w.name} after its "
                       f"{w.prompt}-token prompt, every layer (hash, gather + dequant, "
                       f"projection, gate), {el:.1f} s")


def cpu_baseline_prefill(w, ht, host, sample_tokens=64, threads=None):
    """The oracle on the host cores over a bounded sample of the prefill
    workload: its first sample_tokens tokens as one call through every layer
    (one hash pass, then gather + dequant, projection and gate per layer).
    The tokens and highway are the first rows of the workload's own."""
    import oracle
    from synth import generate as G
    threads = threads or oracle_threads()
    S = sample_tokens
    ids = G.token_ids(w)[:S]
    h = np.ascontiguousarray(G.highway(w, w.prompt)[:S])
    wkv = [layer_wkv(oracle, L) for L in host]
    t0 = time.perf_counter()
    hasher = oracle.Hasher(ht["token_map"], ht["pad_id"], ht["multipliers"], ht["primes"],
                           ht["offsets"], S)
    rid = hasher.hash(ids, 0)
    for l in range(w.n_layers):
        L = host[l]
        rows = layer_rows(oracle, w, L, rid[:, l, :])
        kv = oracle.linear_bf16(rows, wkv[l], nthreads=threads)
        h = oracle.gate_and_add(h, kv, L["q"], L["k"], w.eps, nthreads=threads)
    el = time.perf_counter() - t0
    return dict(value=S * w.n_layers / el, unit="engram tokens/s per layer", cores=threads,
                kind="oracle", tokens=S, seconds=el,
                sample=f"the first {S} of the {w.prompt} tokens of {w.name} as one call, every "
                       f"layer (hash, gather + dequant, projection, gate), {el:.1f} s")


def q2kw_valu_roofline(avg_ms, w):
    """The Q2_K-wkv decode kernel against the vector-ALU issue peak: its
    wave64 VALU instructions per launch (committed counter summary, current
    source only) over the live average launch time."""
    instr = counter_value("decode_q2kw_counters.md", "decode.hip", "valu_instructions_per_launch")
    if instr is None:
        return None
    achieved = instr / (avg_ms / 1e3)
    return {"bound": "alu", "achieved": achieved / 1e9, "peak": VALU_PEAK_WAVE_INSTR / 1e9,
            "unit": "G wave64 VALU instructions/s", "frac": achieved / VALU_PEAK_WAVE_INSTR,
            "instructions_per_launch": instr,
            "lane_instructions_per_weight": instr * 64 / (w.N * w.K)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the many-token legs (prefill, gather stress, e4m3 split)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle decode steps for cpu_baseline")
    ap.add_argument("--cpu-prefill-tokens", type=int, default=64,
                    help="tokens of the prefill workload the oracle runs for "
                         "prefill.cpu_baseline")
    ap.add_argument("--batch-sequences", type=int, nargs="*", default=[4],
                    help="also decode this many sequences together (one weight pass per step)")
    ap.add_argument("--no-decode", action="store_true",
                    help="run only the prefill measurement (for counter passes)")
    ap.add_argument("--stress-steps", type=int, default=3)
    ap.add_argument("--split-passes", type=int, default=2)
    ap.add_argument("--only-stress", action="store_true",
                    help="run only the gather-stress measurement (for counter passes)")
    ap.add_argument("--host-tables", action="store_true",
                    help="also time decode and the gather stress with the tables in pinned "
                         "host memory (off by default: its launches of the same kernels would "
                         "mix into a kernel trace of the default run)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain elementwise copy of BYTES bytes (read BYTES, write "
                         "BYTES) three times: the calibration kernel for the HBM counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the engram path here runs on a single MI355X "
              "(no sharded or multi-GPU path is built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import gram_hashed_embedding_engram_amd as E
    import synth
    from synth import generate as G
    E.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_probe:
        n = args.copy_probe // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": 4 * n, "copy_probe_bytes_written": 4 * n,
                          "kernel": "torch.neg float32, 3 launches"}))
        return
    if args.no_decode:
        pre = bench_prefill(args, torch, E, G, synth)
        pre.pop("ht")
        pre.pop("host")
        print(json.dumps({"prefill": pre}), flush=True)
        return
    if args.only_stress:
        print(json.dumps({"gather_stress": bench_gather_stress(args, torch, E, G, synth)}),
              flush=True)
        return
    ceiling = read_ceiling(torch, E, synth)
    log(f"read ceiling: {ceiling['avg_launch_us']:.2f} us a launch, {ceiling['GBps']:.0f} GB/s")
    inputs = device_inputs(synth.DECODE_Q2K, torch, E, G)
    dec = bench_decode(args, torch, E, G, synth, fused=True, inputs=inputs)
    log(f"decode (fused): {dec['ms_per_step'] * 1e3:.1f} us/step, stages(ms) {dec['stages']}")
    staged = run_leg("decode (staged)", lambda: bench_decode(args, torch, E, G, synth,
                                                             fused=False, inputs=inputs))
    if not failed(staged):
        log(f"decode (staged): {staged['ms_per_step'] * 1e3:.1f} us/step, stages(ms) "
            f"{staged['stages']}")
    host_dec = None
    if args.host_tables:
        def host_leg():
            hinputs = host_table_inputs(synth.DECODE_Q2K, inputs, torch, E)
            return bench_decode(args, torch, E, G, synth, fused=True, inputs=hinputs)
        host_dec = run_leg("decode (host tables)", host_leg)
        if not failed(host_dec):
            log(f"decode (host tables): {host_dec['ms_per_step'] * 1e3:.1f} us/step, "
                f"stages(ms) {host_dec['stages']}")
    graph = run_leg("decode (graph replay)",
                    lambda: bench_decode_graph(args, torch, E, G, synth, inputs))
    if not failed(graph):
        log(f"decode (graph replay): {graph['ms_per_step'] * 1e3:.1f} us/step with the token "
            f"copy, {graph['replay_only_ms_per_step'] * 1e3:.1f} us/step replay only; host "
            f"{graph['host_ms_per_step'] * 1e3:.1f} / "
            f"{graph['replay_only_host_ms_per_step'] * 1e3:.1f} us/step (eager "
            f"{dec['host_ms_per_step'] * 1e3:.1f})")
    batched = []
    for B in args.batch_sequences:
        r = run_leg(f"decode ({B} sequences)",
                    lambda B=B: bench_decode_batched(args, torch, E, G, synth, inputs, B))
        if not failed(r):
            log(f"decode ({B} sequences): {r['ms_per_step'] * 1e3:.1f} us/step, "
                f"{r['value']:.0f} tokens/s per layer, stages(ms) {r['stages_ms_per_layer_step']}")
        batched.append(r)
    wq = synth.DECODE_WKVQ2K

    def q2kw_leg():
        qinputs = wkv_q2k_inputs(wq, inputs, torch, E, G)
        decq = bench_decode(args, torch, E, G, synth, fused=True, inputs=qinputs, w=wq)
        log(f"decode (Q2_K wkv): {decq['ms_per_step'] * 1e3:.1f} us/step, stages(ms) "
            f"{decq['stages']}")
        decq_staged = bench_decode(args, torch, E, G, synth, fused=False, inputs=qinputs, w=wq)
        log(f"decode (Q2_K wkv, staged): {decq_staged['ms_per_step'] * 1e3:.1f} us/step, "
            f"stages(ms) {decq_staged['stages']}")
        return {
            "workload": wq.name, "ms_per_step": decq["ms_per_step"], "value": decq["value"],
            "unit": "engram tokens/s per layer",
            "stages_ms_per_layer_step": decq["stages"],
            "kernel": "decode_q2kw_kernel<Q2K,6> (hash + gather/dequant + projection off the "
                      "Q2_K wkv blocks; vector-ALU bound)",
            "bytes_per_launch": decq["proj_bytes"], "avg_launch_ms": decq["proj_avg_ms"],
            "traffic": counter_traffic("decode_q2kw_counters.md", "decode.hip"),
            "hbm_GBps": decq["proj_bytes"] / (decq["proj_avg_ms"] / 1e3) / 1e9,
            "weights_per_s": wq.N * wq.K / (decq["proj_avg_ms"] / 1e3),
            "roofline": q2kw_valu_roofline(decq["proj_avg_ms"], wq),
            "staged": {"ms_per_step": decq_staged["ms_per_step"], "value": decq_staged["value"],
                       "stages_ms_per_layer_step": decq_staged["stages"]}}
    decode_wkv_q2k = run_leg("decode (Q2_K wkv)", q2kw_leg)
    del inputs
    pre = None
    if not args.no_prefill:
        pre = run_leg("prefill", lambda: bench_prefill(args, torch, E, G, synth))
        if not failed(pre):
            log(f"prefill: {pre['ms_per_step']:.3f} ms/step, stages(ms) {pre['stages_ms']}")
    stress = split = tiny = None
    if not args.no_prefill:
        tiny = run_leg("tiny", lambda: bench_tiny(args, torch, E, G, synth))
        if not failed(tiny):
            log(f"tiny: {tiny['ms_per_forward'] * 1e3:.1f} us a forward of {tiny['T']} tokens")
        stress = run_leg("gather stress", lambda: bench_gather_stress(args, torch, E, G, synth))
        if not failed(stress):
            log(f"gather stress: {stress['ms_per_step']:.3f} ms/step, gather "
                f"{stress['gather']['achieved']:.0f} GB/s, stages(ms) {stress['stages_ms']}")
        split = run_leg("split", lambda: bench_split(args, torch, E, G, synth))
        if not failed(split):
            log(f"split: prefill {split['prefill']['ms_per_chunk']:.3f} ms/chunk, decode "
                f"{split['decode']['ms_per_step'] * 1e3:.1f} us/step")
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on the host cores")
        cpu = run_leg("cpu baseline", lambda: cpu_baseline(synth.DECODE_Q2K, dec["ht"],
                                                           dec["host"], args.cpu_budget))
        if not failed(cpu):
            log(f"cpu baseline: {cpu['steps']} decode steps in {cpu['seconds']:.1f} s on "
                f"{cpu['cores']} threads")
        if pre and not failed(pre):
            pre["cpu_baseline"] = run_leg("cpu baseline (prefill)", lambda: cpu_baseline_prefill(
                synth.PREFILL_Q2K, pre["ht"], pre["host"], args.cpu_prefill_tokens))
            if not failed(pre["cpu_baseline"]):
                log(f"cpu baseline (prefill): {pre['cpu_baseline']['tokens']} tokens in "
                    f"{pre['cpu_baseline']['seconds']:.1f} s")
    if pre and not failed(pre):
        pre.pop("ht", None)
        pre.pop("host", None)
    w = synth.DECODE_Q2K
    gbps = dec["proj_bytes"] / (dec["proj_avg_ms"] / 1e3) / 1e9
    out = {
        "metric": "engram tokens/s per layer (decode T=1, prefill T=4096) + % HBM/MFMA roofline",
        "value_is": "decode T=1 on the decode workload (prefill T=4096: the prefill entry)",
        "value": dec["value"],
        "unit": "engram tokens/s per layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded generator; the pages publish no throughput to compare)",
        "config": {"workload": w.name, "layers": w.n_layers, "tokens_per_step": 1,
                   "prompt": w.prompt, "table": "q2k", "rows_per_layer": int(
                       dec["ht"]["rows"][0]), "K": w.K, "N": w.N, "hc": w.hc, "dim": w.dim},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS,
                     "traffic": counter_traffic("decode_kernel_counters.md", "decode.hip"),
                     "kernel": "decode_kernel<Q2K,12> (hash + gather/dequant + projection of "
                               "one layer for one token; one launch per layer-step)",
                     "bytes_per_launch": dec["proj_bytes"], "avg_launch_ms": dec["proj_avg_ms"],
                     "frac_of_read_ceiling": gbps / ceiling["GBps"]},
        "hbm_read_ceiling": ceiling,
        "stages_ms_per_layer_step": dec["stages"],
        "host_ms_per_step": dec["host_ms_per_step"],
        "decode_staged": staged if failed(staged) else {
            "ms_per_step": staged["ms_per_step"], "value": staged["value"],
            "stages_ms_per_layer_step": staged["stages"],
            "gemv_GBps": staged["proj_bytes"] / (staged["proj_avg_ms"] / 1e3) / 1e9,
            "gather_GBps": staged["gather_GBps"],
            "gemv_traffic": counter_traffic("gemv_decode_counters.md", "gemv.hip")},
        "decode_wkv_q2k": decode_wkv_q2k,
        "decode_graph": graph,
        "decode_host_tables": host_dec if host_dec is None or failed(host_dec) else {
            "tables": "pinned host memory, rows read across the host link",
            "ms_per_step": host_dec["ms_per_step"], "value": host_dec["value"],
            "unit": "engram tokens/s per layer",
            "stages_ms_per_layer_step": host_dec["stages"]},
        "decode_batched": batched,
        "prefill": pre,
        "tiny_e4m3": tiny,
        "gather_stress": stress,
        "split_e4m3": split,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
