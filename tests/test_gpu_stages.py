"""GPU parity of each C-ABI entry point against the oracle, on seeded
synthetic inputs (run on an MI355X).

Bars: hash ids and dequantised rows bit for bit; the projection within a
relative error of 1e-2 and the gated highway within 2e-3 (metric: _gpu_util
.relerr).  Shapes cover several tiles with ragged tails, the full workload
shapes (K = 6144, N = 20480, dim = 4096), and the degenerate cases (T = 0,
bad ids, unmapped windows).
"""
import numpy as np
import pytest

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


@pytest.fixture(scope="module")
def tiny(E):
    log("setup: tiny e4m3 workload")
    return Device(synth.TINY_E4M3.name)


@pytest.fixture(scope="module")
def decode(E):
    log("setup: decode Q2_K workload (2 layers, 4.6M rows, wkv 20480x6144)")
    return Device(synth.DECODE_Q2K.name)


def bf16_rand(rng, shape, std):
    x = (rng.standard_normal(shape) * std).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def cuda(a):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# ------------------------------------------------------------------ hash
def test_hash_batch_matches_per_sequence_oracle(E, decode):
    """B sequences hashed together, each against its own history row, over two
    calls (look-back across the calls), equal the oracle hasher run on each
    sequence alone."""
    w = decode.w
    B, T0, T1, max_seq = 5, 6, 3, 16
    rng = np.random.default_rng(17)
    ids = rng.integers(0, w.vocab, size=(B, T0 + T1)).astype(np.int32)
    ids[2, 4] = int(np.nonzero(decode.ht["token_map"] == -1)[0][0])    # an unmapped token
    hist = torch.zeros(B, max_seq, dtype=torch.int64, device="cuda")
    got = []
    for start, T in ((0, T0), (T0, T1)):
        out = torch.empty(B * T, w.n_layers, w.cols, dtype=torch.int64, device="cuda")
        E.hash_batch(decode.tables, cuda(ids[:, start:start + T]), start, hist, out)
        got.append(out.cpu().numpy().reshape(B, T, w.n_layers, w.cols))
    log(f"hash batch: B={B}, calls of {T0} and {T1} tokens")
    for b in range(B):
        h = decode.oracle_hasher(max_seq)
        want0 = h.hash(ids[b, :T0], 0)
        want1 = h.hash(ids[b, T0:], T0)
        np.testing.assert_array_equal(got[0][b], want0, err_msg=f"sequence {b} call 0")
        np.testing.assert_array_equal(got[1][b], want1, err_msg=f"sequence {b} call 1")


def run_hash(E, dev, ids, start, hist):
    T = ids.size
    out = torch.empty(T, dev.w.n_layers, dev.w.cols, dtype=torch.int64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    E.hash(dev.tables, cuda(ids.astype(np.int32)), start, hist, out, err)
    return out.cpu().numpy(), int(err.item())


def test_hash_tiny(E, tiny):
    log("hash: tiny T=64 single pass")
    ids = G.token_ids(tiny.w)
    hist = torch.zeros(256, dtype=torch.int64, device="cuda")
    got, err = run_hash(E, tiny, ids, 0, hist)
    want = tiny.oracle_hasher(256).hash(ids, 0)
    assert err == 0
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(hist[:64].cpu().numpy(), tiny.ht["token_map"][ids])


@pytest.mark.parametrize("seed", range(4))
def test_hash_chunked_equals_single_pass(E, tiny, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, tiny.w.vocab, size=300)
    cuts = np.unique(np.concatenate([[0, 300], rng.integers(0, 300, size=12)]))
    log(f"hash: tiny chunked at {cuts.tolist()}")
    hist = torch.zeros(300, dtype=torch.int64, device="cuda")
    parts = [run_hash(E, tiny, ids[a:b], a, hist)[0] for a, b in zip(cuts[:-1], cuts[1:])]
    want = tiny.oracle_hasher(300).hash(ids, 0)
    np.testing.assert_array_equal(np.concatenate(parts), want)


def test_hash_split_workload(E):
    """8192 Zipf tokens in 4 chunks of 2048, then 128 single-token steps: every
    call equals the single-pass hash of the 8320-token sequence."""
    import oracle
    w = synth.SPLIT_E4M3
    ht = G.hash_tables(w)
    tm = torch.from_numpy(ht["token_map"]).cuda()
    tables = E.HashTables(tm, ht["pad_id"], ht["multipliers"], ht["primes"], ht["offsets"])
    ids = G.token_ids(w)
    n = ids.size
    log(f"hash: split workload {n} tokens, 4x2048 + 128x1")
    hist = torch.zeros(n, dtype=torch.int64, device="cuda")
    d_ids = cuda(ids.astype(np.int32))
    out = torch.empty(n, w.n_layers, w.cols, dtype=torch.int64, device="cuda")
    bounds = [0, 2048, 4096, 6144, 8192] + list(range(8193, n + 1))
    for a, b in zip(bounds[:-1], bounds[1:]):
        E.hash(tables, d_ids[a:b], a, hist, out[a:b])
    chunked = out.cpu().numpy()
    hist2 = torch.zeros(n, dtype=torch.int64, device="cuda")
    out2 = torch.empty_like(out)
    E.hash(tables, d_ids, 0, hist2, out2)
    want = oracle.Hasher(ht["token_map"], ht["pad_id"], ht["multipliers"], ht["primes"],
                         ht["offsets"], n).hash(ids, 0)
    np.testing.assert_array_equal(out2.cpu().numpy(), want)
    np.testing.assert_array_equal(chunked, want)
    lo = ht["offsets"][None]
    assert (want >= lo).all() and (want < lo + ht["primes"][None]).all()


def test_hash_bad_token_ids(E, tiny):
    """An id outside the vocabulary raises the error bit and is hashed as an
    unmapped token; the oracle refuses it, so it is compared on the same
    stream with that id replaced by a vocabulary id that maps to -1."""
    ids = G.token_ids(tiny.w)[:40].copy()
    unmapped = int(np.nonzero(tiny.ht["token_map"] == -1)[0][0])
    bad = ids.copy()
    bad[[3, 17]] = [tiny.w.vocab, -5]
    subst = ids.copy()
    subst[[3, 17]] = unmapped
    hist = torch.zeros(64, dtype=torch.int64, device="cuda")
    got, err = run_hash(E, tiny, bad, 0, hist)
    assert err == E.DEVERR_TOKEN
    np.testing.assert_array_equal(got, tiny.oracle_hasher(64).hash(subst, 0))


def test_hash_degenerate_windows(E, tiny):
    """Degenerate n-gram windows, bit for bit against the oracle: every token
    unmapped (every window blocked at once), every token the pad token, and
    unmapped tokens every third position (windows blocked part way)."""
    tm = tiny.ht["token_map"]
    unmapped = np.nonzero(tm == -1)[0]
    mapped = np.nonzero(tm >= 0)[0]
    rng = np.random.default_rng(5)
    cases = {
        "all unmapped": rng.choice(unmapped, size=48),
        "all pad": np.zeros(48, dtype=np.int64),
        "every third unmapped": np.where(np.arange(48) % 3 == 1, rng.choice(unmapped, size=48),
                                         rng.choice(mapped, size=48)),
    }
    for name, ids in cases.items():
        hist = torch.zeros(64, dtype=torch.int64, device="cuda")
        got, err = run_hash(E, tiny, ids.astype(np.int32), 0, hist)
        assert err == 0, name
        np.testing.assert_array_equal(got, tiny.oracle_hasher(64).hash(ids, 0), err_msg=name)


def test_hash_large_moduli(E, tiny):
    """The 64-bit hash at the extremes of its arithmetic, bit for bit against
    the oracle: multipliers near 2^63 (the wrapping products use every bit),
    moduli from 2^31 - 1 up to 2^62 - 57 (the remainder of a full 64-bit
    value), the offsets' upper bound, and a long window (n-gram 8)."""
    import oracle
    tm_host = tiny.ht["token_map"]
    tm = torch.from_numpy(tm_host).cuda()
    for ng, nh in ((3, 2), (8, 1)):
        cols = (ng - 1) * nh
        rng = np.random.default_rng(ng)
        mult = ((rng.integers(2**62, 2**63 - 1, size=(1, ng), dtype=np.int64)) | 1)
        moduli = np.array([2**61 - 1, 2**31 - 1, 4294967291, 2**62 - 57, 1000000007,
                           2**40 + 15, 3, 2**62 - 1][:cols], dtype=np.int64).reshape(1, cols)
        offsets = (2**62 - moduli).reshape(1, cols)            # the largest allowed
        offsets[0, ::2] = np.arange(0, cols, 2)
        tables = E.HashTables(tm, tiny.ht["pad_id"], mult, moduli, offsets)
        ids = G.token_ids(tiny.w)[:40]
        hist = torch.zeros(64, dtype=torch.int64, device="cuda")
        out = torch.empty(40, 1, cols, dtype=torch.int64, device="cuda")
        E.hash(tables, cuda(ids.astype(np.int32)), 0, hist, out)
        want = oracle.Hasher(tm_host, tiny.ht["pad_id"], mult, moduli, offsets, 64).hash(ids, 0)
        np.testing.assert_array_equal(out.cpu().numpy(), want, err_msg=f"n-gram {ng}")
        assert (want >= 0).all() and (want < 2**62).all()


def test_hash_start_pos_and_empty(E, tiny):
    ids = G.token_ids(tiny.w)[:10]
    hist = torch.zeros(64, dtype=torch.int64, device="cuda")
    got, _ = run_hash(E, tiny, ids, 20, hist)
    np.testing.assert_array_equal(got, tiny.oracle_hasher(64).hash(ids, 20))
    out = torch.empty(0, 1, 4, dtype=torch.int64, device="cuda")
    E.hash(tiny.tables, torch.empty(0, dtype=torch.int32, device="cuda"), 0, hist, out)


# --------------------------------------------------------------- gather
def run_gather(E, dev, layer, ids2d, id_stride=None):
    T, cols = ids2d.shape
    id_stride = id_stride or cols
    full = np.zeros((T, id_stride), dtype=np.int64)
    full[:, :cols] = ids2d
    rows = torch.empty(T * cols, dev.w.head_dim, dtype=torch.int16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    E.gather_dequant(dev.tab[layer], cuda(full), T, cols, id_stride, rows, err)
    return to_np_u16(rows), int(err.item())


@pytest.mark.parametrize("T", [1, 5, 37, 300])
def test_gather_q2k(E, decode, T):
    rng = np.random.default_rng(T)
    for layer in range(2):
        n = decode.layers[layer]["rows"]
        ids = rng.integers(0, n, size=(T, 24))
        ids[0, :3] = [0, n - 1, n // 2]
        log(f"gather q2k: layer {layer} T={T}")
        got, err = run_gather(E, decode, layer, ids, id_stride=48)
        assert err == 0
        np.testing.assert_array_equal(got, decode.oracle_rows(layer, ids))


@pytest.mark.parametrize("T", [1, 7, 64])
def test_gather_e4m3(E, tiny, T):
    rng = np.random.default_rng(100 + T)
    n = tiny.layers[0]["rows"]
    ids = rng.integers(0, n, size=(T, 4))
    log(f"gather e4m3: T={T}")
    got, err = run_gather(E, tiny, 0, ids)
    assert err == 0
    np.testing.assert_array_equal(got, tiny.oracle_rows(0, ids))


def test_gather_every_tiny_row(E, tiny):
    n = tiny.layers[0]["rows"]
    ids = np.arange(n + (-n) % 4).reshape(-1, 4) % n
    got, _ = run_gather(E, tiny, 0, ids)
    np.testing.assert_array_equal(got, tiny.oracle_rows(0, ids))


def test_gather_e4m3_every_code(E):
    """Every e4m3 code (subnormals, signed zeros, the largest values and both
    NaN codes) under power-of-two scales 2^0 .. 2^-4 and scale blocks of 128
    and 16, gathered bit for bit as the oracle decodes them."""
    import oracle
    codes = np.tile(np.arange(256, dtype=np.uint8), (5, 1))          # row r: all codes
    for sb in (128, 16):
        nb = 256 // sb
        scales = np.array([[2.0 ** -((r + j) % 5) for j in range(nb)] for r in range(5)],
                          dtype=np.float32)
        tab = E.Table(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                      head_dim=256, scale_block=sb)
        ids = np.array([[4, 0, 3], [1, 2, 4]], dtype=np.int64)
        rows = torch.empty(6, 256, dtype=torch.int16, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        E.gather_dequant(tab, cuda(ids), 2, 3, 3, rows, err)
        assert int(err.item()) == 0
        want = oracle.gather(codes, scales, ids, 256, sb)
        np.testing.assert_array_equal(to_np_u16(rows), want, err_msg=f"scale block {sb}")


def test_gather_bad_row_ids(E, tiny, decode):
    for dev in (tiny, decode):
        n = dev.layers[0]["rows"]
        cols = dev.w.cols
        ids = np.tile(np.arange(cols, dtype=np.int64), (3, 1))
        ids[1, 2] = n
        ids[2, 0] = -1
        got, err = run_gather(E, dev, 0, ids)
        assert err == E.DEVERR_ROW
        got = got.reshape(3, cols, -1)
        assert (got[1, 2] == 0).all() and (got[2, 0] == 0).all()
        ok = ids.copy()
        ok[1, 2] = ok[2, 0] = 0
        want = dev.oracle_rows(0, ok).reshape(3, cols, -1)
        mask = np.ones((3, cols), bool)
        mask[1, 2] = mask[2, 0] = False
        np.testing.assert_array_equal(got[mask], want[mask])


# ----------------------------------------------------------- projection
def check_project(E, x, w_dev, w_host, sample_rows=None, sample_cols=None):
    import oracle
    T, K = x.shape
    N = w_host.shape[0]
    y = torch.empty(T, N, dtype=torch.int16, device="cuda")
    E.project(cuda(x), w_dev, y)
    got = to_np_u16(y)
    rows = np.arange(T) if sample_rows is None else sample_rows
    want = oracle.linear_bf16(x[rows], w_host)
    e = relerr(widen(got[rows]), widen(want))
    ulp = (got[rows] != want).mean()
    msg = f"rows: relerr {e:.2e}, {ulp:.2e} of outputs differ"
    if sample_cols is not None:
        want_c = oracle.linear_bf16(x, w_host[sample_cols])
        ec = relerr(widen(got[:, sample_cols]), widen(want_c))
        msg += f"; cols: relerr {ec:.2e}"
        assert ec <= 1e-2, msg
    log("  " + msg)
    assert e <= 1e-2, msg
    return got


@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_project_gemv_decode_shape(E, decode, T):
    rng = np.random.default_rng(T)
    ids = rng.integers(0, decode.layers[0]["rows"], size=(T, 24))
    x = decode.oracle_rows(0, ids).reshape(T, -1)
    log(f"project gemv: T={T} K=6144 N=20480")
    check_project(E, x, decode.wkv[0], decode.layers[0]["wkv"])


@pytest.mark.parametrize("M", [2, 5, 16, 17, 33, 64, 65, 100, 128])
def test_project_small_decode_shape(E, decode, M):
    """A few tokens (several sequences' decode tokens, short prompts) through
    the decode-shape wkv: the multi-token GEMV (M <= 4) or the MFMA GEMM laid
    out as a weight stream (twelve, eight or four wavefronts a workgroup up to
    128 tokens), every output checked (partial token tiles at M = 17, 33, 65,
    100)."""
    rng = np.random.default_rng(100 + M)
    ids = rng.integers(0, decode.layers[0]["rows"], size=(M, 24))
    x = decode.oracle_rows(0, ids).reshape(M, -1)
    log(f"project small: M={M} K=6144 N=20480")
    check_project(E, x, decode.wkv[0], decode.layers[0]["wkv"])


@pytest.mark.parametrize("M,K,N", [(5, 1024, 12320), (40, 1024, 12320), (24, 2048, 8208),
                                   (64, 3072, 4112), (100, 1024, 12320), (128, 2048, 1296)])
def test_project_few_token_ragged_rows(E, M, K, N):
    """The few-token GEMM where its row tiles do not divide among the
    workgroups (12320 outputs: 770 tiles of 16 in workgroups of 4, or of 5
    from five token tiles; 8208: 513 tiles in threes; 1296: 81 tiles in
    fives, the last workgroup one tile) and where the rows fit one workgroup a
    tile, with one to eight token tiles (twelve, eight and four wavefronts),
    against the oracle."""
    rng = np.random.default_rng(M * 31 + N)
    x = bf16_rand(rng, (M, K), 0.5)
    w = bf16_rand(rng, (N, K), 0.05)
    log(f"project few-token ragged: M={M} K={K} N={N}")
    check_project(E, x, cuda(w), w)


@pytest.mark.parametrize("T,K,N", [(2, 6144, 20480), (4, 6144, 20480), (3, 1280, 1008),
                                   (4, 8192, 2064), (2, 512, 16), (3, 1088, 4000)])
def test_project_multi_token_equals_one_token(E, T, K, N):
    """2..4 tokens in one pass over the weights: each token's outputs equal
    a one-token call's bit for bit (same summation order), and the oracle's
    within the projection tolerance.  K from one 1 KiB load a row to 8192 (and
    one not a multiple of 1024), N not a multiple of the 16 wavefronts of a
    workgroup."""
    import oracle
    rng = np.random.default_rng(1000 + 7 * T + K)
    x = bf16_rand(rng, (T, K), 1.0)
    w = bf16_rand(rng, (N, K), 0.02)
    d_w = cuda(w)
    y = torch.empty(T, N, dtype=torch.int16, device="cuda")
    log(f"project multi-token: T={T} K={K} N={N}")
    E.project(cuda(x), d_w, y)
    got = to_np_u16(y)
    for t in range(T):
        y1 = torch.empty(1, N, dtype=torch.int16, device="cuda")
        E.project(cuda(x[t:t + 1]), d_w, y1)
        np.testing.assert_array_equal(got[t], to_np_u16(y1)[0], err_msg=f"token {t}")
    want = oracle.linear_bf16(x, w)
    assert relerr(widen(got), widen(want)) <= 1e-2


@pytest.mark.parametrize("M", [2, 5, 64, 255, 257, 300, 513])
def test_project_gemm_tiny_shape(E, tiny, M):
    rng = np.random.default_rng(M)
    x = bf16_rand(rng, (M, tiny.w.K), 0.5)
    log(f"project gemm: M={M} K=1024 N=1280")
    check_project(E, x, tiny.wkv[0], tiny.layers[0]["wkv"])


@pytest.mark.parametrize("M,K,N", [(300, 64, 336), (257, 128, 16), (600, 192, 656),
                                   (5, 64, 32), (2, 64, 48), (1, 64, 16)])
def test_project_short_k(E, M, K, N):
    """The shortest contractions (K = 64..192: fewer K tiles than the GEMM's
    pipeline stages, so its prefetch runs past the end and reloads the last
    tile) at ragged M and N, on every projection kernel the token count
    selects, against the oracle."""
    rng = np.random.default_rng(M + K + N)
    x = bf16_rand(rng, (M, K), 0.5)
    w = bf16_rand(rng, (N, K), 0.05)
    log(f"project short K: M={M} K={K} N={N}")
    check_project(E, x, cuda(w), w)


@pytest.mark.parametrize("M", [32, 4096])
def test_project_gemm_full_shape(E, decode, M):
    """The prefill shape (and a 32-token call): sampled by strata so every
    256 x 320 output tile has a compared token row (all 20480 outputs) and a
    compared output column (all M tokens)."""
    rng = np.random.default_rng(7 + M)
    ids = rng.integers(0, decode.layers[1]["rows"], size=(M, 24))
    x = decode.oracle_rows(1, ids).reshape(M, -1)
    rows = tile_strata(M, GEMM_TILE_M, rng)
    cols = tile_strata(20480, GEMM_TILE_N, rng)
    assert_tiles_covered(rows, cols, M, 20480)
    log(f"project gemm: M={M} K=6144 N=20480 (sampled rows {rows.size}, cols {cols.size})")
    check_project(E, x, decode.wkv[1], decode.layers[1]["wkv"], rows, cols)


def test_project_gemm_token_tiles_agree(E, decode):
    """A few hundred tokens take 128-token tiles, more take 256-token ones;
    each output adds the same products in the same order either way, so 300
    tokens alone equal the same 300 tokens inside a 1100-token call bit for
    bit (and the oracle within the projection tolerance, on sampled rows)."""
    import oracle
    rng = np.random.default_rng(4242)
    ids = rng.integers(0, decode.layers[0]["rows"], size=(1100, 24))
    x = decode.oracle_rows(0, ids).reshape(1100, -1)
    big = torch.empty(1100, 20480, dtype=torch.int16, device="cuda")
    small = torch.empty(300, 20480, dtype=torch.int16, device="cuda")
    log("project: 300 tokens (128-token tiles) vs 1100 tokens (256-token tiles)")
    E.project(cuda(x), decode.wkv[0], big)
    E.project(cuda(x[400:700]), decode.wkv[0], small)
    np.testing.assert_array_equal(to_np_u16(small), to_np_u16(big)[400:700])
    rows = np.array([0, 127, 128, 255, 256, 299])
    want = oracle.linear_bf16(x[400:700][rows], decode.layers[0]["wkv"])
    assert relerr(widen(to_np_u16(small)[rows]), widen(want)) <= 1e-2


@pytest.mark.parametrize("M", [300, 1000, 4133])
def test_project_gemm_ragged_full_k(E, decode, M):
    """Token counts that leave a partly filled last 256-token tile, at the
    decode workload's K and N (6144, 20480), sampled by tile strata against
    the oracle: the tail rows read as zeros past M and are never stored."""
    rng = np.random.default_rng(17 + M)
    ids = rng.integers(0, decode.layers[0]["rows"], size=(M, 24))
    x = decode.oracle_rows(0, ids).reshape(M, -1)
    rows = tile_strata(M, GEMM_TILE_M, rng)
    cols = tile_strata(20480, GEMM_TILE_N, rng)
    assert_tiles_covered(rows, cols, M, 20480)
    log(f"project gemm ragged: M={M} K=6144 N=20480 (sampled rows {rows.size}, cols {cols.size})")
    check_project(E, x, decode.wkv[0], decode.layers[0]["wkv"], rows, cols)


def test_project_run_twice_bit_identical(E, decode):
    """Every projection kernel is deterministic: the same call twice gives
    the same bits, at the token counts that select each kernel (one-token
    GEMV, multi-token GEMV, few-token GEMM, tiled GEMM with a ragged tail and
    at the prefill shape)."""
    rng = np.random.default_rng(11)
    w = decode.wkv[1]
    for T in (1, 3, 8, 64, 100, 300, 4096):
        x = cuda(bf16_rand(rng, (T, 6144), 0.5))
        ys = []
        for _ in range(2):
            y = torch.full((T, 20480), 0x7FC0, dtype=torch.int16, device="cuda")
            E.project(x, w, y)
            ys.append(y)
        torch.cuda.synchronize()
        log(f"project twice: T={T}")
        assert torch.equal(ys[0], ys[1]), f"T={T}"


# ---------------------------------------------- projection off Q2_K wkv
def q2k_blocks(rng, n_out, nb):
    """Random Q2_K weight blocks [n_out, nb, 84] with fp16 d, dmin in the
    Q2_K-wkv recipe's range."""
    blk = rng.integers(0, 256, size=(n_out, nb, 84)).astype(np.uint8)
    blk[..., 80:84] = rng.uniform(1e-3, 2e-3, size=(n_out, nb, 2)).astype(
        np.float16).view(np.uint8)
    return blk


def test_dequant_q2k_exact(E):
    """The library's expansion of a Q2_K weight array equals the oracle's,
    bit for bit: a slice of the decode-shape wkv (984 blocks, not a multiple
    of the 64 a workgroup stages) and blocks with extreme fp16 scales."""
    import oracle
    w = synth.DECODE_WKVQ2K
    blocks = G.wkv_q2k(w, 0)[:41]                         # [41, 24, 84]
    rng = np.random.default_rng(5)
    extra = rng.integers(0, 256, size=(7, 84)).astype(np.uint8)
    for i, (d, dmin) in enumerate(((6e-8, 3e-8), (60000.0, 1.0), (1.0, 60000.0),
                                   (-2.0, 0.5), (0.0, 0.0), (1e-3, -1e-3), (65504.0, 65504.0))):
        extra[i, 80:82] = np.array([d], dtype=np.float16).view(np.uint8)
        extra[i, 82:84] = np.array([dmin], dtype=np.float16).view(np.uint8)
    flat = np.concatenate([blocks.reshape(-1, 84), extra])
    out = torch.empty(flat.shape[0] * 256, dtype=torch.int16, device="cuda")
    log(f"dequant_q2k: {flat.shape[0]} blocks")
    E.dequant_q2k(torch.from_numpy(flat).cuda(), out)
    want = oracle.expand_q2k_matrix(flat[:, None, :]).reshape(-1)
    np.testing.assert_array_equal(to_np_u16(out), want)


def check_project_q2k(E, x, blocks_host, blocks_dev=None, expanded=None, sample=None):
    """The projection off the blocks against the oracle (over the oracle's
    expansion) within the projection tolerance, and against the library's
    bf16 GEMV over the library's expansion of the same blocks bit for bit (the
    pages claim byte-identical results for the two)."""
    import oracle
    K = x.shape[1]
    N = blocks_host.shape[0]
    if blocks_dev is None:
        blocks_dev = torch.from_numpy(np.ascontiguousarray(blocks_host)).cuda()
    y = torch.empty(1, N, dtype=torch.int16, device="cuda")
    E.project_q2k(cuda(x), blocks_dev, y)
    got = to_np_u16(y)[0]
    # engram_project takes N in multiples of 16: zero blocks pad the rows
    n16 = -(-N // 16) * 16
    padded = torch.zeros(n16, K // 256, 84, dtype=torch.uint8, device="cuda")
    padded[:N] = blocks_dev.view(N, K // 256, 84)
    bf = torch.empty(n16, K, dtype=torch.int16, device="cuda")
    E.dequant_q2k(padded, bf)
    y_bf = torch.empty(1, n16, dtype=torch.int16, device="cuda")
    E.project(cuda(x), bf, y_bf)
    np.testing.assert_array_equal(got, to_np_u16(y_bf)[0, :N],
                                  err_msg="Q2_K-wkv projection differs from the bf16 GEMV")
    del padded
    del bf
    rows = np.arange(N) if sample is None else sample
    w = oracle.expand_q2k_matrix(blocks_host[rows]) if expanded is None else expanded[rows]
    want = oracle.linear_bf16(x, w)[0]
    e = relerr(widen(got[rows]), widen(want))
    diff = (got[rows] != want).mean()
    log(f"  relerr {e:.2e}, {diff:.2e} of outputs differ from the oracle's bits")
    assert e <= 1e-2
    return got


def test_project_q2k_decode_shape(E):
    """One token of dequantised table rows through the decode-shape Q2_K wkv
    (K 6144, N 20480), every output checked."""
    import oracle
    w = synth.DECODE_WKVQ2K
    dev = Device(w.name)
    rng = np.random.default_rng(21)
    ids = rng.integers(0, dev.layers[0]["rows"], size=(1, 24))
    x = dev.oracle_rows(0, ids).reshape(1, -1)
    log("project_q2k: K=6144 N=20480")
    check_project_q2k(E, x, dev.layers[0]["wkv_q2k"], dev.wkvq[0], dev.oracle_wkv(0))


@pytest.mark.parametrize("K,N", [(256, 7), (1280, 1000), (1024, 1), (8192, 515), (3072, 4097)])
def test_project_q2k_ragged(E, K, N):
    """K from one block to the 8192 limit (lanes left idle, partial sub-block
    rounds) and N not a multiple of the wavefronts in the grid."""
    rng = np.random.default_rng(K + N)
    blocks = q2k_blocks(rng, N, K // 256)
    x = bf16_rand(rng, (1, K), 1.0)
    log(f"project_q2k: K={K} N={N}")
    check_project_q2k(E, x, blocks)


def test_project_q2k_empty(E):
    x = torch.empty(0, 1024, dtype=torch.int16, device="cuda")
    y = torch.empty(0, 64, dtype=torch.int16, device="cuda")
    E.project_q2k(x, torch.empty(64, 4, 84, dtype=torch.uint8, device="cuda"), y)


def test_project_empty(E, tiny):
    x = torch.empty(0, tiny.w.K, dtype=torch.int16, device="cuda")
    y = torch.empty(0, tiny.w.N, dtype=torch.int16, device="cuda")
    E.project(x, tiny.wkv[0], y)


# ----------------------------------------------------------------- gate
def test_qk_product_exact(E, decode):
    L = decode.layers[0]
    want = widen(L["q"]) * widen(L["k"])
    np.testing.assert_array_equal(decode.qk[0].cpu().numpy().view(np.uint32),
                                  want.view(np.uint32))


@pytest.mark.parametrize("T,hc,dim", [(64, 4, 256), (1, 4, 4096), (37, 3, 4096), (5, 2, 768),
                                      (3, 1, 4352), (9, 4, 1024), (4096, 4, 4096), (2, 2, 8192),
                                      (3, 2, 9216)])
def test_gate(E, T, hc, dim):
    import oracle
    rng = np.random.default_rng(T * 7 + dim)
    h = rng.standard_normal((T, hc, dim)).astype(np.float32)
    kv = bf16_rand(rng, (T, dim * (hc + 1)), 0.5)
    q = bf16_rand(rng, (hc, dim), 0.05)
    k = bf16_rand(rng, (hc, dim), 0.05)
    q = (widen(q) + 1).astype(np.float32)
    k = (widen(k) + 1).astype(np.float32)
    qb = torch.from_numpy(q).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    kb = torch.from_numpy(k).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    d_qk = torch.empty(hc, dim, dtype=torch.float32, device="cuda")
    E.qk_product(cuda(qb), cuda(kb), d_qk)
    d_h = torch.from_numpy(h).cuda()
    log(f"gate: T={T} hc={hc} dim={dim}")
    E.gate_apply(d_h, cuda(kv), d_qk, 1e-6)
    got = d_h.cpu().numpy()
    want = oracle.gate_and_add(h, kv, qb, kb, 1e-6)
    e = relerr(got, want)
    log(f"  relerr {e:.2e}")
    assert e <= 2e-3
    # value = 0 leaves h bit for bit
    kv0 = kv.reshape(T, hc + 1, dim).copy()
    kv0[:, hc] = 0
    d_h = torch.from_numpy(h).cuda()
    E.gate_apply(d_h, cuda(kv0.reshape(T, -1)), d_qk, 1e-6)
    np.testing.assert_array_equal(d_h.cpu().numpy().view(np.uint32), h.view(np.uint32))


def test_gate_degenerate_rows(E):
    """The gate's degenerate inputs against the oracle: a zero highway row
    (h.h = 0, the eps floor sets the norm), a zero key (key.key = 0), a key
    orthogonal to h.qk (the dot 0: the signed square root's 1e-6 clamp decides
    the gate), and huge values (1e30, squares overflow to inf in f32)."""
    import oracle
    hc, dim, T = 4, 256, 4
    rng = np.random.default_rng(3)
    h = rng.standard_normal((T, hc, dim)).astype(np.float32)
    kv = bf16_rand(rng, (T, hc + 1, dim), 0.5)
    h[0, 1] = 0.0                                   # zero highway row
    kv[1, 2] = 0                                    # zero key
    kv[2, 0, ::2] = 0                               # key on odd positions ...
    h[2, 0, 1::2] = 0.0                             # ... h on even ones: dot = 0
    h[3, 3] = np.float32(1e30)                      # squares overflow
    q = np.full((hc, dim), 0x3F80, dtype=np.uint16)  # q = k = 1
    d_qk = torch.empty(hc, dim, dtype=torch.float32, device="cuda")
    E.qk_product(cuda(q), cuda(q), d_qk)
    d_h = torch.from_numpy(h).cuda()
    E.gate_apply(d_h, cuda(kv.reshape(T, -1)), d_qk, 1e-6)
    got = d_h.cpu().numpy()
    want = oracle.gate_and_add(h, kv.reshape(T, -1), q, q, 1e-6)
    finite = np.isfinite(want)
    np.testing.assert_array_equal(np.isfinite(got), finite)
    rows = [(0, 1), (1, 2), (2, 0)]
    for t, c in rows:
        e = relerr(got[t, c], want[t, c])
        assert e <= 2e-3, f"row {(t, c)}: relerr {e:.2e}"


@pytest.mark.parametrize("dim", [4096, 9216])
def test_gate_rows_independent_of_T(E, dim):
    """A token's gated rows are the same bits whether it is gated alone
    (decode) or inside a batch (prefill): the reduction order is per row."""
    rng = np.random.default_rng(dim)
    T, hc = 6, 4
    h = rng.standard_normal((T, hc, dim)).astype(np.float32)
    kv = bf16_rand(rng, (T, dim * (hc + 1)), 0.5)
    d_qk = torch.from_numpy(rng.standard_normal((hc, dim)).astype(np.float32) * 0.05).cuda()
    d_all = torch.from_numpy(h).cuda()
    E.gate_apply(d_all, cuda(kv), d_qk, 1e-6)
    for t in (0, 5):
        d_one = torch.from_numpy(h[t:t + 1].copy()).cuda()
        E.gate_apply(d_one, cuda(kv[t:t + 1].copy()), d_qk, 1e-6)
        np.testing.assert_array_equal(d_one.cpu().numpy().view(np.uint32),
                                      d_all[t:t + 1].cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("rows", [1, 37, 20480])
def test_stream_read_folds_every_word(E, rows):
    """The read-rate yardstick reads every word of its buffer exactly once:
    the XOR of its sink words equals the XOR of all the buffer's 32-bit
    words (1 row: most wavefronts have no row; 20480 rows: one layer's wkv
    bytes at the decode shape)."""
    rng = np.random.default_rng(rows)
    words = rows * E.STREAM_ROW_BYTES // 4
    src = rng.integers(0, 2**32, size=words, dtype=np.uint64).astype(np.uint32)
    want = np.bitwise_xor.reduce(src)
    d_src = torch.from_numpy(src.view(np.int32)).cuda()
    sink = torch.full((E.STREAM_SINK_WORDS,), -1, dtype=torch.int32, device="cuda")
    E.stream_read(d_src, sink)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want, f"{got:#x} != {want:#x}"
