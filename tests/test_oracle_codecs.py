"""Pins of the oracle's number formats and row dequantisers (stage 2) against
library routines and independent re-derivations:

* bf16 rounding vs torch's float32 -> bfloat16 cast (round to nearest even);
* fp16 decode, all 65536 codes, vs numpy's float16 -> float32;
* e4m3 decode, all 256 codes, vs torch's float8_e4m3fn;
* e4m3 encode vs torch's cast inside the e4m3 range, and the pages' special
  cases (NaN -> 0x7F, saturation to 0x7E, subnormals, ties to even)
  (metrale "deepseek_v41_ref/engram.rs", f32_to_e4m3_rne / e4m3_to_f32);
* e4m3 times a power of two is exact in bf16 (metrale module doc, stage 2);
* Q2_K rows: designed blocks built by an encoder written here in the
  streaming form of the k-quant block (two 128-halves, four 2-bit planes,
  two 16-value runs per plane), and random blocks decoded by a second
  decoder of that same streaming form with numpy float32 arithmetic and
  torch's bf16 cast.
"""
import numpy as np
import pytest
import torch


def torch_bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    edge = np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.4028235e38, -3.4028235e38,
                     1e-45, -1e-45, 1.1754944e-38, 1.00390625, 1.01171875, 1.0078125,
                     1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 65504.0], dtype=np.float32)
    # exact ties: low 16 bits == 0x8000 with even and odd kept parts
    ties = (np.arange(0, 4096, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    for arr in (x, edge, ties):
        np.testing.assert_array_equal(orc.bf16_from_f32(arr), torch_bf16_bits(arr))


def test_f16_decode_exhaustive(orc):
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    want = codes.view(np.float16).astype(np.float32)
    got = np.array([orc.f32_from_f16(int(c)) for c in codes], dtype=np.float32)
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all()
    np.testing.assert_array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_e4m3_decode_exhaustive(orc):
    codes = torch.arange(256, dtype=torch.int16).to(torch.uint8)
    want = codes.view(torch.float8_e4m3fn).float().numpy()
    got = np.array([orc.e4m3_to_f32(c) for c in range(256)], dtype=np.float32)
    nan = np.isnan(want)
    assert nan.sum() == 2 and (np.isnan(got) == nan).all()
    np.testing.assert_array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_e4m3_encode(orc):
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000), rng.standard_normal(5000) * 100,
                        rng.standard_normal(5000) * 0.01]).astype(np.float32)
    x = np.clip(x, -448, 448)
    # every e4m3 value, and every midpoint between neighbours (ties)
    vals = np.array([orc.e4m3_to_f32(c) for c in range(256)], dtype=np.float64)
    pos = np.unique(vals[np.isfinite(vals) & (vals >= 0)])
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, pos.astype(np.float32), mids, -mids])
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.f32_to_e4m3_rne(float(v)) for v in x], dtype=np.uint8)
    np.testing.assert_array_equal(got, want)
    # the pages' own special cases
    assert orc.f32_to_e4m3_rne(float("nan")) == 0x7F
    assert orc.f32_to_e4m3_rne(449.0) == 0x7E and orc.f32_to_e4m3_rne(1e6) == 0x7E
    assert orc.f32_to_e4m3_rne(-1e6) == 0xFE
    assert orc.f32_to_e4m3_rne(1e-40) == 0x00 and orc.f32_to_e4m3_rne(-1e-40) == 0x80
    assert orc.f32_to_e4m3_rne(2.0 ** -6) == 0x08          # first normal
    assert orc.f32_to_e4m3_rne(2.0 ** -10) == 0x00         # tie to even (0)
    assert orc.f32_to_e4m3_rne(3 * 2.0 ** -10) == 0x02     # tie to even (2)


def test_e4m3_times_pow2_exact_in_bf16(orc):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    exact = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    for k in range(-4, 1):
        for block in (32, 128, 256):
            row = np.resize(codes, 256).astype(np.uint8)
            scales = np.full(256 // block, 2.0 ** k, dtype=np.float32)
            out = orc.e4m3_row(row, scales, block)
            got = orc.f32_from_bf16(out).astype(np.float64)
            want = np.resize(exact, 256) * 2.0 ** k
            np.testing.assert_array_equal(got, want)
            # -0 stays -0
            assert (out[np.resize(codes, 256) == 0x80] == 0x8000).all()


def test_e4m3_row_mixed_scales(orc):
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 256, size=256).astype(np.uint8)
    codes[codes == 0x7F] = 0x7E
    codes[codes == 0xFF] = 0xFE
    scales = np.array([0.25, 0.0625], dtype=np.float32)
    out = orc.e4m3_row(codes, scales, 128)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    want = dec * np.repeat(scales.astype(np.float64), 128)
    np.testing.assert_array_equal(orc.f32_from_bf16(out).astype(np.float64), want)


# ------------------------------------------------------------------- Q2_K
def encode_q2k(Q, sc, mn, d, dmin):
    """84-byte block in the k-quant streaming order: for each 128-value half
    (32 quant bytes), four 2-bit planes (shift 0, 2, 4, 6), each plane two runs
    of 16 values (quant bytes 0..15, then 16..31); every run of 16 takes the
    next scale byte (low nibble scale, high nibble min)."""
    blk = np.zeros(84, dtype=np.uint8)
    out = 0
    for half in range(2):
        for shift in (0, 2, 4, 6):
            for run in (0, 16):
                j = out // 16
                blk[j] = (sc[j] & 15) | ((mn[j] & 15) << 4)
                for l in range(16):
                    blk[16 + 32 * half + run + l] |= (int(Q[out]) & 3) << shift
                    out += 1
    blk[80:82] = np.array([d], dtype=np.float16).view(np.uint8)
    blk[82:84] = np.array([dmin], dtype=np.float16).view(np.uint8)
    return blk


def decode_q2k_stream(blk):
    """Second decoder, same streaming order, numpy float32 arithmetic and
    torch's bf16 cast."""
    d = blk[80:82].view(np.float16)[0].astype(np.float32)
    dmin = blk[82:84].view(np.float16)[0].astype(np.float32)
    y = np.zeros(256, dtype=np.float32)
    out = 0
    for half in range(2):
        for shift in (0, 2, 4, 6):
            for run in (0, 16):
                s = blk[out // 16]
                dl = d * np.float32(s & 15)
                ml = dmin * np.float32(s >> 4)
                for l in range(16):
                    q = np.float32((int(blk[16 + 32 * half + run + l]) >> shift) & 3)
                    y[out] = dl * q - ml
                    out += 1
    return torch_bf16_bits(y)


def f32_bits_of(v):
    return torch_bf16_bits(np.asarray(v, dtype=np.float32))


def test_q2k_quant_positions(orc):
    rng = np.random.default_rng(3)
    Q = rng.integers(0, 4, size=256)
    blk = encode_q2k(Q, np.ones(16, int), np.zeros(16, int), 1.0, 0.0)
    np.testing.assert_array_equal(orc.q2k_row(blk), f32_bits_of(Q))


def test_q2k_scale_mapping(orc):
    Q = np.random.default_rng(4).integers(0, 4, size=256)
    j = np.arange(256) // 16
    for sc in (np.arange(16), 15 - np.arange(16)):
        blk = encode_q2k(Q, sc, np.zeros(16, int), 1.0, 0.0)
        np.testing.assert_array_equal(orc.q2k_row(blk), f32_bits_of(sc[j] * Q))


def test_q2k_min_mapping(orc):
    Q = np.random.default_rng(5).integers(0, 4, size=256)
    j = np.arange(256) // 16
    blk = encode_q2k(Q, np.zeros(16, int), 15 - np.arange(16), 0.0, 1.0)
    want = -(15 - j).astype(np.float32)
    want[want == 0] = 0.0          # sub-block 15: 0 - 0 = +0
    got = orc.q2k_row(blk)
    np.testing.assert_array_equal(got, f32_bits_of(want))
    assert (got[j == 15] == 0x0000).all()


def test_q2k_zero_block(orc):
    blk = encode_q2k(np.full(256, 3), np.full(16, 15), np.full(16, 15), 0.0, 0.0)
    assert (orc.q2k_row(blk) == 0).all()


def test_q2k_round_trip(orc):
    rng = np.random.default_rng(6)
    for _ in range(20):
        Q = rng.integers(0, 4, size=256)
        blk = encode_q2k(Q, np.ones(16, int), np.zeros(16, int), 1.0, 0.0)
        back = orc.f32_from_bf16(orc.q2k_row(blk)).astype(int)
        np.testing.assert_array_equal(back, Q)


def test_q2k_random_blocks(orc):
    """Random bytes with fp16 d/dmin in U(1e-3, 1e-2) (the tables' recipe)."""
    rng = np.random.default_rng(7)
    for _ in range(300):
        blk = rng.integers(0, 256, size=84).astype(np.uint8)
        dd = rng.uniform(1e-3, 1e-2, size=2).astype(np.float16)
        blk[80:84] = dd.view(np.uint8)
        np.testing.assert_array_equal(orc.q2k_row(blk), decode_q2k_stream(blk))


def test_q2k_extreme_scales(orc):
    """fp16 subnormal and large d/dmin still decode by the same rule."""
    rng = np.random.default_rng(8)
    for d, dmin in ((6e-8, 3e-8), (60000.0, 1.0), (1.0, 60000.0), (-2.0, 0.5)):
        blk = rng.integers(0, 256, size=84).astype(np.uint8)
        blk[80:82] = np.array([d], dtype=np.float16).view(np.uint8)
        blk[82:84] = np.array([dmin], dtype=np.float16).view(np.uint8)
        np.testing.assert_array_equal(orc.q2k_row(blk), decode_q2k_stream(blk))


def test_gather_bounds(orc):
    tab = np.zeros((4, 84), dtype=np.uint8)
    with pytest.raises(ValueError):
        orc.gather(tab, None, np.array([4]))
    with pytest.raises(ValueError):
        orc.gather(tab, None, np.array([-1]))
    rows = orc.gather(tab, None, np.array([[0, 3], [2, 1]]))
    assert rows.shape == (4, 256)


# ------------------------------------------- wkv shipped as Q2_K blocks
def test_expand_q2k_matrix_layout(orc):
    """Block b of output row o must land on columns [256b, 256b+256) of row o.
    Designed blocks: zero quants, min nibble 1, scale 0, dmin = (16o+b+1)/64,
    so every value of block (o, b) is -(16o+b+1)/64 (exact in bf16)."""
    out_f, nb = 3, 4
    blocks = np.zeros((out_f, nb, 84), dtype=np.uint8)
    for o in range(out_f):
        for b in range(nb):
            blocks[o, b] = encode_q2k(np.zeros(256, int), np.zeros(16, int), np.ones(16, int),
                                      0.0, (16 * o + b + 1) / 64)
    w = orc.f32_from_bf16(orc.expand_q2k_matrix(blocks))
    assert w.shape == (out_f, nb * 256)
    want = -(16 * np.arange(out_f)[:, None] + np.arange(nb * 256)[None, :] // 256 + 1) / 64
    np.testing.assert_array_equal(w, want.astype(np.float32))


def test_expand_q2k_matrix_values_within_block(orc):
    """Inside a block the expansion follows the block's own value order: a block
    whose quants count 0,1,2,3,0,... with scale 1, min 0, d 1 expands to that
    count at every position of the row it sits in."""
    Q = np.arange(256) % 4
    blk = encode_q2k(Q, np.ones(16, int), np.zeros(16, int), 1.0, 0.0)
    blocks = np.stack([np.stack([blk, blk])] * 2)          # [2, 2, 84]
    w = orc.f32_from_bf16(orc.expand_q2k_matrix(blocks))
    np.testing.assert_array_equal(w, np.tile(Q, (2, 2)).astype(np.float32))


def test_project_q2k_contracts_over_inputs(orc):
    """A one-hot token at input k returns column k of the expanded matrix, for
    every output row (the input axis is the block axis, not the output axis)."""
    rng = np.random.default_rng(11)
    out_f, nb = 5, 3
    blocks = rng.integers(0, 256, size=(out_f, nb, 84)).astype(np.uint8)
    blocks[..., 80:84] = rng.uniform(1e-3, 2e-3, size=(out_f, nb, 2)).astype(
        np.float16).view(np.uint8)
    w = orc.expand_q2k_matrix(blocks)
    for k in (0, 255, 256, 700):
        x = np.zeros((1, nb * 256), dtype=np.float32)
        x[0, k] = 1.0
        y = orc.project_q2k(torch_bf16_bits(x).reshape(1, -1), blocks)
        np.testing.assert_array_equal(y[0], w[:, k])


# ------------------------------------------- gather by id (which row, which scales)
def _id_patterns(n_rows, rng):
    """Ids that a gather reading row i instead of row ids[i] (or the scales of
    row i) cannot satisfy: a permutation, repeats, a descending run, the
    first and the last row, and a 2-D shape."""
    perm = rng.permutation(n_rows)
    return [perm,
            np.array([n_rows - 1, 0, n_rows - 1, 5, 5, 5, 2]),
            np.arange(n_rows - 1, -1, -1),
            rng.integers(0, n_rows, size=(3, 7)),
            np.array([n_rows - 1])]


def test_gather_q2k_selects_rows_by_id(orc):
    """oracle.gather row i is the decode of table row ids[i] (metrale
    "deepseek_v41_ref/engram.rs", embed_rows: rows selected by hash id from
    the dequantised table; atlascybernetics "engram_v41.rs", rows_from_q2k).
    Every table row differs (random bytes, distinct fp16 d/dmin per row), and
    the expected rows come from the second, streaming-order decoder."""
    rng = np.random.default_rng(21)
    n_rows = 37
    table = rng.integers(0, 256, size=(n_rows, 84)).astype(np.uint8)
    dd = (np.arange(2 * n_rows, dtype=np.float64) * 1e-4 + 1e-3).reshape(n_rows, 2)
    table[:, 80:84] = dd.astype(np.float16).view(np.uint8).reshape(n_rows, 4)
    want_rows = np.stack([decode_q2k_stream(table[r]) for r in range(n_rows)])
    assert len({r.tobytes() for r in want_rows}) == n_rows
    for ids in _id_patterns(n_rows, rng):
        got = orc.gather(table, None, ids)
        np.testing.assert_array_equal(got, want_rows[np.asarray(ids).ravel()])


def test_gather_q2k_rows_carry_their_index(orc):
    """Designed table: row r has zero quants, scale 0, every min nibble 1 and
    dmin = (r + 1) / 64, so every value of row r is -(r + 1) / 64, exact in
    bf16; the gathered values name the row that was read."""
    n_rows = 64
    table = np.stack([encode_q2k(np.zeros(256, int), np.zeros(16, int), np.ones(16, int),
                                 0.0, (r + 1) / 64) for r in range(n_rows)])
    ids = np.array([63, 0, 17, 17, 42, 1, 62, 63])
    got = orc.f32_from_bf16(orc.gather(table, None, ids))
    want = np.repeat((-(ids + 1) / 64).astype(np.float32)[:, None], 256, axis=1)
    np.testing.assert_array_equal(got, want)


def test_gather_e4m3_selects_codes_and_scales_by_id(orc):
    """oracle.gather of an e4m3 table: row i is the codes of row ids[i] times
    that row's own block scales (metrale "deepseek_v41_ref/engram.rs",
    regen_table: a row's values times its block's scale; embed_rows: rows
    selected by id).  Codes differ per row and the scales differ per row and
    per block (2^k, k in [-4, 0]); expected values come from torch's e4m3fn
    decode times the scale, in float64 (exact in bf16)."""
    rng = np.random.default_rng(22)
    for head_dim, block in ((256, 128), (256, 16), (64, 32)):
        n_rows = 29
        nb = head_dim // block
        codes = rng.integers(0, 256, size=(n_rows, head_dim)).astype(np.uint8)
        codes[codes == 0x7F] = 0x7E
        codes[codes == 0xFF] = 0xFE
        k = rng.integers(-4, 1, size=(n_rows, nb))
        k[np.arange(n_rows), np.arange(n_rows) % nb] = -(np.arange(n_rows) % 5)
        scales = np.ldexp(1.0, k).astype(np.float32)
        dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
        full = dec * np.repeat(scales.astype(np.float64), block, axis=1)
        for ids in _id_patterns(n_rows, rng):
            flat = np.asarray(ids).ravel()
            got = orc.gather(codes, scales, ids, head_dim, block)
            np.testing.assert_array_equal(orc.f32_from_bf16(got).astype(np.float64), full[flat])


def test_gather_e4m3_scales_name_the_row(orc):
    """Designed e4m3 table: every code is 1.0 (0x38) and row r's scales are
    2^-(r % 5) in block 0 and 2^-((r + 2) % 5) in block 1, so each gathered
    half-row shows which row's scales were applied."""
    n_rows, head_dim, block = 10, 256, 128
    codes = np.full((n_rows, head_dim), 0x38, dtype=np.uint8)
    r = np.arange(n_rows)
    scales = np.stack([np.ldexp(1.0, -(r % 5)), np.ldexp(1.0, -((r + 2) % 5))],
                      axis=1).astype(np.float32)
    ids = np.array([9, 3, 3, 0, 7])
    got = orc.f32_from_bf16(orc.gather(codes, scales, ids, head_dim, block))
    np.testing.assert_array_equal(got[:, :128], np.repeat(scales[ids, :1], 128, axis=1))
    np.testing.assert_array_equal(got[:, 128:], np.repeat(scales[ids, 1:], 128, axis=1))
