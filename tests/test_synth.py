"""The seeded input generator: reproducible, and the arrays follow the stated
recipe (distinct primes in range, exclusive offsets, odd positive
multipliers, pad mapping, fp16 scales in range, power-of-two e4m3 scales)."""
import numpy as np

import synth
from synth import generate as G


def test_deterministic():
    w = synth.TINY_E4M3
    a, b = G.hash_tables(w), G.hash_tables(w)
    for key in ("token_map", "multipliers", "primes", "offsets"):
        np.testing.assert_array_equal(a[key], b[key])
    la, lb = G.layer_inputs(w, a, 0), G.layer_inputs(w, b, 0)
    for key in ("table", "scales", "wkv", "q", "k"):
        np.testing.assert_array_equal(la[key], lb[key])
    np.testing.assert_array_equal(G.token_ids(w), G.token_ids(w))
    np.testing.assert_array_equal(G.highway(w, 8), G.highway(w, 8))


def test_chunking_independent_of_threads(monkeypatch):
    w = synth.TINY_E4M3
    monkeypatch.setattr(G, "CHUNK", 1000)
    monkeypatch.setattr(G, "_workers", lambda: 1)
    one = G.wkv(w, 0)
    monkeypatch.setattr(G, "_workers", lambda: 7)
    many = G.wkv(w, 0)
    np.testing.assert_array_equal(one, many)


def is_prime(n):
    n = int(n)
    if n < 2:
        return False
    i = 2
    while i * i <= n:
        if n % i == 0:
            return False
        i += 1
    return True


def test_hash_table_recipe():
    for w in (synth.TINY_E4M3, synth.DECODE_Q2K):
        ht = G.hash_tables(w)
        p = ht["primes"]
        assert p.shape == (w.n_layers, w.cols)
        assert len(np.unique(p)) == p.size
        assert (p >= w.prime_lo).all() and (p <= w.prime_hi).all()
        assert all(is_prime(v) for v in p.ravel()[:24])
        o = ht["offsets"]
        for l in range(w.n_layers):
            assert o[l, 0] == 0
            np.testing.assert_array_equal(o[l, 1:], np.cumsum(p[l])[:-1])
            assert ht["rows"][l] == p[l].sum()
        m = ht["multipliers"]
        assert m.shape == (w.n_layers, w.max_ngram)
        assert (m > 0).all() and (m % 2 == 1).all()
        tm = ht["token_map"]
        assert tm[0] == 0 and tm.min() >= -1 and tm.max() < w.compressed
        frac = (tm == -1).mean()
        assert abs(frac - w.p_unmapped) < 0.03


def test_table_recipes():
    w = synth.TINY_E4M3
    ht = G.hash_tables(w)
    codes, scales = G.e4m3_table(w, 0, int(ht["rows"][0]))
    assert codes.shape == (ht["rows"][0], 256) and scales.shape == (ht["rows"][0], 2)
    k = np.log2(scales)
    assert (k == np.round(k)).all() and k.min() >= -4 and k.max() <= 0
    assert not np.isin(codes, [0x7F, 0xFF]).any()
    tab = G.q2k_table(synth.DECODE_Q2K, 0, 5000)
    dd = tab[:, 80:84].copy().view(np.float16).astype(np.float32)
    # fp16 rounding of U(1e-3, 1e-2): at most half an fp16 step outside
    assert dd.min() >= 1e-3 - 2 ** -21 and dd.max() <= 1e-2 + 2 ** -17
    wq = synth.DECODE_WKVQ2K
    blk = G.wkv_q2k(wq, 1)
    assert blk.shape == (wq.N, wq.K // 256, 84) and blk.dtype == np.uint8
    dd = blk[..., 80:84].copy().view(np.float16).astype(np.float32)
    assert dd.min() >= 1e-3 - 2 ** -21 and dd.max() <= 2e-3 + 2 ** -20
    np.testing.assert_array_equal(blk[7], G.wkv_q2k(wq, 1)[7])
    assert not np.array_equal(blk[0], G.wkv_q2k(wq, 0)[0])


def test_token_streams():
    z = G.token_ids(synth.PREFILL_Q2K)
    assert z.shape == (4096,) and z.min() >= 0 and z.max() < synth.PREFILL_Q2K.vocab
    counts = np.sort(np.bincount(z))[::-1]
    # Zipf(1.1): the most frequent id carries a large share of the stream
    assert counts[0] > 0.05 * z.size
    u = G.token_ids(synth.GATHER_Q2K)
    assert u.shape == (16384,) and np.bincount(u).max() < 10


def test_workload_registry():
    """Every workload has its own token / highway stream; workloads that share
    a table family share its hash geometry, vocabulary and table format (they
    reuse the same seeded tables); distinct primes fit each prime range."""
    import synth
    from synth import generate as G
    names = list(synth.WORKLOADS)
    from synth.workloads import STREAM_INDEX
    assert sorted(STREAM_INDEX) == sorted(names)
    assert len(set(STREAM_INDEX.values())) == len(names)
    fam = {}
    for w in synth.WORKLOADS.values():
        key = (w.vocab, w.compressed, w.p_unmapped, w.max_ngram, w.n_heads, w.n_layers,
               w.prime_lo, w.prime_hi, w.fmt, w.head_dim, w.scale_block)
        assert fam.setdefault(w.family, key) == key, w.name
        n_primes = len(G.primes_in(w.prime_lo, w.prime_hi))
        assert n_primes >= w.n_layers * w.cols, w.name
