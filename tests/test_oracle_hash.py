"""Pins of the oracle's n-gram hash (stage 1) against what the pages and
arithmetic fix, independent of the oracle's own code:

* hand-worked examples (tests/golden/hash_worked_example.json);
* a brute-force evaluator written here from the definition with Python big
  integers: every n-gram is recomputed from scratch (no rolling state), the
  wrap is an explicit reduction mod 2**64, and Python's % is the Euclidean
  remainder for a positive prime;
* the range invariant id in [offset, offset + prime);
* split invariance: chunked prefill and decode equal one pass;
* closed forms: all-pad window -> the offsets; a -1 at shift k pads every
  shift >= k.

Definition: atlascybernetics "spark_model/layers/engram_v41.rs",
EngramHasher::hash; metrale "metrale_model_arch/deepseek_v41_ref/engram.rs",
NgramHashState::forward.
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hash_worked_example.json")
M64 = 1 << 64


def brute_force(token_map, pad_id, mult, primes, offsets, ids, start_pos=0, history=None):
    """Row ids [T][nl][cols] straight from the definition (big integers)."""
    mult = [[int(v) for v in row] for row in mult]
    nl, ng = len(mult), len(mult[0])
    cols = len(primes[0])
    nh = cols // (ng - 1)
    comp = dict(enumerate(history or []))
    for s, i in enumerate(ids):
        comp[start_pos + s] = int(token_map[int(i)])
    out = []
    for s in range(len(ids)):
        p = start_pos + s
        window = []
        for k in range(ng):
            # shift k reads the pad id when any shift up to k falls before
            # the sequence start or finds an unmapped id
            blocked = any(p - j < 0 or comp.get(p - j, 0) == -1 for j in range(k + 1))
            window.append(pad_id if blocked else comp.get(p - k, 0))
        per_layer = []
        for l in range(nl):
            row = [0] * cols
            for n in range(2, ng + 1):
                x = 0
                for j in range(n):
                    x ^= (int(window[j]) * mult[l][j]) % M64
                signed = x - M64 if x >= (1 << 63) else x
                for h in range(nh):
                    c = (n - 2) * nh + h
                    row[c] = signed % int(primes[l][c]) + int(offsets[l][c])
            per_layer.append(row)
        out.append(per_layer)
    return np.array(out, dtype=np.int64).reshape(len(ids), nl, cols)


def random_tables(rng, vocab, comp, nl, ng, nh, p_unmapped=0.2, big=True):
    cols = (ng - 1) * nh
    tm = rng.integers(0, comp, size=vocab).astype(np.int64)
    tm[rng.random(vocab) < p_unmapped] = -1
    tm[0] = 0
    if big:
        mult = (rng.integers(0, 1 << 62, size=(nl, ng), dtype=np.int64) * 2 + 1)
        mult[0, 0] = (1 << 63) - 1          # products that wrap and go negative
    else:
        mult = rng.integers(1, 50, size=(nl, ng)).astype(np.int64)
    primes = rng.choice([101, 103, 107, 109, 113, 127, 131, 137, 139, 149, 151, 157, 163,
                         167, 173, 179, 181, 191, 193, 197, 199, 211, 223, 227, 229, 233,
                         239, 241, 251, 257, 263, 269, 271, 277, 281, 283, 293, 307, 311,
                         313, 317, 331, 337, 347, 349, 353, 359, 367, 373, 379, 383, 389],
                        size=nl * cols, replace=False).astype(np.int64).reshape(nl, cols)
    offsets = np.zeros_like(primes)
    offsets[:, 1:] = np.cumsum(primes, axis=1)[:, :-1]
    return tm, mult, primes, offsets


def test_worked_examples(orc):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        h = orc.Hasher(np.array(c["token_map"]), c["pad_id"], np.array(c["multipliers"]),
                       np.array(c["primes"]), np.array(c["offsets"]), max_seq=16)
        got = h.hash(np.array(c["ids"]), c["start_pos"])
        assert got.tolist() == c["expected"], c["name"]


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_tiny(orc, seed):
    rng = np.random.default_rng(seed)
    nl = int(rng.integers(1, 4))
    ng = int(rng.integers(2, 6))
    nh = int(rng.integers(1, 4))
    vocab = 40
    comp = int(rng.choice([7, 1000, 1 << 40]))
    tm, mult, primes, offsets = random_tables(rng, vocab, comp, nl, ng, nh, big=seed % 3 != 0)
    T = int(rng.integers(1, 30))
    ids = rng.integers(0, vocab, size=T)
    h = orc.Hasher(tm, 0, mult, primes, offsets, max_seq=64)
    got = h.hash(ids, 0)
    want = brute_force(tm, 0, mult, primes, offsets, ids.tolist())
    np.testing.assert_array_equal(got, want)


def test_brute_force_nonzero_pad(orc):
    """A pad id other than 0 enters the products like any token."""
    rng = np.random.default_rng(99)
    tm, mult, primes, offsets = random_tables(rng, 30, 500, 2, 4, 2)
    tm[0] = 17
    ids = rng.integers(0, 30, size=25)
    h = orc.Hasher(tm, 17, mult, primes, offsets, max_seq=32)
    np.testing.assert_array_equal(h.hash(ids, 0), brute_force(tm, 17, mult, primes, offsets,
                                                              ids.tolist()))


def test_range_invariant(orc):
    rng = np.random.default_rng(5)
    tm, mult, primes, offsets = random_tables(rng, 500, 1 << 50, 3, 4, 3)
    ids = rng.integers(0, 500, size=400)
    out = orc.Hasher(tm, 0, mult, primes, offsets, 400).hash(ids, 0)
    lo = offsets[None, :, :]
    assert (out >= lo).all() and (out < lo + primes[None, :, :]).all()


def test_split_invariance(orc):
    """prefill-N then decode == prefill-(N+1), and any chunking == one pass."""
    rng = np.random.default_rng(7)
    tm, mult, primes, offsets = random_tables(rng, 300, 1 << 33, 2, 4, 3)
    ids = rng.integers(0, 300, size=200)
    one = orc.Hasher(tm, 0, mult, primes, offsets, 256).hash(ids, 0)
    for cuts in ([0, 199, 200], [0, 1, 2, 3, 200], [0, 64, 128, 192, 193, 194, 200],
                 list(range(0, 201, 7)) + [200]):
        cuts = sorted(set(cuts))
        h = orc.Hasher(tm, 0, mult, primes, offsets, 256)
        parts = [h.hash(ids[a:b], a) for a, b in zip(cuts[:-1], cuts[1:])]
        np.testing.assert_array_equal(np.concatenate(parts), one)


def test_history_reset_and_start_pos(orc):
    """reset zeroes the look-back; a window reaching into never-written cache
    positions reads 0, as the zero-initialised cache does."""
    rng = np.random.default_rng(8)
    tm, mult, primes, offsets = random_tables(rng, 50, 900, 1, 3, 2)
    ids = rng.integers(1, 50, size=10)
    h = orc.Hasher(tm, 0, mult, primes, offsets, 64)
    h.hash(ids, 0)
    h.reset()
    got = h.hash(ids[:4], 20)
    want = brute_force(tm, 0, mult, primes, offsets, ids[:4].tolist(), start_pos=20)
    np.testing.assert_array_equal(got, want)


def test_closed_forms(orc):
    rng = np.random.default_rng(11)
    tm, mult, primes, offsets = random_tables(rng, 64, 1 << 45, 2, 4, 2)
    tm[5] = -1
    tm[6] = 1234
    h = orc.Hasher(tm, 0, mult, primes, offsets, 16)
    out = h.hash(np.array([6, 5, 6, 6, 6]), 0)
    # current token unmapped: whole window pad (0) -> every id equals its offset
    np.testing.assert_array_equal(out[1], offsets)
    # position 0, mapped a: window [a, pad, ...]; every n gives E(a*m0) + O
    a = 1234
    for l in range(2):
        x = (a * int(mult[l, 0])) % M64
        x = x - M64 if x >= (1 << 63) else x
        np.testing.assert_array_equal(out[0, l], x % primes[l] + offsets[l])
    # position 3: shift 2 lands on the -1 at position 1 -> shifts 2, 3 are pad,
    # so the 3-gram and 4-gram equal the 2-gram's XOR value
    nh = 2
    r2 = ((a * int(mult[0, 0])) % M64) ^ ((a * int(mult[0, 1])) % M64)
    r2 = r2 - M64 if r2 >= (1 << 63) else r2
    for n in (2, 3, 4):
        for hh in range(nh):
            c = (n - 2) * nh + hh
            assert out[3, 0, c] == r2 % primes[0, c] + offsets[0, c]


def test_errors(orc):
    tm = np.array([0, 1, 2], dtype=np.int64)
    mult = np.array([[1, 3]], dtype=np.int64)
    primes = np.array([[5]], dtype=np.int64)
    offs = np.array([[0]], dtype=np.int64)
    h = orc.Hasher(tm, 0, mult, primes, offs, 4)
    with pytest.raises(ValueError):
        h.hash(np.array([0, 1, 2, 1, 0]), 0)          # exceeds max_seq
    with pytest.raises(ValueError):
        h.hash(np.array([3]), 0)                      # outside token_map
