"""Seeded synthetic inputs for the engram workloads.

Every array is drawn from numpy's PCG64 under a SeedSequence whose entropy is
``(20261202, family)`` and whose spawn key names the array (purpose, layer,
chunk), so each array is reproducible on its own and independent of the order
in which arrays are requested or of the number of worker threads.

This module holds no arithmetic of the engram method.  Where an input has to
be stored in a narrow float format (bf16 weights, fp16 Q2_K super-block
scales, e4m3 table codes) it uses the library casts of numpy and torch, which
round to nearest even.

Recipe (one line per array):

* token_map [vocab] int64: -1 with probability p_unmapped, else uniform in
  [0, compressed); then token_map[0] = 0 so the pad token maps to the
  compressed pad id 0.
* multipliers [n_layers, max_ngram] int64: odd, uniform in [1, 2**63).
* primes [n_layers, cols] int64: distinct primes drawn uniformly without
  replacement from all primes in [prime_lo, prime_hi].
* offsets [n_layers, cols] int64: exclusive running sum of the layer's primes,
  so the ids of a layer tile [0, sum(primes)) and the table has that many rows.
* Q2_K table [rows, 84] uint8: bytes uniform; bytes 80..83 overwritten with
  fp16 d and dmin drawn from U(1e-3, 1e-2).
* e4m3 table: codes [rows, head_dim] uint8 = e4m3(clip(N(0,1), +-448));
  scales [rows, head_dim/scale_block] float32 = 2**k, k uniform in [k_lo, k_hi].
* wkv [dim*(hc+1), cols*head_dim] bf16 bits = bf16(N(0, wkv_std)).
* wkv as Q2_K blocks [dim*(hc+1), cols*head_dim/256, 84] uint8 (workloads with
  wkv_fmt "q2k", instead of the bf16 wkv): bytes uniform; bytes 80..83
  overwritten with fp16 d and dmin drawn from U(wkv_d_lo, wkv_d_hi), which puts
  the dequantised weights at a spread of about 0.02.
* q, k [hc, dim] bf16 bits = bf16(1 + qk_std*N(0,1)) each.
* token ids [prompt + decode_steps] int32: uniform over the vocabulary, or
  Zipf(s) truncated to the vocabulary (pmf proportional to rank**-s) mapped
  through a seeded rank -> id permutation.
* highway [T, hc, dim] float32: N(0, 1).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from .workloads import Workload, STREAM_INDEX

ROOT_SEED = 20261202
CHUNK = 1 << 24            # elements per independently seeded chunk

# spawn-key purposes
_HASH, _TABLE, _SCALES, _WKV, _QK, _TOKENS, _HIGHWAY, _DECODE_HIGHWAY, _WKV_Q2K, \
    _WKV_Q2K_SCALES = range(10)


def _seq(entropy_idx: int, *key: int) -> np.random.SeedSequence:
    return np.random.SeedSequence(entropy=[ROOT_SEED, entropy_idx], spawn_key=tuple(key))


def _rng(entropy_idx: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(_seq(entropy_idx, *key)))


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _chunked(n: int, dtype, fill, entropy_idx: int, *key: int) -> np.ndarray:
    """Fill a flat array of n elements chunk by chunk; chunk i uses its own
    generator keyed by (*key, i), so the result does not depend on threads."""
    out = np.empty(n, dtype=dtype)
    starts = list(range(0, n, CHUNK))

    def work(i_s):
        i, s = i_s
        e = min(n, s + CHUNK)
        fill(_rng(entropy_idx, *key, i), out[s:e])

    if len(starts) == 1:
        work((0, 0))
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(work, enumerate(starts)))
    return out


def primes_in(lo: int, hi: int) -> np.ndarray:
    """All primes p with lo <= p <= hi (sieve of Eratosthenes)."""
    sieve = np.ones(hi + 1, dtype=bool)
    sieve[:2] = False
    for p in range(2, int(hi ** 0.5) + 1):
        if sieve[p]:
            sieve[p * p::p] = False
    return np.nonzero(sieve[lo:])[0].astype(np.int64) + lo


def hash_tables(w: Workload) -> dict:
    """token_map, multipliers, primes, offsets and the per-layer row count."""
    rng = _rng(w.family, _HASH)
    tm = rng.integers(0, w.compressed, size=w.vocab, dtype=np.int64)
    unmapped = rng.random(w.vocab) < w.p_unmapped
    tm[unmapped] = -1
    tm[0] = w.pad_id
    mult = (rng.bit_generator.random_raw(w.n_layers * w.max_ngram) >> np.uint64(1))
    mult = (mult | np.uint64(1)).astype(np.int64).reshape(w.n_layers, w.max_ngram)
    cands = primes_in(w.prime_lo, w.prime_hi)
    primes = rng.choice(cands, size=w.n_layers * w.cols, replace=False)
    primes = primes.astype(np.int64).reshape(w.n_layers, w.cols)
    offsets = np.zeros_like(primes)
    offsets[:, 1:] = np.cumsum(primes, axis=1)[:, :-1]
    rows = primes.sum(axis=1)
    return dict(token_map=tm, multipliers=mult, primes=primes, offsets=offsets,
                pad_id=np.int64(w.pad_id), rows=rows)


def _fill_bytes(g, dst):
    n = dst.size
    raw = g.bit_generator.random_raw((n + 7) // 8)
    dst[:] = raw.view(np.uint8)[:n]


def q2k_table(w: Workload, layer: int, rows: int) -> np.ndarray:
    """[rows, 84] uint8 Q2_K blocks: uniform bytes, fp16 d/dmin in U(1e-3, 1e-2)."""
    tab = _chunked(rows * 84, np.uint8, _fill_bytes, w.family, _TABLE, layer).reshape(rows, 84)

    def fill_dd(g, dst):
        dst[:] = g.uniform(1e-3, 1e-2, size=dst.size).astype(np.float32)

    dd = _chunked(rows * 2, np.float32, fill_dd, w.family, _SCALES, layer)
    tab[:, 80:84] = dd.astype(np.float16).view(np.uint8).reshape(rows, 4)
    return tab


def e4m3_table(w: Workload, layer: int, rows: int):
    """(codes [rows, head_dim] uint8, scales [rows, head_dim/scale_block] f32)."""
    def fill_codes(g, dst):
        x = g.standard_normal(dst.size, dtype=np.float32)
        np.clip(x, -448.0, 448.0, out=x)
        dst[:] = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()

    codes = _chunked(rows * w.head_dim, np.uint8, fill_codes, w.family, _TABLE, layer)
    nb = w.head_dim // w.scale_block

    def fill_k(g, dst):
        dst[:] = g.integers(w.scale_k_lo, w.scale_k_hi + 1, size=dst.size)

    k = _chunked(rows * nb, np.int8, fill_k, w.family, _SCALES, layer)
    scales = np.ldexp(np.float32(1.0), k.astype(np.int32)).astype(np.float32)
    return codes.reshape(rows, w.head_dim), scales.reshape(rows, nb)


def table(w: Workload, layer: int, rows: int):
    if w.fmt == "q2k":
        return q2k_table(w, layer, rows)
    return e4m3_table(w, layer, rows)


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def wkv(w: Workload, layer: int) -> np.ndarray:
    """[N, K] bf16 bits, N(0, wkv_std)."""
    def fill(g, dst):
        x = g.standard_normal(dst.size, dtype=np.float32)
        x *= np.float32(w.wkv_std)
        dst[:] = _bf16_bits(x)

    return _chunked(w.N * w.K, np.uint16, fill, w.family, _WKV, layer).reshape(w.N, w.K)


def wkv_q2k(w: Workload, layer: int) -> np.ndarray:
    """[N, K/256, 84] uint8 Q2_K blocks of wkv: uniform bytes, fp16 d/dmin in
    U(wkv_d_lo, wkv_d_hi)."""
    nb = w.N * (w.K // 256)
    blk = _chunked(nb * 84, np.uint8, _fill_bytes, w.family, _WKV_Q2K, layer).reshape(nb, 84)

    def fill_dd(g, dst):
        dst[:] = g.uniform(w.wkv_d_lo, w.wkv_d_hi, size=dst.size).astype(np.float32)

    dd = _chunked(nb * 2, np.float32, fill_dd, w.family, _WKV_Q2K_SCALES, layer)
    blk[:, 80:84] = dd.astype(np.float16).view(np.uint8).reshape(nb, 4)
    return blk.reshape(w.N, w.K // 256, 84)


def qk_weights(w: Workload, layer: int):
    """(q, k), each [hc, dim] bf16 bits of 1 + qk_std * N(0, 1)."""
    g = _rng(w.family, _QK, layer)
    q = 1.0 + w.qk_std * g.standard_normal((w.hc, w.dim))
    k = 1.0 + w.qk_std * g.standard_normal((w.hc, w.dim))
    return _bf16_bits(q.astype(np.float32)), _bf16_bits(k.astype(np.float32))


def token_ids(w: Workload, n: int = None) -> np.ndarray:
    """[n] int32 token ids (default: prompt + decode steps)."""
    n = w.total_tokens if n is None else n
    g = _rng(100 + STREAM_INDEX[w.name], _TOKENS)
    if w.token_dist == "uniform":
        return g.integers(0, w.vocab, size=n, dtype=np.int64).astype(np.int32)
    ranks = np.arange(1, w.vocab + 1, dtype=np.float64)
    cdf = np.cumsum(ranks ** -w.zipf_s)
    cdf /= cdf[-1]
    perm = g.permutation(w.vocab)
    r = np.searchsorted(cdf, g.random(n), side="right")
    r = np.minimum(r, w.vocab - 1)
    return perm[r].astype(np.int32)


def highway(w: Workload, T: int, decode: bool = False) -> np.ndarray:
    """[T, hc, dim] float32 N(0,1).  decode=True draws the per-step highways
    (one [1, hc, dim] slice per decode step) from their own stream."""
    purpose = _DECODE_HIGHWAY if decode else _HIGHWAY

    def fill(g, dst):
        dst[:] = g.standard_normal(dst.size, dtype=np.float32)

    flat = _chunked(T * w.hc * w.dim, np.float32, fill, 100 + STREAM_INDEX[w.name], purpose)
    return flat.reshape(T, w.hc, w.dim)


def layer_inputs(w: Workload, ht: dict, layer: int) -> dict:
    """Everything one engram layer needs besides the hash tables."""
    rows = int(ht["rows"][layer])
    if w.wkv_fmt == "q2k":
        out = dict(rows=rows, wkv=None, wkv_q2k=wkv_q2k(w, layer))
    else:
        out = dict(rows=rows, wkv=wkv(w, layer), wkv_q2k=None)
    out["q"], out["k"] = qk_weights(w, layer)
    if w.fmt == "q2k":
        out["table"] = q2k_table(w, layer, rows)
        out["scales"] = None
    else:
        out["table"], out["scales"] = e4m3_table(w, layer, rows)
    return out
