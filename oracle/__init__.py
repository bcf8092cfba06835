"""Python access to the engram oracle (``engram_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the benchmark's CPU-baseline leg.  The product path never imports it.
It shares no code with the HIP library; inputs come from ``synth`` (or from the
tests themselves) as numpy arrays.
"""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "engram_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain C, no FMA contraction)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                        "-ffp-contract=off", "-fno-fast-math", "-o", tmp, SRC, "-lm"],
                       check=True)
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        p, i64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
        L.orc_bf16_from_f32.restype = ctypes.c_uint16
        L.orc_bf16_from_f32.argtypes = [f32]
        L.orc_bf16_from_f32_n.restype = None
        L.orc_bf16_from_f32_n.argtypes = [p, i64, p]
        L.orc_f32_from_bf16.restype = f32
        L.orc_f32_from_bf16.argtypes = [ctypes.c_uint16]
        L.orc_f32_from_f16.restype = f32
        L.orc_f32_from_f16.argtypes = [ctypes.c_uint16]
        L.orc_e4m3_to_f32.restype = f32
        L.orc_e4m3_to_f32.argtypes = [ctypes.c_uint8]
        L.orc_f32_to_e4m3_rne.restype = ctypes.c_uint8
        L.orc_f32_to_e4m3_rne.argtypes = [f32]
        L.orc_hash.restype = ctypes.c_int
        L.orc_hash.argtypes = [i64, p, i64, i64, i64, i64, p, p, p, p, i64, p, i64, i64, p]
        L.orc_q2k_row.restype = None
        L.orc_q2k_row.argtypes = [p, p]
        L.orc_e4m3_row.restype = None
        L.orc_e4m3_row.argtypes = [p, p, i64, i64, p]
        L.orc_gather_q2k.restype = ctypes.c_int
        L.orc_gather_q2k.argtypes = [p, i64, p, i64, p]
        L.orc_gather_e4m3.restype = ctypes.c_int
        L.orc_gather_e4m3.argtypes = [p, p, i64, i64, i64, p, i64, p]
        L.orc_linear_bf16.restype = None
        L.orc_linear_bf16.argtypes = [p, i64, i64, p, i64, p, i64]
        L.orc_gate_and_add.restype = None
        L.orc_gate_and_add.argtypes = [p, p, p, p, i64, i64, i64, f32, i64, i64]
        _lib = L
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    return max(1, os.cpu_count() or 1)


# ------------------------------------------------------------------ formats
def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    x = _c(np.asarray(x, dtype=np.float32).ravel(), np.float32)
    out = np.zeros(x.size, dtype=np.uint16)
    lib().orc_bf16_from_f32_n(_ptr(x), x.size, _ptr(out))
    return out


def f32_from_bf16(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def e4m3_to_f32(code: int) -> float:
    return lib().orc_e4m3_to_f32(code)


def f32_to_e4m3_rne(x: float) -> int:
    return lib().orc_f32_to_e4m3_rne(x)


def f32_from_f16(h: int) -> float:
    return lib().orc_f32_from_f16(h)


# ------------------------------------------------------------------- stages
class Hasher:
    """The per-sequence n-gram hasher: holds the compressed-id cache across
    calls, so a decode step sees the prefill's look-back."""

    def __init__(self, token_map, pad_id, multipliers, primes, offsets, max_seq):
        self.token_map = _c(token_map, np.int64)
        self.pad_id = int(pad_id)
        self.mult = _c(multipliers, np.int64)
        self.primes = _c(primes, np.int64)
        self.offsets = _c(offsets, np.int64)
        self.n_layers, self.max_ngram = self.mult.shape
        self.cols = self.primes.shape[1]
        self.n_heads = self.cols // (self.max_ngram - 1)
        self.cache = np.zeros(max_seq, dtype=np.int64)

    def reset(self):
        self.cache[:] = 0

    def hash(self, ids, start_pos: int) -> np.ndarray:
        ids = _c(ids, np.int64)
        T = ids.size
        out = np.zeros((T, self.n_layers, self.cols), dtype=np.int64)
        rc = lib().orc_hash(self.token_map.size, _ptr(self.token_map), self.pad_id,
                            self.n_layers, self.max_ngram, self.n_heads,
                            _ptr(self.mult), _ptr(self.primes), _ptr(self.offsets),
                            _ptr(self.cache), self.cache.size, _ptr(ids), T, start_pos,
                            _ptr(out))
        if rc == -1:
            raise ValueError("oracle hash: start_pos + T exceeds max_seq")
        if rc == -2:
            raise ValueError("oracle hash: token id outside token_map")
        return out


def q2k_row(block: np.ndarray) -> np.ndarray:
    block = _c(block, np.uint8)
    assert block.size == 84
    out = np.zeros(256, dtype=np.uint16)
    lib().orc_q2k_row(_ptr(block), _ptr(out))
    return out


def e4m3_row(codes, scales, scale_block: int) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float32)
    out = np.zeros(codes.size, dtype=np.uint16)
    lib().orc_e4m3_row(_ptr(codes), _ptr(scales), codes.size, scale_block, _ptr(out))
    return out


def gather(table, scales, ids, head_dim: int = 256, scale_block: int = 128) -> np.ndarray:
    """Rows of the dequantised table at `ids` (any shape) -> [n_ids, head_dim]
    bf16 bits.  scales is None for a Q2_K table."""
    ids = _c(ids, np.int64).ravel()
    out = np.zeros((ids.size, head_dim), dtype=np.uint16)
    if scales is None:
        table = np.ascontiguousarray(table, dtype=np.uint8)
        rc = lib().orc_gather_q2k(_ptr(table), table.shape[0], _ptr(ids), ids.size, _ptr(out))
    else:
        table = np.ascontiguousarray(table, dtype=np.uint8)
        scales = _c(scales, np.float32)
        rc = lib().orc_gather_e4m3(_ptr(table), _ptr(scales), table.shape[0], head_dim,
                                   scale_block, _ptr(ids), ids.size, _ptr(out))
    if rc != 0:
        raise ValueError("oracle gather: id outside the table")
    return out


def linear_bf16(x, w, nthreads: int = None) -> np.ndarray:
    """x [rows, in] bf16 bits, w [out, in] bf16 bits -> y [rows, out] bf16 bits."""
    x = _c(x, np.uint16)
    w = _c(w, np.uint16)
    rows, in_f = x.shape
    out_f = w.shape[0]
    assert w.shape[1] == in_f
    y = np.zeros((rows, out_f), dtype=np.uint16)
    lib().orc_linear_bf16(_ptr(x), rows, in_f, _ptr(w), out_f, _ptr(y),
                          nthreads or default_threads())
    return y


def expand_q2k_matrix(blocks) -> np.ndarray:
    """A weight matrix shipped as Q2_K blocks, [out, in/256, 84] uint8 -> its
    bf16 expansion [out, in] (bits).  Block b of output row o holds that row's
    weights [256b, 256b+256) and dequantises exactly as a table row does
    (atlascybernetics "spark_model/layers/engram_v41.rs",
    EngramLayerWeights::wkv_q2k: wkv as the GGUF ships it, whose one-token
    projection gives the results of the bf16 expansion)."""
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    out_f, nb, nbytes = blocks.shape
    assert nbytes == 84
    rows = gather(blocks.reshape(out_f * nb, 84), None, np.arange(out_f * nb, dtype=np.int64))
    return rows.reshape(out_f, nb * 256)


def project_q2k(x, blocks, nthreads: int = None) -> np.ndarray:
    """x [rows, in] bf16 bits through a Q2_K-shipped weight matrix: the
    projection of the bf16 expansion ([metrale] linear_bf16)."""
    return linear_bf16(x, expand_q2k_matrix(blocks), nthreads)


def gate_and_add(h, kv, q_w, k_w, eps: float, round_bf16: bool = False,
                 nthreads: int = None) -> np.ndarray:
    """Returns the gated highway (a new f32 array) for h [T, hc, dim] f32,
    kv [T, dim*(hc+1)] bf16 bits, q_w, k_w [hc, dim] bf16 bits."""
    out = np.array(h, dtype=np.float32, copy=True, order="C")
    T, hc, dim = out.shape
    kv = _c(kv, np.uint16)
    assert kv.shape == (T, dim * (hc + 1))
    q_w = _c(q_w, np.uint16)
    k_w = _c(k_w, np.uint16)
    lib().orc_gate_and_add(_ptr(out), _ptr(kv), _ptr(q_w), _ptr(k_w), T, hc, dim, eps,
                           int(round_bf16), nthreads or default_threads())
    return out
