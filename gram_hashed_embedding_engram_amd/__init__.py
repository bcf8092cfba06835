"""Python binding of libengram.so, the gfx950 engram hot path.

Argument marshalling only: torch tensors provide device memory and the
current HIP stream; every step of the path runs in the library's kernels.
The names follow the C ABI in include/engram.h.  There is no fallback: if
the library is not built, every call raises.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libengram.so")

OK = 0
E_ARG, E_RANGE, E_UNSUPPORTED, E_STATE, E_HIP, E_DEVICE = -1, -2, -3, -4, -5, -6
DEVERR_TOKEN, DEVERR_ROW, DEVERR_POSITION = 1, 2, 4
FMT_Q2K, FMT_E4M3 = 0, 1
Q2K_ROW_BYTES = 84
STREAM_ROW_BYTES = 12288      # engram_stream_read's row (ENGRAM_STREAM_ROW_BYTES)
STREAM_SINK_WORDS = 8192      # its sink (ENGRAM_STREAM_SINK_WORDS)
STATIC_SCRATCH_BYTES = 32 << 20   # engram_layer_static's scratch (ENGRAM_STATIC_SCRATCH_BYTES)
STAGES = ("hash", "gather", "project", "gate")

# Every symbol include/engram.h declares.
EXPORTS = (
    "engram_last_error", "engram_abi_version", "engram_hash", "engram_hash_batch",
    "engram_gather_dequant",
    "engram_project", "engram_project_q2k", "engram_dequant_q2k", "engram_qk_product",
    "engram_gate_apply", "engram_workspace_bytes",
    "engram_ctx_create", "engram_ctx_add_layer", "engram_ctx_set_wkv_q2k", "engram_reset",
    "engram_forward",
    "engram_check", "engram_position", "engram_ctx_buffers", "engram_ctx_set_fused_decode",
    "engram_ctx_set_timing",
    "engram_ctx_timing", "engram_ctx_destroy", "engram_map_host", "engram_stream_read",
    "engram_ctx_set_graph_mode", "engram_ctx_set_position", "engram_layer_static",
)


class EngramError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"engram error {code}: {msg}")
        self.code = code


class HashTablesC(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("max_ngram", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("vocab", ctypes.c_int64), ("pad_id", ctypes.c_int64),
                ("d_token_map", ctypes.c_void_p), ("multipliers", ctypes.c_void_p),
                ("primes", ctypes.c_void_p), ("offsets", ctypes.c_void_p)]


class TableC(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("scale_block", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("n_rows", ctypes.c_int64), ("d_data", ctypes.c_void_p),
                ("d_scales", ctypes.c_void_p)]


class ConfigC(ctypes.Structure):
    _fields_ = [("hc", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dim", ctypes.c_int64),
                ("eps", ctypes.c_float), ("batch", ctypes.c_int32),
                ("max_tokens", ctypes.c_int64), ("max_seq", ctypes.c_int64),
                ("hash", HashTablesC)]


_lib = None
ABI_VERSION = 7           # ENGRAM_ABI_VERSION of include/engram.h this binding follows


def lib():
    """The loaded libengram.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run python -m "
                               "gram_hashed_embedding_engram_amd.build (the engram path has no "
                               "non-HIP fallback)")
        L = ctypes.CDLL(LIB_PATH)
        p, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        sig = {
            "engram_last_error": (ctypes.c_char_p, []),
            "engram_abi_version": (i32, []),
            "engram_hash": (i32, [p, p, i64, i64, p, i64, p, p, p]),
            "engram_hash_batch": (i32, [p, p, i64, i64, i64, p, i64, p, p, p]),
            "engram_gather_dequant": (i32, [p, p, i64, i32, i64, p, p, p]),
            "engram_project": (i32, [p, p, p, i64, i64, i64, p]),
            "engram_project_q2k": (i32, [p, p, p, i64, i64, i64, p]),
            "engram_dequant_q2k": (i32, [p, i64, p, p]),
            "engram_qk_product": (i32, [p, p, p, i64, p]),
            "engram_gate_apply": (i32, [p, p, p, i64, i32, i64, ctypes.c_float, p]),
            "engram_workspace_bytes": (ctypes.c_size_t, [p]),
            "engram_ctx_create": (i32, [p, p, ctypes.c_size_t, p]),
            "engram_ctx_add_layer": (i32, [p, i32, p, p, p]),
            "engram_ctx_set_wkv_q2k": (i32, [p, i32, p]),
            "engram_reset": (i32, [p, p]),
            "engram_forward": (i32, [p, i32, p, i64, p, p]),
            "engram_check": (i32, [p, p]),
            "engram_position": (i64, [p]),
            "engram_ctx_buffers": (i32, [p, p, p, p, p]),
            "engram_ctx_set_fused_decode": (i32, [p, i32]),
            "engram_ctx_set_timing": (i32, [p, i32]),
            "engram_ctx_timing": (i32, [p, p, p]),
            "engram_ctx_destroy": (None, [p]),
            "engram_map_host": (i32, [p, p]),
            "engram_stream_read": (i32, [p, i64, p, p]),
            "engram_ctx_set_graph_mode": (i32, [p, i32, p]),
            "engram_ctx_set_position": (i32, [p, i64, p]),
            "engram_layer_static": (i32, [p, i32, p, p, p, i32, i64, ctypes.c_float, p, i64,
                                          i64, p, i64, p, p, p]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        if L.engram_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {L.engram_abi_version()}, this "
                               f"binding {ABI_VERSION}: rebuild it (python -m "
                               "gram_hashed_embedding_engram_amd.build)")
        _lib = L
    return _lib


def last_error() -> str:
    return lib().engram_last_error().decode()


def _check(rc):
    if rc != OK:
        raise EngramError(rc, last_error())


def _ptr(t):
    """Device (or host numpy) address of a tensor / array; None -> NULL."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _room(t):
    """Bytes from a tensor's (or array's) first element to the end of its
    storage: what a kernel may touch through its address."""
    if isinstance(t, np.ndarray):
        return t.nbytes if t.flags.c_contiguous else -1
    return t.untyped_storage().nbytes() - t.storage_offset() * t.element_size()


def _need(t, name, nbytes, dense=True):
    """Refuse, before the library sees the address, a tensor that a call of
    these sizes would read or write past the end of its storage, or a strided
    view where the kernel takes rows to be back to back.  The C entry points
    cannot see a buffer's size; the binding can."""
    if t is None:
        return
    if dense and not isinstance(t, np.ndarray) and not t.is_contiguous():
        raise EngramError(E_ARG, f"{name}: a contiguous tensor is needed")
    room = _room(t)
    if nbytes > room:
        raise EngramError(E_ARG, f"{name}: the call needs {nbytes} bytes, its storage holds "
                                 f"{max(room, 0)} from this address")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class HashTables:
    """Hash tables for the ABI: token_map on the device (torch int64
    tensor), multipliers / primes / offsets as host arrays."""

    def __init__(self, d_token_map, pad_id, multipliers, primes, offsets):
        self.mult = np.ascontiguousarray(multipliers, dtype=np.int64)
        self.primes = np.ascontiguousarray(primes, dtype=np.int64)
        self.offsets = np.ascontiguousarray(offsets, dtype=np.int64)
        self.token_map = d_token_map
        self.n_layers, self.max_ngram = self.mult.shape
        self.cols = self.primes.shape[1]
        self.n_heads = self.cols // (self.max_ngram - 1)
        self.c = HashTablesC(self.n_layers, self.max_ngram, self.n_heads, 0,
                             int(d_token_map.numel()), int(pad_id), _ptr(d_token_map),
                             self.mult.ctypes.data, self.primes.ctypes.data,
                             self.offsets.ctypes.data)


def map_host(t):
    """Device address of a pinned host tensor (engram_map_host)."""
    dev = ctypes.c_void_p()
    _check(lib().engram_map_host(ctypes.c_void_p(t.data_ptr()), ctypes.byref(dev)))
    return dev.value


def _table_ptr(t):
    if t is None:
        return None
    return t.data_ptr() if t.is_cuda else map_host(t)


class Table:
    """One layer's table (Q2_K blocks, or e4m3 codes with f32 block scales),
    as device tensors or as pinned host tensors the kernels read across the
    host link."""

    def __init__(self, d_data, d_scales=None, head_dim=256, scale_block=128):
        fmt = FMT_Q2K if d_scales is None else FMT_E4M3
        n_rows = int(d_data.shape[0])
        self.data, self.scales = d_data, d_scales
        self.c = TableC(fmt, head_dim, scale_block if fmt == FMT_E4M3 else 0, 0, n_rows,
                        _table_ptr(d_data), _table_ptr(d_scales))


def hash(tables: HashTables, d_ids, start_pos, d_history, d_row_ids, d_err=None, stream=None):
    T = int(d_ids.numel())
    _need(d_ids, "ids", 4 * T)
    _need(d_history, "history", 8 * int(d_history.numel()))
    _need(d_row_ids, "row_ids", 8 * T * tables.n_layers * tables.cols)
    _need(d_err, "err", 4)
    _check(lib().engram_hash(ctypes.byref(tables.c), _ptr(d_ids), int(d_ids.numel()),
                             int(start_pos), _ptr(d_history), int(d_history.numel()),
                             _ptr(d_row_ids), _ptr(d_err), _stream(stream)))


def hash_batch(tables: HashTables, d_ids, start_pos, d_history, d_row_ids, d_err=None,
               stream=None):
    """d_ids [B, T] int32, d_history [B, max_seq] int64, d_row_ids [B*T, nl, cols]."""
    B, T = d_ids.shape
    _need(d_ids, "ids", 4 * B * T)
    _need(d_history, "history", 8 * B * d_history.shape[1])
    _need(d_row_ids, "row_ids", 8 * B * T * tables.n_layers * tables.cols)
    _need(d_err, "err", 4)
    _check(lib().engram_hash_batch(ctypes.byref(tables.c), _ptr(d_ids), int(B), int(T),
                                   int(start_pos), _ptr(d_history), int(d_history.shape[1]),
                                   _ptr(d_row_ids), _ptr(d_err), _stream(stream)))


def gather_dequant(table: Table, d_row_ids, T, cols, id_stride, d_rows, d_err=None,
                   stream=None):
    if T > 0:
        # ids of token t at d_row_ids + t*id_stride: any view that reaches them will do
        _need(d_row_ids, "row_ids", 8 * ((T - 1) * id_stride + cols), dense=False)
        _need(d_rows, "rows", 2 * T * cols * table.c.head_dim)
    _need(d_err, "err", 4)
    _check(lib().engram_gather_dequant(ctypes.byref(table.c), _ptr(d_row_ids), int(T),
                                       int(cols), int(id_stride), _ptr(d_rows), _ptr(d_err),
                                       _stream(stream)))


def project(d_x, d_w, d_y, stream=None):
    T, K = d_x.shape
    N = d_w.shape[0]
    _need(d_x, "x", 2 * T * K)
    _need(d_w, "w", 2 * N * K)
    _need(d_y, "y", 2 * T * N)
    _check(lib().engram_project(_ptr(d_x), _ptr(d_w), _ptr(d_y), T, K, N, _stream(stream)))


def project_q2k(d_x, d_wq, d_y, stream=None):
    """d_x [T, K] bf16 bits (T <= 1), d_wq [N, K/256, 84] uint8 Q2_K blocks."""
    T, K = d_x.shape
    N = d_wq.shape[0]
    _need(d_x, "x", 2 * T * K)
    _need(d_wq, "wkv_q2k", N * (K // 256) * 84)
    _need(d_y, "y", 2 * T * N)
    _check(lib().engram_project_q2k(_ptr(d_x), _ptr(d_wq), _ptr(d_y), T, K, N, _stream(stream)))


def dequant_q2k(d_blocks, d_out, stream=None):
    """Q2_K blocks (any shape [..., 84] uint8) -> d_out [n_blocks * 256] bf16 bits."""
    n = d_blocks.numel() // 84
    _need(d_blocks, "blocks", 84 * n)
    _need(d_out, "out", 2 * 256 * n)
    _check(lib().engram_dequant_q2k(_ptr(d_blocks), n, _ptr(d_out), _stream(stream)))


def qk_product(d_q, d_k, d_qk, stream=None):
    n = int(d_q.numel())
    _need(d_q, "q", 2 * n)
    _need(d_k, "k", 2 * n)
    _need(d_qk, "qk", 4 * n)
    _check(lib().engram_qk_product(_ptr(d_q), _ptr(d_k), _ptr(d_qk), int(d_q.numel()),
                                   _stream(stream)))


def stream_read(d_src, d_sink, stream=None):
    """Stream d_src once, one XOR fold per wavefront into d_sink [8192]
    int32 (the read-rate yardstick; engram_stream_read)."""
    _need(d_sink, "sink", 4 * STREAM_SINK_WORDS)
    _check(lib().engram_stream_read(_ptr(d_src), int(d_src.numel() * d_src.element_size()),
                                    _ptr(d_sink), _stream(stream)))


def gate_apply(d_h, d_kv, d_qk, eps, stream=None):
    T, hc, dim = d_h.shape
    _need(d_h, "h", 4 * T * hc * dim)
    _need(d_kv, "kv", 2 * T * dim * (hc + 1))
    _need(d_qk, "qk", 4 * hc * dim)
    _check(lib().engram_gate_apply(_ptr(d_h), _ptr(d_kv), _ptr(d_qk), T, hc, dim,
                                   float(eps), _stream(stream)))


def layer_static(tables: HashTables, hash_index, table: Table, d_wkv, d_qk, eps, d_ids,
                 start_pos, d_history, d_h, d_err=None, stream=None):
    """One engram layer over d_ids [T] at start_pos with its row ids, rows
    and kv in the library's static scratch (engram_layer_static: allocates
    nothing).  d_history [max_seq] int64, d_h [T, hc, dim] f32 in place."""
    T = int(d_ids.numel())
    _, hc, dim = d_h.shape
    K = tables.cols * table.c.head_dim
    _need(d_ids, "ids", 4 * T)
    _need(d_history, "history", 8 * int(d_history.numel()))
    _need(d_wkv, "wkv", 2 * dim * (hc + 1) * K)
    _need(d_qk, "qk", 4 * hc * dim)
    _need(d_h, "h", 4 * T * hc * dim)
    _need(d_err, "err", 4)
    _check(lib().engram_layer_static(ctypes.byref(tables.c), int(hash_index),
                                     ctypes.byref(table.c), _ptr(d_wkv), _ptr(d_qk), int(hc),
                                     int(dim), float(eps), _ptr(d_ids), T, int(start_pos),
                                     _ptr(d_history), int(d_history.numel()), _ptr(d_h),
                                     _ptr(d_err), _stream(stream)))


class Context:
    """The stateful engram of one sequence (engram_ctx)."""

    def __init__(self, tables: HashTables, hc, dim, head_dim, eps, max_tokens, max_seq,
                 d_workspace=None, batch=1):
        import torch
        self.tables = tables
        self.batch = batch
        self.cfg = ConfigC(hc, head_dim, dim, eps, batch, max_tokens, max_seq, tables.c)
        nbytes = lib().engram_workspace_bytes(ctypes.byref(self.cfg))
        if nbytes == 0:
            raise EngramError(E_ARG, "invalid engram configuration")
        if d_workspace is None:
            d_workspace = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        self.workspace = d_workspace
        self.nl, self.cols = tables.n_layers, tables.cols
        self.hc, self.dim, self.head_dim = hc, dim, head_dim
        h = ctypes.c_void_p()
        _check(lib().engram_ctx_create(ctypes.byref(self.cfg), _ptr(d_workspace),
                                       int(d_workspace.numel()), ctypes.byref(h)))
        self.h = h
        self._keep = {}

    def add_layer(self, hash_index, table: Table, d_wkv, d_qk):
        K = self.cols * self.head_dim
        _need(d_wkv, "wkv", 2 * self.dim * (self.hc + 1) * K)
        _need(d_qk, "qk", 4 * self.hc * self.dim)
        self._keep[hash_index] = (table, d_wkv, d_qk)
        _check(lib().engram_ctx_add_layer(self.h, hash_index, ctypes.byref(table.c),
                                          _ptr(d_wkv), _ptr(d_qk)))

    def set_wkv_q2k(self, hash_index, d_wq):
        """Registers (or, with None, drops) the layer's wkv as Q2_K blocks."""
        table, wkv, qk = self._keep[hash_index][:3]
        N, K = self.dim * (self.hc + 1), self.cols * self.head_dim
        _need(d_wq, "wkv_q2k", N * (K // 256) * 84)
        self._keep[hash_index] = (table, wkv, qk, d_wq)
        _check(lib().engram_ctx_set_wkv_q2k(self.h, hash_index, _ptr(d_wq)))

    def reset(self, stream=None):
        _check(lib().engram_reset(self.h, _stream(stream)))

    def forward(self, hash_index, d_ids, T, d_h, stream=None):
        M = self.batch * int(T)
        _need(d_ids, "ids", 4 * M)
        _need(d_h, "h", 4 * M * self.hc * self.dim)
        _check(lib().engram_forward(self.h, hash_index, _ptr(d_ids), int(T), _ptr(d_h),
                                    _stream(stream)))

    def check(self, stream=None):
        _check(lib().engram_check(self.h, _stream(stream)))

    @property
    def position(self):
        return lib().engram_position(self.h)

    def buffers(self):
        """(row_ids, rows, kv, err) device addresses."""
        ptrs = [ctypes.c_void_p() for _ in range(4)]
        _check(lib().engram_ctx_buffers(self.h, *[ctypes.byref(q) for q in ptrs]))
        return tuple(q.value for q in ptrs)

    def views(self, T):
        """torch views of the workspace for a call of T tokens a sequence
        (M = batch*T): row ids [M, nl, cols] int64, rows [M, cols*head_dim]
        bf16 bits (int16), kv [M, dim*(hc+1)] (int16)."""
        import torch
        ws = self.workspace
        base = ws.data_ptr()
        rid, rows, kv, _ = self.buffers()

        def view(addr, n, dtype, shape):
            size = torch.empty(0, dtype=dtype).element_size()
            off = addr - base
            return ws[off:off + n * size].view(dtype).view(*shape)

        K, N = self.cols * self.head_dim, self.dim * (self.hc + 1)
        M = self.batch * T
        return (view(rid, M * self.nl * self.cols, torch.int64, (M, self.nl, self.cols)),
                view(rows, M * K, torch.int16, (M, K)),
                view(kv, M * N, torch.int16, (M, N)))

    def set_fused_decode(self, on: bool):
        _check(lib().engram_ctx_set_fused_decode(self.h, 1 if on else 0))

    def set_timing(self, on: bool):
        _check(lib().engram_ctx_set_timing(self.h, 1 if on else 0))

    def history(self):
        """The hasher's history rows, a view of the workspace: [batch, max_seq]
        int64 compressed ids (what a checkpoint of the sequence holds)."""
        import torch
        n = self.batch * int(self.cfg.max_seq)
        return self.workspace[:8 * n].view(torch.int64).view(self.batch, -1)

    def set_position(self, pos, stream=None):
        """Resume at pos over history rows the caller restored into the
        workspace (engram_ctx_set_position)."""
        _check(lib().engram_ctx_set_position(self.h, int(pos), _stream(stream)))

    def set_graph_mode(self, on: bool, stream=None):
        """Single-token steps read their position from the device, so their
        launches can be captured once and replayed (engram_ctx_set_graph_mode)."""
        _check(lib().engram_ctx_set_graph_mode(self.h, 1 if on else 0, _stream(stream)))

    def timing(self):
        ms = (ctypes.c_double * 4)()
        n = (ctypes.c_int64 * 4)()
        _check(lib().engram_ctx_timing(self.h, ms, n))
        return {STAGES[i]: (ms[i], n[i]) for i in range(4)}

    def close(self):
        if getattr(self, "h", None):
            lib().engram_ctx_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
