"""Helpers shared by the GPU parity tests: device upload of the synthetic
workloads, the tolerance metric, and bf16 helpers.  Inputs come from
``synth``; expected values from ``oracle``; nothing here computes a stage."""
import functools
import sys

import numpy as np

import synth
from synth import generate as G


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def relerr(got, want):
    """max_i |g_i - o_i| / max(|o_i|, rms(o)): elementwise relative error with
    values below the rms measured against the rms (so cancellation in a
    single output does not blow the ratio up)."""
    g = np.asarray(got, dtype=np.float64).ravel()
    o = np.asarray(want, dtype=np.float64).ravel()
    rms = np.sqrt(np.mean(o * o)) if o.size else 0.0
    den = np.maximum(np.abs(o), rms)
    den[den == 0] = 1.0
    return float(np.max(np.abs(g - o) / den)) if o.size else 0.0


def widen(bits):
    b = np.asarray(bits).view(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def to_np_u16(t):
    return t.cpu().numpy().view(np.uint16)


@functools.lru_cache(maxsize=4)
def family_data(name):
    """Host arrays of a workload: hash tables and every layer's inputs."""
    w = synth.WORKLOADS[name]
    ht = G.hash_tables(w)
    layers = [G.layer_inputs(w, ht, l) for l in range(w.n_layers)]
    return w, ht, layers


class Device:
    """The workload on the GPU: tables, wkv, qk, token map, hash tables."""

    def __init__(self, name, host_tables=False):
        """host_tables: keep the tables (and e4m3 scales) in pinned host
        memory, read by the kernels across the host link."""
        import torch
        import gram_hashed_embedding_engram_amd as E
        self.w, self.ht, self.layers = family_data(name)
        w = self.w
        dev = "cuda"
        self.token_map = torch.from_numpy(self.ht["token_map"]).to(dev)
        self.tables = E.HashTables(self.token_map, self.ht["pad_id"], self.ht["multipliers"],
                                   self.ht["primes"], self.ht["offsets"])
        self.tab, self.wkv, self.wkvq, self.qk = [], [], [], []
        self._oracle_wkv = {}
        for L in self.layers:
            place = ((lambda a: torch.from_numpy(a).pin_memory()) if host_tables
                     else (lambda a: torch.from_numpy(a).to(dev)))
            data = place(L["table"])
            scales = None if L["scales"] is None else place(L["scales"])
            self.tab.append(E.Table(data, scales, head_dim=w.head_dim, scale_block=w.scale_block))
            if L["wkv_q2k"] is None:
                self.wkv.append(torch.from_numpy(L["wkv"].view(np.int16)).to(dev))
                self.wkvq.append(None)
            else:
                # wkv shipped as Q2_K blocks: the library expands them for T > 1
                blocks = torch.from_numpy(L["wkv_q2k"]).to(dev)
                bf = torch.empty(w.N, w.K, dtype=torch.int16, device=dev)
                E.dequant_q2k(blocks, bf)
                self.wkv.append(bf)
                self.wkvq.append(blocks)
            q = torch.from_numpy(L["q"].view(np.int16)).to(dev)
            k = torch.from_numpy(L["k"].view(np.int16)).to(dev)
            qk = torch.empty(w.hc, w.dim, dtype=torch.float32, device=dev)
            E.qk_product(q, k, qk)
            self.qk.append(qk)
        torch.cuda.synchronize()

    def context(self, max_tokens, max_seq, batch=1):
        import gram_hashed_embedding_engram_amd as E
        w = self.w
        ctx = E.Context(self.tables, w.hc, w.dim, w.head_dim, w.eps, max_tokens, max_seq,
                        batch=batch)
        for l in range(w.n_layers):
            ctx.add_layer(l, self.tab[l], self.wkv[l], self.qk[l])
            if self.wkvq[l] is not None:
                ctx.set_wkv_q2k(l, self.wkvq[l])
        ctx.reset()
        return ctx

    def oracle_wkv(self, layer):
        """The layer's bf16 wkv as the oracle sees it: the stored matrix, or
        the oracle's expansion of the Q2_K blocks."""
        import oracle
        if layer not in self._oracle_wkv:
            L = self.layers[layer]
            self._oracle_wkv[layer] = (L["wkv"] if L["wkv_q2k"] is None
                                       else oracle.expand_q2k_matrix(L["wkv_q2k"]))
        return self._oracle_wkv[layer]

    def oracle_hasher(self, max_seq):
        import oracle
        ht = self.ht
        return oracle.Hasher(ht["token_map"], ht["pad_id"], ht["multipliers"], ht["primes"],
                             ht["offsets"], max_seq)

    def oracle_rows(self, layer, ids):
        import oracle
        L = self.layers[layer]
        return oracle.gather(L["table"], L["scales"], ids, self.w.head_dim, self.w.scale_block)


# the prefill GEMM's output tile: 256 tokens x 320 outputs
GEMM_TILE_M = 256
GEMM_TILE_N = 320


def tile_strata(n, tile, rng, interior=1):
    """Indices into [0, n) that meet every tile of `tile` consecutive indices:
    each tile's first and last index and `interior` seeded indices inside it.
    Sampling tokens this way (all outputs of each) and outputs this way (all
    tokens of each) puts a compared row slice and a compared column slice in
    every output tile of the projection, so a tile that is skipped, written
    twice or written to the wrong place cannot hide between samples."""
    out = []
    for s in range(0, n, tile):
        e = min(s + tile, n)
        out += [s, e - 1]
        out += list(rng.integers(s, e, size=interior))
    return np.unique(np.asarray(out, dtype=np.int64))


def assert_tiles_covered(tokens, cols, T, N):
    """Every (256-token, 320-output) tile holds a sampled token and a sampled
    output."""
    tm = set((np.asarray(tokens) // GEMM_TILE_M).tolist())
    tn = set((np.asarray(cols) // GEMM_TILE_N).tolist())
    assert tm == set(range(-(-T // GEMM_TILE_M))), "a token tile has no sample"
    assert tn == set(range(-(-N // GEMM_TILE_N))), "an output tile has no sample"
