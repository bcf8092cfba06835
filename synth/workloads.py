"""Geometry of the synthetic engram workloads.

Each workload fixes the hash geometry (vocabulary, compressed id space, n-gram
size, heads, layers, prime range), the table format, the projection shape and
the token stream.  Sizes follow the DeepSeek-V4.1 Flash engram as the
atlascybernetics page "spark_model/layers/engram_v41.rs" describes it (module
doc: four stages; `EngramV41::new`: hc in 1..=4; `ENGRAM_ROW_BYTES`: one 84-byte
Q2_K block per 256-wide row) and the metrale page
"metrale_model_arch/deepseek_v41_ref/engram.rs" (`EngramTables`: fp8 e4m3 rows
with power-of-two scales per `scale_block` values).

No arithmetic of the method lives here: only shapes and distributions.
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    # table family: workloads that share hash tables, tables and weights
    # share a family id (the prefill workload reuses the decode tables)
    family: int
    vocab: int
    compressed: int          # size of the compressed id space
    p_unmapped: float        # probability that a vocab id maps to -1
    max_ngram: int
    n_heads: int
    n_layers: int
    prime_lo: int            # primes drawn distinct from [prime_lo, prime_hi]
    prime_hi: int
    fmt: str                 # "q2k" or "e4m3"
    head_dim: int = 256
    scale_block: int = 128   # e4m3 only: values per power-of-two scale
    scale_k_lo: int = -4     # e4m3 only: scale = 2**k, k uniform in [lo, hi]
    scale_k_hi: int = 0
    dim: int = 4096
    hc: int = 4
    token_dist: str = "uniform"   # "uniform" or "zipf"
    zipf_s: float = 1.1
    # token stream: `prompt` tokens as one prefill call (in chunks of
    # `chunk`), then `decode_steps` single-token steps
    prompt: int = 64
    chunk: int = 0           # 0 = one call for the whole prompt
    decode_steps: int = 0
    eps: float = 1e-6
    wkv_std: float = 0.02
    # "bf16": wkv as bf16 [N, K]; "q2k": wkv as Q2_K blocks [N, K/256, 84]
    # (the form the GGUF ships), fp16 d and dmin uniform in [wkv_d_lo, wkv_d_hi]
    wkv_fmt: str = "bf16"
    wkv_d_lo: float = 1e-3
    wkv_d_hi: float = 2e-3
    qk_std: float = 0.05     # q, k = bf16(1 + qk_std * N(0,1))
    pad_id: int = 0

    @property
    def cols(self) -> int:
        return (self.max_ngram - 1) * self.n_heads

    @property
    def K(self) -> int:
        return self.cols * self.head_dim

    @property
    def N(self) -> int:
        return self.dim * (self.hc + 1)

    @property
    def total_tokens(self) -> int:
        return self.prompt + self.decode_steps

    @property
    def row_bytes(self) -> int:
        if self.fmt == "q2k":
            return 84
        return self.head_dim + 4 * (self.head_dim // self.scale_block)


TINY_E4M3 = Workload(
    name="tiny_e4m3_T64", family=0, vocab=1024, compressed=800, p_unmapped=0.10,
    max_ngram=3, n_heads=2, n_layers=1, prime_lo=500, prime_hi=1000, fmt="e4m3",
    dim=256, hc=4, token_dist="uniform", prompt=64)

DECODE_Q2K = Workload(
    name="decode_q2k_2layer_T1", family=1, vocab=129280, compressed=100000,
    p_unmapped=0.15, max_ngram=4, n_heads=8, n_layers=2, prime_lo=2**17,
    prime_hi=2**18, fmt="q2k", token_dist="uniform", prompt=32, decode_steps=256)

PREFILL_Q2K = replace(
    DECODE_Q2K, name="prefill_q2k_2layer_T4096", token_dist="zipf", prompt=4096,
    decode_steps=0)

# the decode workload with wkv given as Q2_K blocks (atlascybernetics
# "engram_v41.rs", EngramLayerWeights::wkv_q2k): same tables, tokens per step
# and highway shape
DECODE_WKVQ2K = replace(DECODE_Q2K, name="decode_q2k_wkvq2k_2layer_T1", wkv_fmt="q2k")

SPLIT_E4M3 = Workload(
    name="split_e4m3_2layer_8192x2048_then_128", family=3, vocab=129280,
    compressed=100000, p_unmapped=0.15, max_ngram=4, n_heads=8, n_layers=2,
    prime_lo=2**17, prime_hi=2**18, fmt="e4m3", token_dist="zipf", prompt=8192,
    chunk=2048, decode_steps=128)

GATHER_Q2K = Workload(
    name="gather_stress_q2k_1layer_T16384", family=4, vocab=129280,
    compressed=100000, p_unmapped=0.15, max_ngram=4, n_heads=8, n_layers=1,
    prime_lo=2**21, prime_hi=2**22, fmt="q2k", token_dist="uniform", prompt=16384)

# edge-case geometry for the tests: an odd number of columns (max_ngram 2, 5
# heads -> 5 columns, K 1280 = 2.5 KiB rows of bf16: an odd number of 1 KiB
# loads a row and a partial last 16-value-sub-block round), small tables and
# hc * dim = 1024; Q2_K and e4m3 tables, and wkv as Q2_K blocks
ODD_Q2K = Workload(
    name="odd_cols_q2k_2layer", family=5, vocab=1024, compressed=800, p_unmapped=0.10,
    max_ngram=2, n_heads=5, n_layers=2, prime_lo=500, prime_hi=1000, fmt="q2k", dim=256,
    hc=4, token_dist="uniform", prompt=8, decode_steps=24)
ODD_E4M3 = replace(ODD_Q2K, name="odd_cols_e4m3_2layer", family=6, fmt="e4m3")
ODD_WKVQ2K = replace(ODD_Q2K, name="odd_cols_q2k_wkvq2k_2layer", wkv_fmt="q2k")
ODD_E4M3_WKVQ2K = replace(ODD_E4M3, name="odd_cols_e4m3_wkvq2k_2layer", wkv_fmt="q2k")

# the largest hash geometries the library takes: 4 layers of 32 columns (128
# hash slots, K 8192: the one-launch decode kernels' limit) with Q2_K tables,
# and the longest n-gram (8) with 4 heads (28 columns a layer, 112 slots) with
# e4m3 tables; small vocabularies and tables, hc * dim = 1024
MAX_SLOTS_Q2K = Workload(
    name="max_slots_q2k_4layer", family=7, vocab=1024, compressed=800, p_unmapped=0.10,
    max_ngram=5, n_heads=8, n_layers=4, prime_lo=500, prime_hi=3000, fmt="q2k", dim=256,
    hc=4, token_dist="uniform", prompt=8, decode_steps=16)
MAX_NGRAM_E4M3 = Workload(
    name="max_ngram_e4m3_4layer", family=8, vocab=1024, compressed=800, p_unmapped=0.10,
    max_ngram=8, n_heads=4, n_layers=4, prime_lo=500, prime_hi=3000, fmt="e4m3", dim=256,
    hc=4, token_dist="uniform", prompt=8, decode_steps=16)

# other hyper-connection counts (atlascybernetics "engram_v41.rs", EngramV41::new:
# hc in 1..=4): one stream with dim 512, three with dim 768 and 9 columns (K 2304,
# not a multiple of 1024), and two streams with wkv as Q2_K blocks
HC1_Q2K = Workload(
    name="hc1_q2k_2layer", family=9, vocab=1024, compressed=800, p_unmapped=0.10,
    max_ngram=3, n_heads=4, n_layers=2, prime_lo=500, prime_hi=1000, fmt="q2k", dim=512,
    hc=1, token_dist="uniform", prompt=8, decode_steps=16)
HC3_E4M3 = Workload(
    name="hc3_e4m3_2layer", family=10, vocab=1024, compressed=800, p_unmapped=0.10,
    max_ngram=4, n_heads=3, n_layers=2, prime_lo=500, prime_hi=1000, fmt="e4m3", dim=768,
    hc=3, token_dist="uniform", prompt=8, decode_steps=16)
HC2_WKVQ2K = replace(HC1_Q2K, name="hc2_q2k_wkvq2k_2layer", dim=256, hc=2, wkv_fmt="q2k")

WORKLOADS = {w.name: w for w in (TINY_E4M3, DECODE_Q2K, PREFILL_Q2K, SPLIT_E4M3, GATHER_Q2K,
                                 DECODE_WKVQ2K, ODD_Q2K, ODD_E4M3, ODD_WKVQ2K, ODD_E4M3_WKVQ2K,
                                 MAX_SLOTS_Q2K, MAX_NGRAM_E4M3, HC1_Q2K, HC3_E4M3, HC2_WKVQ2K)}
# seed index of each workload's token / highway stream (tables use `family`)
STREAM_INDEX = {TINY_E4M3.name: 0, DECODE_Q2K.name: 1, PREFILL_Q2K.name: 2,
                SPLIT_E4M3.name: 3, GATHER_Q2K.name: 4, DECODE_WKVQ2K.name: 5,
                ODD_Q2K.name: 6, ODD_E4M3.name: 7, ODD_WKVQ2K.name: 8,
                MAX_SLOTS_Q2K.name: 9, MAX_NGRAM_E4M3.name: 10, ODD_E4M3_WKVQ2K.name: 11,
                HC1_Q2K.name: 12, HC3_E4M3.name: 13, HC2_WKVQ2K.name: 14}
