"""Seeded synthetic inputs for the engram hot path (shared by the tests, the
benchmark and the smoke check).  Holds shapes and distributions only."""
from .workloads import (Workload, WORKLOADS, TINY_E4M3, DECODE_Q2K, PREFILL_Q2K,
                        SPLIT_E4M3, GATHER_Q2K, DECODE_WKVQ2K, ODD_Q2K, ODD_E4M3,
                        ODD_WKVQ2K, ODD_E4M3_WKVQ2K, MAX_SLOTS_Q2K,
                        MAX_NGRAM_E4M3, HC1_Q2K, HC3_E4M3, HC2_WKVQ2K)
from . import generate

__all__ = ["Workload", "WORKLOADS", "TINY_E4M3", "DECODE_Q2K", "PREFILL_Q2K",
           "SPLIT_E4M3", "GATHER_Q2K", "DECODE_WKVQ2K", "ODD_Q2K", "ODD_E4M3", "ODD_WKVQ2K",
           "ODD_E4M3_WKVQ2K", "MAX_SLOTS_Q2K", "MAX_NGRAM_E4M3", "HC1_Q2K", "HC3_E4M3",
           "HC2_WKVQ2K", "generate"]
