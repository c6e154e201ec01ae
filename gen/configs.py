"""Workload shapes for the synthetic block-sparse attention inputs.

Each configuration is a plain description of sizes, value ranges and the
planted structure; ``gen.synth`` turns it into seeded arrays.  Nothing here
computes any part of the attention method.

The five named workloads follow the shapes the pages measure on: long
contexts of 32K-128K tokens (RTPurbo "Resultados Clave"; SpotAttention
"Resultados"), 64-token chunks (HGA "Mecanismo Central", partitioning),
16-token selector blocks (SpotAttention §1 "Arquitectura del Selector"),
rank-16 indexer projections (RTPurbo §2), dual top-p with sink and recency
blocks and a floor K_min (SpotAttention §3), retrieval vs. local heads
(RTPurbo §1) and segment-wise permutation of 4096-token segments (PBS-Attn
§2).  ``small_*`` variants keep the structure at sizes the CPU oracle
finishes in seconds, with ragged sequence lengths.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    cfg_id: int
    B: int
    Hq: int
    Hkv: int
    d: int
    T: int                      # cache capacity (tokens) per sequence
    blk: int                    # key-block size in tokens
    H_idx: int
    r: int
    dtype: str                  # "f32" or "bf16"
    n_sink: int                 # reserved sink blocks
    n_local: int                # reserved most-recent blocks
    select: str                 # "topk" or "topp"
    k: int = 0                  # top-k budget
    p: float = 0.0              # top-p threshold
    beta: float = 1.0           # logit scale applied to integer scores
    k_min: int = 0
    k_max: int = 0
    idx_lo: int = -8            # indexer int8 value range (inclusive)
    idx_hi: int = 7
    # planting
    plant_kind: str = "noise"   # "noise": kI = qI + U{-1,0,1}; "copy": kI = qI
    n_plant: Tuple[int, int] = (0, 0)   # per-sequence count ~ U{lo..hi}
    plant_boost: Optional[float] = None  # K += boost*qbar; None -> solved for plant_mass
    # (the 128K top-p workload reuses 1.5, the value solved for the 32K workload, rounded)
    plant_mass: float = 0.0              # target head-averaged planted mass
    n_retrieval_groups: Optional[int] = None  # None -> every KV group retrieves
    local_sink_tok: int = 0
    local_window_tok: int = 0
    seq_lens: Optional[Tuple[int, ...]] = None  # None -> every sequence is full (T)
    # one selection per KV group from its own indexer heads (H_idx / Hkv each),
    # with blocks planted per group (SparDA §2, one forecast head per GQA group)
    per_group: bool = False
    # selector key cache held as micro-scaled int4 (SpotAttention §4)
    selector_q4: bool = False

    @property
    def nb(self) -> int:
        return -(-self.T // self.blk)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def cap(self) -> int:
        """Longest selected-block list a row can produce."""
        budget = self.k if self.select == "topk" else self.k_max
        return min(self.nb, self.n_sink + self.n_local + budget)


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    cfg_id: int
    B: int
    T: int
    Hq: int
    Hkv: int
    d: int
    blk: int                    # query block == key block size
    H_idx: int
    r: int
    k: int                      # top-k past blocks per query block
    n_sink: int                 # sink blocks always kept (block 0 of the permuted order)
    n_local: int                # recent blocks kept right before the diagonal
    seg: int                    # permutation segment length (tokens)
    idx_lo: int = -128
    idx_hi: int = 127
    dtype: str = "bf16"
    # heavy-hitter keys (PBS-Attn §3): a fraction of key positions, scattered
    # uniformly, that every query attends strongly (a shared direction c_g per
    # KV head: q += hh_q*c, k_hh += hh_k*c) and whose indexer keys copy a
    # shared indexer direction; 0 = none
    hh_frac: float = 0.0
    hh_q: float = 0.7
    hh_k: float = 0.7
    # key order: "random" (one uniform permutation per segment) or
    # "importance" (sorted by the importance of the last query block)
    perm_kind: str = "random"
    proxy: int = 64             # proxy queries for the importance (the last block)

    @property
    def nb(self) -> int:
        return -(-self.T // self.blk)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def cap(self) -> int:
        return min(self.nb, self.n_sink + self.n_local + 1 + self.k)


# --- the five named workloads -------------------------------------------

TINY_DECODE = DecodeConfig(
    name="tiny_decode_f32", cfg_id=1, B=1, Hq=4, Hkv=1, d=64, T=1024, blk=16,
    H_idx=2, r=16, dtype="f32", n_sink=1, n_local=2, select="topk", k=8,
    plant_kind="noise", n_plant=(3, 3), plant_boost=2.0)

DECODE_32K = DecodeConfig(
    name="decode_32k_bf16", cfg_id=2, B=1, Hq=32, Hkv=8, d=128, T=32768, blk=64,
    H_idx=8, r=16, dtype="bf16", n_sink=1, n_local=4, select="topk", k=64,
    plant_kind="noise", n_plant=(16, 16), plant_mass=0.60)

DECODE_128K_TOPP = DecodeConfig(
    name="decode_128k_topp_bf16", cfg_id=3, B=16, Hq=64, Hkv=8, d=128, T=131072,
    blk=64, H_idx=8, r=16, dtype="bf16", n_sink=1, n_local=4, select="topp",
    p=0.9, beta=0.125, k_min=16, k_max=512,
    plant_kind="copy", n_plant=(1, 200), plant_boost=1.5)

DECODE_64K_HEADSPLIT = DecodeConfig(
    name="decode_64k_headsplit_bf16", cfg_id=4, B=8, Hq=32, Hkv=8, d=128, T=65536,
    blk=64, H_idx=8, r=16, dtype="bf16", n_sink=1, n_local=4, select="topk", k=32,
    plant_kind="noise", n_plant=(16, 16), plant_mass=0.60, n_retrieval_groups=2,
    local_sink_tok=4, local_window_tok=2048)

DECODE_128K_PERGROUP = DecodeConfig(
    name="decode_128k_pergroup_bf16", cfg_id=6, B=16, Hq=64, Hkv=8, d=128, T=131072,
    blk=64, H_idx=8, r=16, dtype="bf16", n_sink=1, n_local=4, select="topk", k=64,
    plant_kind="copy", n_plant=(8, 32), plant_boost=1.5, per_group=True)

DECODE_128K_TOPP_Q4 = replace(DECODE_128K_TOPP, name="decode_128k_topp_q4_bf16", cfg_id=8, selector_q4=True)

PREFILL_64K = PrefillConfig(
    name="prefill_64k_permuted_bf16", cfg_id=5, B=1, T=65536, Hq=32, Hkv=8, d=128,
    blk=64, H_idx=8, r=16, k=32, n_sink=1, n_local=0, seg=4096)

PREFILL_64K_IMPORTANCE = replace(
    PREFILL_64K, name="prefill_64k_importance_bf16", cfg_id=7, hh_frac=1 / 64, perm_kind="importance")

# --- small variants: same structure, oracle-friendly sizes, ragged tails ---

SMALL_DECODE_TOPK = replace(
    DECODE_32K, name="small_decode_topk_bf16", cfg_id=12, B=3, T=4096,
    n_plant=(6, 6), k=12, seq_lens=(4096, 2949, 1000))

SMALL_DECODE_TOPP = replace(
    DECODE_128K_TOPP, name="small_decode_topp_bf16", cfg_id=13, B=4, Hq=16, Hkv=2,
    T=8192, k_min=4, k_max=48, n_plant=(1, 40), seq_lens=(8192, 8000, 6113, 3001))

SMALL_DECODE_HEADSPLIT = replace(
    DECODE_64K_HEADSPLIT, name="small_decode_headsplit_bf16", cfg_id=14, B=2, Hq=16,
    Hkv=4, T=8192, k=10, n_plant=(5, 5), n_retrieval_groups=2,
    local_sink_tok=4, local_window_tok=1000, seq_lens=(8192, 5001))

SMALL_TINY_RAGGED = replace(
    TINY_DECODE, name="small_tiny_ragged_f32", cfg_id=11, B=2, d=128, Hq=8, Hkv=2,
    seq_lens=(1024, 777))

SMALL_DECODE_PERGROUP = replace(
    DECODE_32K, name="small_decode_pergroup_bf16", cfg_id=16, B=3, Hq=16, Hkv=4, H_idx=8, T=8192,
    n_plant=(3, 8), k=10, per_group=True, plant_mass=0.0, plant_boost=1.5, seq_lens=(8192, 5001, 1500))

SMALL_DECODE_TOPP_Q4 = replace(SMALL_DECODE_TOPP, name="small_decode_topp_q4_bf16", cfg_id=18, selector_q4=True)

SMALL_PREFILL = replace(
    PREFILL_64K, name="small_prefill_bf16", cfg_id=15, T=2048, Hq=8, Hkv=2, k=6,
    seg=512)

SMALL_PREFILL_IMPORTANCE = replace(
    PREFILL_64K_IMPORTANCE, name="small_prefill_importance_bf16", cfg_id=17, T=2048, Hq=8, Hkv=2, k=6,
    seg=512)

NAMED = {c.name: c for c in (
    TINY_DECODE, DECODE_32K, DECODE_128K_TOPP, DECODE_64K_HEADSPLIT, PREFILL_64K,
    DECODE_128K_PERGROUP, PREFILL_64K_IMPORTANCE, SMALL_PREFILL_IMPORTANCE, DECODE_128K_TOPP_Q4,
    SMALL_DECODE_TOPP_Q4,
    SMALL_DECODE_TOPK, SMALL_DECODE_TOPP, SMALL_DECODE_HEADSPLIT, SMALL_TINY_RAGGED,
    SMALL_DECODE_PERGROUP, SMALL_PREFILL)}

BY_ID = {c.cfg_id: c for c in NAMED.values()}
