"""Seeded synthetic inputs for the block-sparse attention workloads.

This module only draws random numbers and lays out arrays.  It contains none
of the method's arithmetic (no scores, no selection, no attention); both the
CPU oracle and the GPU path consume exactly the arrays built here.

Streams: every tensor (and every chunk of a large tensor) draws from its own
``numpy.random.PCG64`` seeded with ``SeedSequence([seed, cfg_id, tensor_id,
*chunk])``, so the bits do not depend on the number of worker threads.

bf16 tensors are returned as ``uint16`` bit patterns; fp32 samples are
rounded to bf16 with round-to-nearest-even on the bit pattern.

Planting (a stand-in for the retrieval cases the pages evaluate, e.g. the
needle test in HGA "Resultados Experimentales"):
  * indexer: planted key blocks get ``kI = qI + U{-1,0,1}`` ("noise") or
    ``kI = qI`` ("copy"), so they rank high under the weighted-ReLU score of
    SpotAttention §1;
  * keys: every token of a planted block in a retrieving KV group gets
    ``K += boost * qbar_g`` with ``qbar_g`` the mean of that group's query
    heads, so the planted tokens carry a known share of the dense softmax
    mass.  ``boost`` is either given or solved on the drawn queries (see
    ``solved_boost``).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List

import numpy as np

from .configs import DecodeConfig, PrefillConfig

# tensor ids for the seed sequences
TID_Q, TID_K, TID_V, TID_QI, TID_KI, TID_W, TID_PLANT, TID_NOISE, TID_GROUPS, TID_PERM = range(1, 11)
TID_HH, TID_HHDIR, TID_HHIDX = range(11, 14)


def rng_for(seed: int, cfg_id: int, tensor_id: int, *chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg_id, tensor_id, *chunk])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even) and return the bit pattern."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads(threads) -> int:
    if threads:
        return int(threads)
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def analytic_boost(d: int, G: int, T: int, n_plant_tok: int, mass: float) -> float:
    """Shape-only key boost for a planted mass.

    With q, k ~ N(0,1) and logit scale 1/sqrt(d), a planted logit gains
    boost * (q_h . qbar_g) / sqrt(d), about boost * sqrt(d) / G on average;
    solving n_p e^{c b} / (n_p e^{c b} + n_u) = mass for b gives the value below.
    """
    c = math.sqrt(d) / G
    n_u = T - n_plant_tok
    return math.log(mass / (1.0 - mass) * n_u / n_plant_tok) / c


def solved_boost(c_heads: np.ndarray, n_plant_tok: int, T: int, mass: float) -> float:
    """Key boost b with mean_h n_p e^{b c_h} / (n_p e^{b c_h} + n_u) = mass.

    ``c_h`` = (q_h . qbar_g) / sqrt(d) is the logit shift a unit boost gives
    head h.  Planted and unplanted logits share the same random part, whose
    moment cancels in the ratio.  Bisection on a monotone function of b.  The
    realised mass is measured with the oracle by the tests.
    """
    n_u = T - n_plant_tok
    c = np.asarray(c_heads, dtype=np.float64)

    def frac(b):
        e = n_plant_tok * np.exp(b * c)
        return float(np.mean(e / (e + n_u)))

    lo, hi = 0.0, 64.0
    for _ in range(80):
        mid = 0.5 * (lo + hi)
        if frac(mid) < mass:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def decode_boost(cfg: DecodeConfig, qf: np.ndarray, qbar: np.ndarray, ret_groups) -> float:
    """Boost for a decode workload: given, or solved on the drawn queries."""
    if cfg.plant_boost is not None:
        return float(cfg.plant_boost)
    G = cfg.G
    c = [float(qf[b, h] @ qbar[b, h // G]) / math.sqrt(cfg.d)
         for b in range(cfg.B) for h in range(cfg.Hq) if (h // G) in set(int(x) for x in ret_groups)]
    n_tok = int(round(0.5 * (cfg.n_plant[0] + cfg.n_plant[1]))) * cfg.blk
    return solved_boost(np.array(c), n_tok, cfg.T, cfg.plant_mass)


def _normal_chunks(shape, seed, cfg_id, tid, chunk_dims: int, dtype: str, threads,
                   post=None) -> np.ndarray:
    """Fill an array of ``shape`` with N(0,1), one stream per leading index tuple.

    ``post(chunk_index, fp32_chunk)`` may modify a chunk in place before rounding.
    """
    out = np.empty(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
    lead = shape[:chunk_dims]
    inner = shape[chunk_dims:]
    idxs = list(np.ndindex(*lead))

    def work(ix):
        x = rng_for(seed, cfg_id, tid, *ix).standard_normal(inner, dtype=np.float32)
        if post is not None:
            post(ix, x)
        out[ix] = f32_to_bf16_bits(x) if dtype == "bf16" else x

    nt = _threads(threads)
    if nt == 1 or len(idxs) == 1:
        for ix in idxs:
            work(ix)
    else:
        with ThreadPoolExecutor(max_workers=nt) as ex:
            list(ex.map(work, idxs))
    return out


def as_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


def make_decode_index(cfg: DecodeConfig, seed: int = 0) -> Dict:
    """Indexer inputs, head roles and planted blocks of a decode workload (no K/V)."""
    B, Hq, Hkv, d, T, blk = cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.T, cfg.blk
    nb, G, Hi, r = cfg.nb, cfg.G, cfg.H_idx, cfg.r
    seq_len = np.array(cfg.seq_lens if cfg.seq_lens is not None else [T] * B, dtype=np.int32)
    assert seq_len.shape == (B,) and int(seq_len.max()) <= T and int(seq_len.min()) >= 1

    # retrieval groups vs local groups (RTPurbo §1 head specialisation)
    if cfg.n_retrieval_groups is None:
        ret_groups = np.arange(Hkv)
    else:
        ret_groups = np.sort(rng_for(seed, cfg.cfg_id, TID_GROUPS).choice(
            Hkv, cfg.n_retrieval_groups, replace=False))
    head_mode = np.ones(Hkv, dtype=np.uint8)
    head_mode[ret_groups] = 0

    # indexer inputs
    qI = rng_for(seed, cfg.cfg_id, TID_QI).integers(cfg.idx_lo, cfg.idx_hi + 1, size=(B, Hi, r), dtype=np.int8)
    kI = rng_for(seed, cfg.cfg_id, TID_KI).integers(cfg.idx_lo, cfg.idx_hi + 1, size=(B, nb, Hi, r), dtype=np.int8)
    w = rng_for(seed, cfg.cfg_id, TID_W).integers(1, 5, size=(B, Hi), dtype=np.int8)

    # planted blocks, drawn without replacement among the non-reserved blocks;
    # with per-group selection each KV group gets its own blocks, copied into
    # its own indexer heads only
    if cfg.per_group:
        assert Hi % Hkv == 0, "per-group selection needs H_idx divisible by Hkv"
        hpg = Hi // Hkv
        planted_g: List[List[np.ndarray]] = []
        for b in range(B):
            nbv = -(-int(seq_len[b]) // blk)
            cand = np.arange(cfg.n_sink, max(cfg.n_sink, nbv - cfg.n_local))
            row = []
            for gq in range(Hkv):
                g = rng_for(seed, cfg.cfg_id, TID_PLANT, b, gq)
                lo, hi = cfg.n_plant
                n = min(int(g.integers(lo, hi + 1)) if hi > lo else lo, len(cand))
                sel = np.sort(g.choice(cand, n, replace=False)) if n > 0 else np.zeros(0, dtype=np.int64)
                row.append(sel.astype(np.int32))
                hs = slice(gq * hpg, (gq + 1) * hpg)
                if n == 0:
                    continue
                if cfg.plant_kind == "copy":
                    kI[b, sel, hs] = qI[b, hs][None]
                else:
                    noise = rng_for(seed, cfg.cfg_id, TID_NOISE, b, gq).integers(-1, 2, size=(n, hpg, r))
                    kI[b, sel, hs] = np.clip(qI[b, hs][None].astype(np.int16) + noise, -128, 127).astype(np.int8)
            planted_g.append(row)
        planted = [np.unique(np.concatenate(row)).astype(np.int32) for row in planted_g]
        return dict(cfg=cfg, seed=seed, qI=qI, kI=kI, w=w, seq_len=seq_len, head_mode=head_mode,
                    planted=planted, planted_g=planted_g, ret_groups=ret_groups.astype(np.int32))
    planted: List[np.ndarray] = []
    for b in range(B):
        g = rng_for(seed, cfg.cfg_id, TID_PLANT, b)
        nbv = -(-int(seq_len[b]) // blk)
        cand = np.arange(cfg.n_sink, max(cfg.n_sink, nbv - cfg.n_local))
        lo, hi = cfg.n_plant
        n = int(g.integers(lo, hi + 1)) if hi > lo else lo
        n = min(n, len(cand))
        sel = np.sort(g.choice(cand, n, replace=False)) if n > 0 else np.zeros(0, dtype=np.int64)
        planted.append(sel.astype(np.int32))
        if n == 0:
            continue
        if cfg.plant_kind == "copy":
            kI[b, sel] = qI[b][None]
        else:
            noise = rng_for(seed, cfg.cfg_id, TID_NOISE, b).integers(-1, 2, size=(n, Hi, r))
            kI[b, sel] = np.clip(qI[b][None].astype(np.int16) + noise, -128, 127).astype(np.int8)
    return dict(cfg=cfg, seed=seed, qI=qI, kI=kI, w=w, seq_len=seq_len, head_mode=head_mode,
                planted=planted, ret_groups=ret_groups.astype(np.int32))


def make_decode(cfg: DecodeConfig, seed: int = 0, threads=None) -> Dict:
    B, Hq, Hkv, d, T, blk = cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.T, cfg.blk
    G = cfg.G
    idx = make_decode_index(cfg, seed)
    planted, ret_groups = idx["planted"], idx["ret_groups"]

    q = _normal_chunks((B, Hq, d), seed, cfg.cfg_id, TID_Q, 0, cfg.dtype, 1)
    qf = as_f32(q, cfg.dtype)
    qbar = qf.reshape(B, Hkv, G, d).mean(axis=2, dtype=np.float32)  # [B, Hkv, d]
    boost = decode_boost(cfg, qf, qbar, ret_groups) if any(len(p) for p in planted) else 0.0
    ret_set = set(int(x) for x in ret_groups)

    planted_g = idx.get("planted_g")

    def plant_k(ix, x):
        b, g = ix
        blocks = planted_g[b][g] if planted_g is not None else planted[b]
        if g not in ret_set or len(blocks) == 0:
            return
        rows = (blocks[:, None] * blk + np.arange(blk)[None, :]).reshape(-1)
        rows = rows[rows < T]
        x[rows] += np.float32(boost) * qbar[b, g][None, :]

    k = _normal_chunks((B, Hkv, T, d), seed, cfg.cfg_id, TID_K, 2, cfg.dtype, threads, post=plant_k)
    v = _normal_chunks((B, Hkv, T, d), seed, cfg.cfg_id, TID_V, 2, cfg.dtype, threads)
    return dict(idx, q=q, k=k, v=v, boost=float(boost))


def make_prefill(cfg: PrefillConfig, seed: int = 0, threads=None) -> Dict:
    B, T, Hq, Hkv, d, blk = cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.d, cfg.blk
    Hi, r, nb, G = cfg.H_idx, cfg.r, cfg.nb, cfg.G
    hh = None
    q_post = k_post = None
    if cfg.hh_frac > 0:
        # heavy hitters: uniform positions per sequence, one shared direction per KV head
        n_hh = max(1, int(round(cfg.hh_frac * T)))
        hh = [np.sort(rng_for(seed, cfg.cfg_id, TID_HH, b).choice(T, n_hh, replace=False)) for b in range(B)]
        c = rng_for(seed, cfg.cfg_id, TID_HHDIR).standard_normal((Hkv, d)).astype(np.float32)

        def q_post(ix, x):
            x += np.float32(cfg.hh_q) * c[ix[1] // G][None, :]

        def k_post(ix, x):
            x[hh[ix[0]]] += np.float32(cfg.hh_k) * c[ix[1]][None, :]
    q = _normal_chunks((B, Hq, T, d), seed, cfg.cfg_id, TID_Q, 2, cfg.dtype, threads, post=q_post)
    k = _normal_chunks((B, Hkv, T, d), seed, cfg.cfg_id, TID_K, 2, cfg.dtype, threads, post=k_post)
    v = _normal_chunks((B, Hkv, T, d), seed, cfg.cfg_id, TID_V, 2, cfg.dtype, threads)
    if hh is None:
        qI_tok = rng_for(seed, cfg.cfg_id, TID_QI).integers(cfg.idx_lo, cfg.idx_hi + 1, size=(B, T, Hi, r),
                                                            dtype=np.int8)
        kI_tok = rng_for(seed, cfg.cfg_id, TID_KI).integers(cfg.idx_lo, cfg.idx_hi + 1, size=(B, T, Hi, r),
                                                            dtype=np.int8)
    else:
        # queries share an indexer direction cI (plus half-range noise); heavy-hitter keys copy it
        cI = rng_for(seed, cfg.cfg_id, TID_HHIDX).integers(-64, 64, size=(Hi, r)).astype(np.int16)
        qn = rng_for(seed, cfg.cfg_id, TID_QI).integers(-64, 64, size=(B, T, Hi, r)).astype(np.int16)
        qI_tok = np.clip(qn + cI[None, None], -128, 127).astype(np.int8)
        kI_tok = rng_for(seed, cfg.cfg_id, TID_KI).integers(cfg.idx_lo, cfg.idx_hi + 1, size=(B, T, Hi, r),
                                                            dtype=np.int8)
        for b in range(B):
            kI_tok[b, hh[b]] = cI.astype(np.int8)[None]
    w = rng_for(seed, cfg.cfg_id, TID_W).integers(1, 5, size=(B, nb, Hi), dtype=np.int8)
    # one independent uniform permutation per segment (PBS-Attn §2)
    perm = np.empty(T, dtype=np.int32)
    for s0 in range(0, T, cfg.seg):
        n = min(cfg.seg, T - s0)
        perm[s0:s0 + n] = s0 + rng_for(seed, cfg.cfg_id, TID_PERM, s0 // cfg.seg).permutation(n)
    return dict(cfg=cfg, seed=seed, q=q, k=k, v=v, qI_tok=qI_tok, kI_tok=kI_tok, w=w, perm=perm, hh=hh,
                seq_len=np.full(B, T, dtype=np.int32))


def make(cfg, seed: int = 0, threads=None) -> Dict:
    if isinstance(cfg, DecodeConfig):
        return make_decode(cfg, seed, threads)
    return make_prefill(cfg, seed, threads)
