"""CPU oracle for query-dependent block-sparse attention with an int8 indexer.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
reference that the HIP path is checked against.  Only the test suite, the
package smoke check and the benchmark's CPU-baseline leg may import it; the
product path never calls it.  It shares no code with the HIP library.

Integers are computed in numpy int64, floating point in float64.  bf16 inputs
arrive as uint16 bit patterns and are widened exactly.

What each function follows (page title, section):
  * scores        -- SpotAttention, §1 "Arquitectura del Selector": per query
                     row and key block, the sum over indexer heads of the head
                     weight times ReLU of the dot product of the head's query
                     and key projections; rank-16 projections per RTPurbo §2.
  * block pooling -- PBS-Attn §4 "Implementación": block importance from mean
                     pooling; HGA "Mecanismo Central" (chunk summaries).
  * top-k         -- RTPurbo §3 (static top-k budget) with the reserved sink /
                     recency blocks of SpotAttention §3 and HGA's always-visible
                     sink, local and current chunks.
  * top-p         -- RTPurbo §3 and SpotAttention §3 (dual top-p): nucleus over
                     the residual distribution (candidates only), stop once the
                     cumulative mass reaches p, floor K_min.
  * per-group     -- SparDA §2 "Indexador de Pronóstico Compacto": one indexer
    selection        head (set) per GQA group, each group with its own top-k.
  * attention     -- HGA "Atención Exacta de Token": a standard softmax over
                     exactly the selected tokens; RTPurbo §1 for local heads
                     (sliding window plus sink tokens).
  * permutation   -- PBS-Attn §1 (key/value permutation invariance, query
                     equivariance, inverse restores the order) and §2
                     (permutation only inside segments of size S).
  * int4 selector -- SpotAttention §4 "Cuantización": the selector's key cache
    keys             in micro-scaled int4 (one scale per r-vector), scored
                     with the dequantized keys.
  * importance    -- PBS-Attn §3 "Permutación de Claves Basada en Importancia
    permutation      Global": the last query block as proxy, mean pooling of
                     its attention probabilities into one importance per key,
                     keys sorted by descending importance inside each segment.

Readings where the pages are silent (sentinel values, tie order, pooling
rounding, reserved counts) are listed at the top of each function.
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import numpy as np

INT32_MIN = -(2 ** 31)


# --------------------------------------------------------------------------
# value widening
# --------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_to_f64(x) if dtype == "bf16" else np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# indexer: pooling and scores
# --------------------------------------------------------------------------

def pool_blocks(x_tok: np.ndarray, blk: int) -> np.ndarray:
    """Mean-pool per-token int8 indexer vectors into per-block int8 vectors.

    x_tok: [B, T, H, r] int8 -> [B, ceil(T/blk), H, r] int8.
    Reading: the mean over the block's n tokens rounded as floor(mean + 1/2),
    i.e. floor((2*sum + n) / (2*n)) in exact integers (the pages say only
    "mean pooling").  A ragged last block averages the tokens it has.
    """
    B, T, H, r = x_tok.shape
    nb = -(-T // blk)
    out = np.empty((B, nb, H, r), dtype=np.int8)
    x = x_tok.astype(np.int64)
    for j in range(nb):
        seg = x[:, j * blk:min(T, (j + 1) * blk)]
        n = seg.shape[1]
        s = seg.sum(axis=1)
        m = np.floor_divide(2 * s + n, 2 * n)
        out[:, j] = m.astype(np.int8)
    return out


def quantize_selector_keys(kI: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Micro-scaled int4 selector keys (SpotAttention §4, quantised selector K cache).

    Readings: one micro-block per r-vector (one key block and indexer head);
    its scale is a power of two 2^e so that code * 2^e stays an exact integer
    and the scores stay exact; e is the smallest exponent for which every
    element's floor(x / 2^e + 1/2) lies in the int4 range [-8, 7], and that
    value is the element's code.  kI [..., r] int8 -> codes [..., r] int8 in
    [-8, 7], exps [...] uint8 in [0, 5].
    """
    x = np.asarray(kI).astype(np.int64)
    codes = np.zeros(x.shape, dtype=np.int8)
    exps = np.full(x.shape[:-1], 255, dtype=np.uint8)
    todo = np.ones(x.shape[:-1], dtype=bool)
    for e in range(8):
        c = np.floor_divide(2 * x + 2 ** e, 2 ** (e + 1))   # floor(x / 2^e + 1/2)
        ok = todo & (c.min(axis=-1) >= -8) & (c.max(axis=-1) <= 7)
        codes[ok] = c[ok]
        exps[ok] = e
        todo &= ~ok
    assert not todo.any()
    return codes, exps


def dequantize_selector_keys(codes: np.ndarray, exps: np.ndarray) -> np.ndarray:
    """code * 2^e as exact integers (int16)."""
    return (codes.astype(np.int16) * (1 << exps.astype(np.int16))[..., None]).astype(np.int16)


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Storage format: two codes per byte, element 2c in the low nibble and 2c+1 in
    the high nibble, each as 4-bit two's complement.  [..., r] -> [..., r/2] uint8."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def head_dots(qv: np.ndarray, kv: np.ndarray) -> np.ndarray:
    """qv [..., H, r], kv [J, H, r] -> per-head dot products [..., J, H] (int64)."""
    return np.einsum("...hc,jhc->...jh", qv.astype(np.int64), kv.astype(np.int64))


def score_decode(qI: np.ndarray, kI: np.ndarray, w: np.ndarray, seq_len: np.ndarray, blk: int) -> np.ndarray:
    """Decode block scores.

    qI [B, H, r], kI [B, nKb, H, r], w [B, H] (int8) -> scores [B, nKb] int64.
    s[b, j] = sum_h w[b,h] * max(0, qI[b,h,:] . kI[b,j,h,:]) for the valid blocks
    j < ceil(seq_len[b]/blk); INT32_MIN marks blocks past the sequence end.
    """
    B, nKb = kI.shape[:2]
    out = np.full((B, nKb), INT32_MIN, dtype=np.int64)
    for b in range(B):
        nbv = min(nKb, -(-int(seq_len[b]) // blk))
        dots = head_dots(qI[b], kI[b, :nbv])              # [nbv, H]
        s = (np.maximum(dots, 0) * w[b].astype(np.int64)[None, :]).sum(axis=1)
        out[b, :nbv] = s
    assert np.all(np.abs(out[out != INT32_MIN]) < 2 ** 31), "score does not fit int32"
    return out


def score_decode_grouped(qI: np.ndarray, kI: np.ndarray, w: np.ndarray, seq_len: np.ndarray, blk: int,
                         groups: int) -> np.ndarray:
    """Per-KV-group decode block scores (SparDA page, "Indexador de Pronóstico
    Compacto": one forecast head per GQA group instead of one shared selection).

    The H indexer heads are split into ``groups`` equal consecutive sets; group
    g sums over heads g*H/groups .. (g+1)*H/groups - 1 only:
    s[b, g, j] = sum_{h in group g} w[b,h] * max(0, qI[b,h,:] . kI[b,j,h,:]).
    Returns [B, groups, nKb] int64, INT32_MIN past the sequence end.
    """
    B, nKb, H = kI.shape[:3]
    assert H % groups == 0, "indexer heads must split evenly over the groups"
    hpg = H // groups
    out = np.full((B, groups, nKb), INT32_MIN, dtype=np.int64)
    for b in range(B):
        nbv = min(nKb, -(-int(seq_len[b]) // blk))
        dots = head_dots(qI[b], kI[b, :nbv])              # [nbv, H]
        terms = np.maximum(dots, 0) * w[b].astype(np.int64)[None, :]
        for g in range(groups):
            out[b, g, :nbv] = terms[:, g * hpg:(g + 1) * hpg].sum(axis=1)
    assert np.all(np.abs(out[out != INT32_MIN]) < 2 ** 31), "score does not fit int32"
    return out


def score_prefill(qIb: np.ndarray, kIb: np.ndarray, w: np.ndarray, q_blk0: int = 0) -> np.ndarray:
    """Prefill block-pair scores.

    qIb [B, M, H, r] (pooled query blocks q_blk0..q_blk0+M-1), kIb [B, nKb, H, r],
    w [B, M, H] -> scores [B, M, nKb] int64, defined for key blocks j strictly
    before the query block (j < q_blk0 + i); INT32_MIN elsewhere.
    """
    B, M = qIb.shape[:2]
    nKb = kIb.shape[1]
    out = np.full((B, M, nKb), INT32_MIN, dtype=np.int64)
    for b in range(B):
        for i in range(M):
            ia = q_blk0 + i
            J = min(ia, nKb)
            if J <= 0:
                continue
            dots = head_dots(qIb[b, i], kIb[b, :J])     # [J, H]
            out[b, i, :J] = (np.maximum(dots, 0) * w[b, i].astype(np.int64)[None, :]).sum(axis=1)
    assert np.all(np.abs(out[out != INT32_MIN]) < 2 ** 31), "score does not fit int32"
    return out


# --------------------------------------------------------------------------
# selection
# --------------------------------------------------------------------------

def decode_sets(seq_len: int, blk: int, n_sink: int, n_local: int) -> Tuple[List[int], List[int]]:
    """Reserved blocks and candidate blocks of one decode row.

    Sink = the first n_sink blocks, local = the last n_local valid blocks
    (SpotAttention §3 reserved prefix and recency suffix); candidates = the
    valid blocks in neither.
    """
    nbv = -(-int(seq_len) // blk)
    reserved = set(range(min(n_sink, nbv))) | set(range(max(0, nbv - n_local), nbv))
    cand = [j for j in range(nbv) if j not in reserved]
    return sorted(reserved), cand


def prefill_sets(i: int, n_sink: int, n_local: int) -> Tuple[List[int], List[int]]:
    """Reserved and candidate key blocks of prefill query block i (absolute).

    Reserved: the sink blocks, the n_local blocks just before i and the
    current (diagonal) block i -- HGA's always-visible current, sink and local
    chunks.  Candidates: the remaining blocks strictly before i.
    """
    reserved = set(range(min(n_sink, i + 1))) | set(range(max(0, i - n_local), i)) | {i}
    cand = [j for j in range(i) if j not in reserved]
    return sorted(reserved), cand


def rank_order(cand: Sequence[int], s: np.ndarray) -> List[int]:
    """Candidates ordered by score descending, ties by lowest block index."""
    return sorted(cand, key=lambda j: (-int(s[j]), j))


def topk_choose(cand: Sequence[int], s: np.ndarray, k: int) -> List[int]:
    return rank_order(cand, s)[:max(0, k)]


def topp_masses(ordered: Sequence[int], s: np.ndarray, beta: float) -> np.ndarray:
    """Masses of the residual distribution softmax(beta*s) over the candidates, in rank order."""
    if len(ordered) == 0:
        return np.zeros(0)
    lg = beta * np.array([float(s[j]) for j in ordered], dtype=np.float64)
    e = np.exp(lg - lg.max())
    return e / e.sum()


def topp_count(ordered: Sequence[int], s: np.ndarray, beta: float, p: float) -> Tuple[int, np.ndarray]:
    """Smallest prefix length whose cumulative mass reaches p; also the cumulative masses."""
    m = topp_masses(ordered, s, beta)
    M = np.cumsum(m)
    if len(M) == 0:
        return 0, M
    hit = np.nonzero(M >= p)[0]
    kp = int(hit[0]) + 1 if len(hit) else len(M)
    return kp, M


def select_row_topk(reserved, cand, s, k) -> List[int]:
    return sorted(set(reserved) | set(topk_choose(cand, s, k)))


def select_row_topp(reserved, cand, s, beta, p, k_min, k_max) -> Tuple[List[int], Dict]:
    order = rank_order(cand, s)
    kp, M = topp_count(order, s, beta, p)
    k = min(len(order), max(k_min, min(kp, k_max)))
    sel = sorted(set(reserved) | set(order[:k]))
    return sel, dict(order=order, cum=M, kp=kp, k=k)


def select_decode(scores, seq_len, blk, n_sink, n_local, mode, k=0, beta=1.0, p=0.9, k_min=0, k_max=0):
    """Per-sequence selected block lists (ascending) for a decode step."""
    out, info = [], []
    for b in range(scores.shape[0]):
        res, cand = decode_sets(int(seq_len[b]), blk, n_sink, n_local)
        if mode == "topk":
            out.append(select_row_topk(res, cand, scores[b], k))
            info.append(None)
        else:
            sel, inf = select_row_topp(res, cand, scores[b], beta, p, k_min, k_max)
            inf["reserved"] = res
            out.append(sel)
            info.append(inf)
    return out, info


def select_decode_grouped(scores, seq_len, blk, n_sink, n_local, mode, k=0, beta=1.0, p=0.9, k_min=0, k_max=0):
    """Per-(sequence, KV group) selections: the decode rule applied to each group's scores.

    scores [B, groups, nKb]; returns sel[b][g] (ascending lists) and info[b][g].
    """
    B, groups = scores.shape[:2]
    per = [select_decode(np.ascontiguousarray(scores[:, g]), seq_len, blk, n_sink, n_local, mode, k=k, beta=beta,
                         p=p, k_min=k_min, k_max=k_max) for g in range(groups)]
    sel = [[per[g][0][b] for g in range(groups)] for b in range(B)]
    info = [[per[g][1][b] for g in range(groups)] for b in range(B)]
    return sel, info


def select_prefill_topk(scores, n_sink, n_local, k, q_blk0=0):
    """Per (sequence, query block) selected key-block lists for prefill."""
    B, M = scores.shape[:2]
    return [[select_row_topk(*prefill_sets(q_blk0 + i, n_sink, n_local), scores[b, i], k)
             for i in range(M)] for b in range(B)]


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def softmax_attend(qv: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> Tuple[np.ndarray, float]:
    """Standard softmax attention of one query over the rows of K/V (fp64)."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1]), -np.inf
    x = (K @ qv) * scale
    m = x.max()
    e = np.exp(x - m)
    z = e.sum()
    return (e @ V) / z, float(m + np.log(z))


def decode_tokens(sel_blocks, seq_len, blk, mode, sink_tok, window_tok) -> np.ndarray:
    """Token positions one decode head attends.

    Retrieval heads: the tokens of the selected blocks below seq_len.
    Local heads: sink tokens [0, sink_tok) plus the window [seq_len - W, seq_len)
    (RTPurbo §1).  The current token sits at seq_len - 1 and is included.
    """
    L = int(seq_len)
    if mode == 0:
        toks = [t for j in sel_blocks for t in range(j * blk, min((j + 1) * blk, L))]
    else:
        toks = sorted(set(range(min(sink_tok, L))) | set(range(max(0, L - window_tok), L)))
    return np.array(toks, dtype=np.int64)


def decode_attention(q, k, v, dtype, seq_len, sel, blk, head_mode=None, sink_tok=0, window_tok=0,
                     scale=None, heads=None, batches=None, per_group=False):
    """Sparse decode attention for every (sequence, query head), fp64.

    q [B, Hq, d]; k, v [B, Hkv, Tcap, d]; query head h reads KV head h // (Hq/Hkv).
    sel[b] is the sequence's block list, or with ``per_group`` a list of one
    block list per KV head (sel[b][g]).
    Returns o [B, Hq, d] and lse [B, Hq] (NaN for rows not computed when
    ``heads``/``batches`` restrict the work).
    """
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if head_mode is None:
        head_mode = np.zeros(Hkv, dtype=np.uint8)
    o = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    for b in (range(B) if batches is None else batches):
        for h in (range(Hq) if heads is None else heads):
            g = h // G
            blocks = sel[b][g] if per_group else sel[b]
            toks = decode_tokens(blocks, seq_len[b], blk, int(head_mode[g]), sink_tok, window_tok)
            K = to_f64(k[b, g, toks], dtype)
            V = to_f64(v[b, g, toks], dtype)
            o[b, h], lse[b, h] = softmax_attend(to_f64(q[b, h], dtype), K, V, scale)
    return o, lse


def prefill_attention(q, k, v, dtype, q_pos, k_pos, sel, blk, scale=None, q_blk0=0,
                      blocks=None, heads=None, batches=None):
    """Block-sparse prefill attention in slot order, fp64.

    q [B, Hq, Tq, d] holds query slots starting at block q_blk0; k, v [B, Hkv, T, d].
    q_pos [Tq_total] / k_pos [T] are the original positions of the slots (identity
    without permutation).  Query slot u of block i attends the slots v of the
    blocks in sel[b][i] with k_pos[v] <= q_pos[u] (causality on original
    positions, PBS-Attn §2).  Returns o [B, Hq, Tq, d], lse [B, Hq, Tq].
    """
    B, Hq, Tq, d = q.shape
    Hkv, T = k.shape[1], k.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    nQb = -(-Tq // blk)
    o = np.full((B, Hq, Tq, d), np.nan)
    lse = np.full((B, Hq, Tq), np.nan)
    for b in (range(B) if batches is None else batches):
        for i in (range(nQb) if blocks is None else blocks):
            kslots = np.array([t for j in sel[b][i] for t in range(j * blk, min((j + 1) * blk, T))], dtype=np.int64)
            for h in (range(Hq) if heads is None else heads):
                g = h // G
                K = to_f64(k[b, g, kslots], dtype)
                V = to_f64(v[b, g, kslots], dtype)
                for u in range(i * blk, min((i + 1) * blk, Tq)):
                    pos_u = q_pos[(q_blk0 * blk) + u]
                    keep = k_pos[kslots] <= pos_u
                    o[b, h, u], lse[b, h, u] = softmax_attend(to_f64(q[b, h, u], dtype), K[keep], V[keep], scale)
    return o, lse


# --------------------------------------------------------------------------
# segment permutation
# --------------------------------------------------------------------------

def check_segment_perm(perm: np.ndarray, seg: int) -> bool:
    """True if perm is a permutation that maps each segment of length seg onto itself."""
    T = len(perm)
    if sorted(perm.tolist()) != list(range(T)):
        return False
    return bool(np.all(np.asarray(perm) // seg == np.arange(T) // seg))


def key_importance(q, k, dtype, seq_len, proxy, scale=None) -> np.ndarray:
    """Global key importance from a proxy query block (PBS-Attn §3), fp64.

    q [B, Hq, T, d], k [B, Hkv, T, d]; query head h reads KV head h // (Hq/Hkv).
    Readings: the proxy queries are the last min(proxy, L) tokens before
    L = seq_len[b], every query head included; each attends causally (keys at
    positions <= its own) with the softmax of q.k * scale; the importance of key
    t is the mean of its probability over all (head, proxy query) rows, so the
    importances of a sequence sum to 1.  Keys at or past L get 0.
    Returns imp [B, T].
    """
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    imp = np.zeros((B, T))
    for b in range(B):
        L = int(seq_len[b])
        n = min(proxy, L)
        u0 = L - n
        # causal mask of the proxy rows: row i (position u0 + i) sees keys 0 .. u0 + i
        visible = np.arange(L)[None, :] <= (u0 + np.arange(n))[:, None]
        for h in range(Hq):
            x = (to_f64(q[b, h, u0:L], dtype) @ to_f64(k[b, h // G, :L], dtype).T) * scale
            x = np.where(visible, x, -np.inf)
            e = np.exp(x - x.max(axis=1, keepdims=True))
            imp[b, :L] += (e / e.sum(axis=1, keepdims=True)).sum(axis=0)
        imp[b] /= Hq * n
    return imp


def importance_permutation(imp: np.ndarray, seq_len, seg: int) -> np.ndarray:
    """Segment-wise key order by descending importance (PBS-Attn §3, inside §2's segments).

    perm[b, s*seg + r] is the key at rank r of segment s: the keys below
    seq_len[b] ordered by importance descending, ties to the lower position;
    keys at or past seq_len[b] follow in their own order.  Returns [B, T] int64.
    """
    B, T = imp.shape
    perm = np.empty((B, T), dtype=np.int64)
    for b in range(B):
        L = int(seq_len[b])
        for s0 in range(0, T, seg):
            keys = range(s0, min(s0 + seg, T))
            valid = sorted((t for t in keys if t < L), key=lambda t: (-imp[b, t], t))
            tail = [t for t in keys if t >= L]
            perm[b, s0:s0 + len(keys)] = valid + tail
    return perm


def segment_permute(x: np.ndarray, perm: np.ndarray, axis: int, inverse: bool = False) -> np.ndarray:
    """Forward: dst[t] = src[perm[t]].  Inverse: dst[perm[t]] = src[t].  Along ``axis``."""
    x = np.asarray(x)
    if not inverse:
        return np.take(x, perm, axis=axis)
    out = np.empty_like(x)
    idx = [slice(None)] * x.ndim
    idx[axis] = perm
    out[tuple(idx)] = x
    return out


# --------------------------------------------------------------------------
# whole-path drivers
# --------------------------------------------------------------------------

def decode_step(inp: Dict, batches=None, heads=None) -> Dict:
    """Score -> select -> sparse attention for one decode step of a workload dict.

    With an int4 selector cache (cfg.selector_q4) the scores use the
    dequantised int4 keys in place of the int8 ones.
    """
    cfg = inp["cfg"]
    if getattr(cfg, "selector_q4", False):
        inp = dict(inp, kI=dequantize_selector_keys(*quantize_selector_keys(inp["kI"])))
    if getattr(cfg, "per_group", False):
        s = score_decode_grouped(inp["qI"], inp["kI"], inp["w"], inp["seq_len"], cfg.blk, cfg.Hkv)
        if cfg.select == "topk":
            sel, info = select_decode_grouped(s, inp["seq_len"], cfg.blk, cfg.n_sink, cfg.n_local, "topk", k=cfg.k)
        else:
            sel, info = select_decode_grouped(s, inp["seq_len"], cfg.blk, cfg.n_sink, cfg.n_local, "topp",
                                              beta=cfg.beta, p=cfg.p, k_min=cfg.k_min, k_max=cfg.k_max)
        o, lse = decode_attention(inp["q"], inp["k"], inp["v"], cfg.dtype, inp["seq_len"], sel, cfg.blk,
                                  inp["head_mode"], cfg.local_sink_tok, cfg.local_window_tok,
                                  batches=batches, heads=heads, per_group=True)
        return dict(scores=s, sel=sel, info=info, o=o, lse=lse)
    s = score_decode(inp["qI"], inp["kI"], inp["w"], inp["seq_len"], cfg.blk)
    if cfg.select == "topk":
        sel, info = select_decode(s, inp["seq_len"], cfg.blk, cfg.n_sink, cfg.n_local, "topk", k=cfg.k)
    else:
        sel, info = select_decode(s, inp["seq_len"], cfg.blk, cfg.n_sink, cfg.n_local, "topp",
                                  beta=cfg.beta, p=cfg.p, k_min=cfg.k_min, k_max=cfg.k_max)
    o, lse = decode_attention(inp["q"], inp["k"], inp["v"], cfg.dtype, inp["seq_len"], sel, cfg.blk,
                              inp["head_mode"], cfg.local_sink_tok, cfg.local_window_tok,
                              batches=batches, heads=heads)
    return dict(scores=s, sel=sel, info=info, o=o, lse=lse)


def prefill_front(inp: Dict) -> Dict:
    """Permute -> pool -> score -> select for the permuted block-sparse prefill."""
    cfg = inp["cfg"]
    perm = inp["perm"]
    assert check_segment_perm(perm, cfg.seg)
    qI_p = segment_permute(inp["qI_tok"], perm, axis=1)
    kI_p = segment_permute(inp["kI_tok"], perm, axis=1)
    qIb = pool_blocks(qI_p, cfg.blk)
    kIb = pool_blocks(kI_p, cfg.blk)
    s = score_prefill(qIb, kIb, inp["w"])
    sel = select_prefill_topk(s, cfg.n_sink, cfg.n_local, cfg.k)
    return dict(qIb=qIb, kIb=kIb, scores=s, sel=sel, pos=perm.astype(np.int64))


def prefill_step(inp: Dict, front: Dict = None, blocks=None, heads=None) -> Dict:
    """Full permuted prefill: front end, attention in slot order, inverse permutation of O.

    With ``blocks``/``heads`` only those slot blocks are computed and the
    slot-order output is returned without the inverse permutation.
    """
    cfg = inp["cfg"]
    front = front or prefill_front(inp)
    perm = inp["perm"]
    qp = segment_permute(inp["q"], perm, axis=2)
    kp = segment_permute(inp["k"], perm, axis=2)
    vp = segment_permute(inp["v"], perm, axis=2)
    o_slot, lse_slot = prefill_attention(qp, kp, vp, cfg.dtype, front["pos"], front["pos"], front["sel"],
                                         cfg.blk, blocks=blocks, heads=heads)
    res = dict(front, o_slot=o_slot, lse_slot=lse_slot)
    if blocks is None and heads is None:
        res["o"] = segment_permute(o_slot, perm, axis=2, inverse=True)
        res["lse"] = segment_permute(lse_slot, perm, axis=2, inverse=True)
    return res


# --------------------------------------------------------------------------
# diagnostics (density and attention mass, cf. RTPurbo "Resultados Clave")
# --------------------------------------------------------------------------

def prefill_block_mass(qp, kp, dtype, q_pos, k_pos, blk, q_blocks, scale=None) -> np.ndarray:
    """Dense causal attention mass per key block, for chosen query blocks (slot order), fp64.

    qp [Hq, T, d], kp [Hkv, T, d] of one sequence in slot order; q_pos / k_pos
    the original positions.  For query block i, mass[i, j] is the share of the
    softmax mass (causal on original positions) that the block's queries put on
    key block j, averaged over its queries and the query heads.  Used to count
    the blocks a query block needs for a given coverage (PBS-Attn "Resultados
    Clave": fewer selected blocks at equal attention coverage).
    """
    Hq, T, d = qp.shape
    G = Hq // kp.shape[0]
    nb = -(-T // blk)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((len(q_blocks), nb))
    blk_of = np.arange(T) // blk
    for n, i in enumerate(q_blocks):
        rows = np.arange(i * blk, min((i + 1) * blk, T))
        visible = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[rows][:, None]
        for h in range(Hq):
            x = np.where(visible, (to_f64(qp[h, rows], dtype) @ to_f64(kp[h // G], dtype).T) * scale, -np.inf)
            e = np.exp(x - x.max(axis=1, keepdims=True))
            p = (e / e.sum(axis=1, keepdims=True)).sum(axis=0)
            out[n] += np.bincount(blk_of, weights=p, minlength=nb)
        out[n] /= Hq * len(rows)
    return out


def blocks_for_coverage(mass_row: np.ndarray, coverage: float) -> int:
    """Fewest key blocks whose mass reaches ``coverage`` (largest blocks first)."""
    c = np.cumsum(np.sort(np.asarray(mass_row))[::-1])
    return int(np.searchsorted(c, coverage * c[-1] * (1 - 1e-12)) + 1)


def dense_mass(q, k, dtype, seq_len, tokens, heads=None, scale=None) -> np.ndarray:
    """Share of each head's dense softmax mass (over [0, seq_len)) that falls on ``tokens``.

    q [Hq, d], k [Hkv, T, d] for one sequence; returns [len(heads)] float64.
    """
    Hq, d = q.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    L = int(seq_len)
    out = []
    for h in (range(Hq) if heads is None else heads):
        K = to_f64(k[h // G, :L], dtype)
        x = (K @ to_f64(q[h], dtype)) * scale
        e = np.exp(x - x.max())
        out.append(e[np.asarray(tokens, dtype=np.int64)].sum() / e.sum())
    return np.array(out)
