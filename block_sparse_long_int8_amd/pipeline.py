"""The two hot paths as sequences of library calls, with buffers preallocated.

DecodeStep:  spa_index_score -> spa_select_topk | spa_select_topp (or both in
             one launch: spa_score_select_decode) -> spa_sparse_decode_attn
PrefillStep: [spa_importance_permutation, or the caller's permutation]
             -> per chunk of query blocks:
                spa_index_score (per-token vectors in original order, pooled per
                block of the permuted order by gathering through the slot
                positions) -> spa_select_topk (prefill rows)
                -> spa_block_sparse_prefill (Q, K, V read and O, lse written at
                   each slot's original position, so nothing is copied into the
                   permuted order and nothing is inverse-permuted)

Only marshalling lives here; every step runs in the HIP library.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib as L


@dataclass
class DecodeSpec:
    B: int
    Hq: int
    Hkv: int
    d: int
    Tcap: int
    blk: int
    H_idx: int
    r: int
    n_sink: int
    n_local: int
    select: str = "topk"          # "topk" | "topp"
    k: int = 0
    beta: float = 1.0
    p: float = 0.9
    k_min: int = 0
    k_max: int = 0
    local_sink_tok: int = 0
    local_window_tok: int = 0
    out_dtype: torch.dtype = torch.float32
    select_algo: str = "sort"     # "sort" (bitonic) | "hist" (radix threshold, no sort)
    per_group: bool = False       # one selection per KV head from its own H_idx/Hkv indexer heads
    selector_q4: bool = False     # selector keys held as int4 codes + exponents (a (codes, exps) pair for kI)

    @property
    def nb(self) -> int:
        return -(-self.Tcap // self.blk)

    @property
    def cap(self) -> int:
        budget = self.k if self.select == "topk" else self.k_max
        return max(1, min(self.nb, self.n_sink + self.n_local + budget))


class DecodeStep:
    """One decode step of one attention layer; owns its scratch and output buffers.

    ``fused=False`` (default) runs spa_index_score (wide, all CUs) then
    spa_select_* (one workgroup per sequence); ``fused=True`` scores and
    selects in one launch (spa_score_select_decode), which saves a launch but
    reads the indexer keys with only one workgroup per sequence.  Replayed as a
    HIP graph (``capture``), where launches cost nothing, the separate pair is
    the faster of the two.

    With ``spec.per_group`` every KV head selects its own blocks: grouped
    scores [B, Hkv, nKb], Hkv selection rows per sequence and
    spa_sparse_decode_attn_grouped (separate launches only).
    """

    def __init__(self, spec: DecodeSpec, device="cuda", fused: bool = False):
        self.spec = s = spec
        if fused and (s.per_group or s.selector_q4):
            raise ValueError("the fused score+select launch has no per-group or int4 mode")
        self.fused = fused
        dev = torch.device(device)
        rows = (s.B, s.Hkv) if s.per_group else (s.B,)
        self.scores = torch.empty(rows + (s.nb,), dtype=torch.int32, device=dev)
        self.idx = torch.empty(rows + (s.cap,), dtype=torch.int32, device=dev)
        self.count = torch.empty(rows, dtype=torch.int32, device=dev)
        self.out = torch.empty((s.B, s.Hq, s.d), dtype=s.out_dtype, device=dev)
        self.lse = torch.empty((s.B, s.Hq), dtype=torch.float32, device=dev)
        n = L.spa_sparse_decode_attn_workspace_size(s.B, s.Hq, s.Hkv, s.d)
        self.ws = torch.empty(max(1, n), dtype=torch.uint8, device=dev)

    @staticmethod
    def quantize_selector(kI):
        """int8 selector keys [B, nKb, H_idx, 16] -> the int4 cache (codes, exps) that ``kI`` takes with selector_q4."""
        return L.spa_quantize_selector_keys(kI)

    def score(self, qI, kI, w, seq_len):
        s = self.spec
        if s.selector_q4:
            codes, exps = kI
            mode = L.SPA_SCORE_DECODE_GROUPED if s.per_group else L.SPA_SCORE_DECODE
            return L.spa_index_score_q4(qI, codes, exps, w, s.blk, seq_len, mode=mode, Mq=s.Hkv if s.per_group else 1,
                                        scores=self.scores)
        if s.per_group:
            return L.spa_index_score(qI, kI, w, s.blk, seq_len=seq_len, mode=L.SPA_SCORE_DECODE_GROUPED, Mq=s.Hkv,
                                     scores=self.scores)
        return L.spa_index_score(qI, kI, w, s.blk, seq_len=seq_len, mode=L.SPA_SCORE_DECODE, scores=self.scores)

    def select(self, seq_len):
        s = self.spec
        if s.select == "topk":
            return L.spa_select_topk(self.scores, s.blk, s.n_sink, s.n_local, s.k, s.cap, seq_len=seq_len,
                                     idx=self.idx, count=self.count, algo=s.select_algo)
        return L.spa_select_topp(self.scores, s.blk, s.n_sink, s.n_local, s.beta, s.p, s.k_min, s.k_max, s.cap,
                                 seq_len=seq_len, idx=self.idx, count=self.count, algo=s.select_algo)

    def score_select(self, qI, kI, w, seq_len, keep_scores: bool = False):
        """Fused scoring + selection (scores are written only if keep_scores)."""
        s = self.spec
        return L.spa_score_select_decode(qI, kI, w, seq_len, s.blk, s.n_sink, s.n_local, s.cap, mode=s.select,
                                         k=s.k, beta=s.beta, p=s.p, k_min=s.k_min, k_max=s.k_max,
                                         scores_out=self.scores if keep_scores else None, idx=self.idx,
                                         count=self.count)

    def attend(self, q, k_cache, v_cache, seq_len, head_mode=None):
        s = self.spec
        fn = L.spa_sparse_decode_attn_grouped if s.per_group else L.spa_sparse_decode_attn
        return fn(q, k_cache, v_cache, seq_len, self.idx, self.count, s.blk,
                  head_mode=head_mode, local_sink_tok=s.local_sink_tok, local_window_tok=s.local_window_tok,
                  out=self.out, lse=self.lse, ws=self.ws)

    def __call__(self, q, k_cache, v_cache, qI, kI, w, seq_len, head_mode=None, keep_scores: bool = False):
        if self.fused:
            self.score_select(qI, kI, w, seq_len, keep_scores=keep_scores)
        else:
            self.score(qI, kI, w, seq_len)
            self.select(seq_len)
        return self.attend(q, k_cache, v_cache, seq_len, head_mode)

    def capture(self, q, k_cache, v_cache, qI, kI, w, seq_len, head_mode=None) -> "torch.cuda.CUDAGraph":
        """Record one whole step on these tensors as a HIP graph (replay with ``graph.replay()``).

        Every launch of the step goes into the graph; none of them allocates,
        clears memory or synchronises, so the graph holds kernel nodes only.
        The graph reads and writes the tensors it was recorded with.
        """
        return self.capture_steps([(q, k_cache, v_cache, qI, kI, w, seq_len, head_mode)])

    def capture_steps(self, steps) -> "torch.cuda.CUDAGraph":
        """Record several consecutive steps (one argument tuple each, in order) as one HIP graph."""
        for a in steps:
            self(*a)  # settle lazy state outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for a in steps:
                self(*a)
        return g


@dataclass
class PrefillSpec:
    B: int
    T: int
    Hq: int
    Hkv: int
    d: int
    blk: int
    H_idx: int
    r: int
    k: int
    n_sink: int
    n_local: int
    seg: int
    out_dtype: torch.dtype = torch.float32
    select_algo: str = "sort"     # "sort" (bitonic) | "hist" (radix threshold, no sort)
    perm_kind: str = "given"      # "given" (the caller's permutation) | "importance" (computed per call)
    proxy: int = 64               # proxy queries of the importance permutation
    chunk: int = 0                # query tokens per chunk (0: one chunk covering T); a multiple of seg

    @property
    def nb(self) -> int:
        return -(-self.T // self.blk)

    @property
    def cap(self) -> int:
        return max(1, min(self.nb, self.n_sink + self.n_local + 1 + self.k))

    @property
    def chunk_blocks(self) -> int:
        """Query blocks per chunk."""
        return self.nb if self.chunk <= 0 else min(self.nb, self.chunk // self.blk)


class PrefillStep:
    """Permuted block-sparse prefill of one attention layer, in chunks of query blocks.

    The permutation is the caller's (``perm`` [T], shared by the batch, or
    [B, T]) or, with ``spec.perm_kind == "importance"``, computed on the device
    from Q and K by spa_importance_permutation (one per sequence).  Nothing is
    copied into slot order: the pooling of the indexer vectors gathers each
    block's tokens through the slot positions, and the attention reads Q, K
    and V and writes O (``out``) and the log-sum-exp (``lse``) in the original
    token order through the same positions.

    With ``spec.chunk`` the query blocks run in chunks of that many tokens
    (chunked prefill): each chunk scores its rows against the key blocks before
    them, selects and attends.  A chunk is a whole number of permutation
    segments, so no segment straddles two chunks, and the results are the
    one-shot results bit for bit.
    """

    def __init__(self, spec: PrefillSpec, device="cuda"):
        self.spec = s = spec
        if s.chunk < 0 or (s.chunk and (s.chunk % s.seg or s.chunk % s.blk)):
            raise ValueError(f"chunk ({s.chunk}) must be a whole number of segments ({s.seg}) and blocks ({s.blk})")
        dev = torch.device(device)
        cb = s.chunk_blocks
        self.chunks = [(a0, min(cb, s.nb - a0)) for a0 in range(0, s.nb, cb)]
        # per chunk: scores [B, m, nb], block lists [B, m, cap], counts [B, m]
        self._scores = [torch.empty((s.B, m, s.nb), dtype=torch.int32, device=dev) for _, m in self.chunks]
        self._idx = [torch.empty((s.B, m, s.cap), dtype=torch.int32, device=dev) for _, m in self.chunks]
        self._count = [torch.empty((s.B, m), dtype=torch.int32, device=dev) for _, m in self.chunks]
        n = max(L.spa_index_score_workspace_size(s.B, s.H_idx, s.r, m, s.nb, L.SPA_SCORE_PREFILL_TOKENS)
                for _, m in self.chunks)
        self.score_ws = torch.empty(max(1, n), dtype=torch.uint8, device=dev)
        self.out = torch.empty((s.B, s.Hq, s.T, s.d), dtype=s.out_dtype, device=dev)
        self.lse = torch.empty((s.B, s.Hq, s.T), dtype=torch.float32, device=dev)
        self.pos = None
        if s.perm_kind == "importance":
            self.imp = torch.empty((s.B, s.T), dtype=torch.float32, device=dev)
            self.perm = torch.empty((s.B, s.T), dtype=torch.int32, device=dev)
            n = L.spa_importance_permutation_workspace_size(s.B, s.Hq, s.T)
            self.imp_ws = torch.empty(max(1, n), dtype=torch.uint8, device=dev)
        elif s.perm_kind != "given":
            raise ValueError(f"perm_kind must be 'given' or 'importance', not {s.perm_kind!r}")

    @staticmethod
    def _rows(parts):
        return parts[0] if len(parts) == 1 else torch.cat(parts, dim=1)

    @property
    def scores(self) -> torch.Tensor:
        """Block-pair scores of every query block, [B, nb, nb] (a copy when chunked)."""
        return self._rows(self._scores)

    @property
    def idx(self) -> torch.Tensor:
        """Selected key blocks of every query block, [B, nb, cap] (a copy when chunked)."""
        return self._rows(self._idx)

    @property
    def count(self) -> torch.Tensor:
        """Number of selected key blocks of every query block, [B, nb] (a copy when chunked)."""
        return self._rows(self._count)

    def importance(self, q, k):
        """Importance-sorted segment permutation of each sequence (PBS-Attn §3) into self.perm."""
        s = self.spec
        L.spa_importance_permutation(q, k, s.seg, proxy=s.proxy, imp=self.imp, perm=self.perm, ws=self.imp_ws)
        return self.perm

    def set_perm(self, perm):
        """Positions of the permuted slots (the causal mask uses original positions)."""
        s = self.spec
        if perm.dim() == 2:
            self.pos = perm
        else:
            self.pos = perm.reshape(1, -1) if s.B == 1 else perm.reshape(1, -1).expand(s.B, -1).contiguous()
        return self.pos

    @staticmethod
    def _w_rows(w, a0, m):
        ws = w[:, a0:a0 + m]
        return ws if ws.is_contiguous() else ws.contiguous()

    def score(self, qI_tok, kI_tok, w, c=None):
        """Pool the per-token vectors (original order) into the blocks of the permuted order, gathered
        through the slot positions, and score each query block of chunk ``c`` (every chunk if None)
        against the key blocks before it."""
        s = self.spec
        for ci in (range(len(self.chunks)) if c is None else (c,)):
            a0, m = self.chunks[ci]
            L.spa_index_score(qI_tok, kI_tok, self._w_rows(w, a0, m), s.blk, mode=L.SPA_SCORE_PREFILL_TOKENS,
                              q_blk0=a0, Mq=m, nKb=s.nb, scores=self._scores[ci], ws=self.score_ws, tok_pos=self.pos)
        return self._scores[0] if len(self.chunks) == 1 else None

    def select(self, c=None):
        s = self.spec
        for ci in (range(len(self.chunks)) if c is None else (c,)):
            a0, _ = self.chunks[ci]
            L.spa_select_topk(self._scores[ci], s.blk, s.n_sink, s.n_local, s.k, s.cap, prefill=True, q_blk0=a0,
                              idx=self._idx[ci], count=self._count[ci], algo=s.select_algo)
        return (self._idx[0], self._count[0]) if len(self.chunks) == 1 else None

    def front(self, qI_tok, kI_tok, w):
        """Pool and score the indexer inputs in the permuted order, then select (after set_perm)."""
        self.score(qI_tok, kI_tok, w)
        self.select()

    def attend(self, q, k, v, c=None):
        """Attention of every query of chunk ``c`` (every chunk if None) over its block's selected key
        blocks (q, k, v and out in original order)."""
        s = self.spec
        for ci in (range(len(self.chunks)) if c is None else (c,)):
            a0, m = self.chunks[ci]
            Tq = min(m * s.blk, s.T - a0 * s.blk)
            L.spa_block_sparse_prefill(q, k, v, self._idx[ci], self._count[ci], s.blk, q_pos=self.pos,
                                       k_pos=self.pos, q_blk0=a0, Tq=Tq, out=self.out, lse=self.lse,
                                       order="original", kv_order="original")
        return self.out, self.lse

    def __call__(self, q, k, v, qI_tok, kI_tok, w, perm=None):
        if self.spec.perm_kind == "importance":
            perm = self.importance(q, k)
        self.set_perm(perm)
        for ci in range(len(self.chunks)):
            self.score(qI_tok, kI_tok, w, ci)
            self.select(ci)
            self.attend(q, k, v, ci)
        return self.out

    def capture(self, q, k, v, qI_tok, kI_tok, w, perm=None) -> "torch.cuda.CUDAGraph":
        """Record one whole prefill step (every chunk) on these tensors as a HIP graph.

        Replay with ``graph.replay()``: the launches of a chunked step then go
        out without a host round trip per call.  The graph reads and writes the
        tensors it was recorded with (a positions tensor that ``set_perm`` had
        to expand is recorded too).
        """
        self(q, k, v, qI_tok, kI_tok, w, perm)  # settle lazy state outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self(q, k, v, qI_tok, kI_tok, w, perm)
        return g
