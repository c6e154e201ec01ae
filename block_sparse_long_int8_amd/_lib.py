"""ctypes binding of libspa.so: argument marshalling only.

Every function here has the name of the C entry point it calls (include/spa.h)
and does nothing but check shapes, allocate outputs with torch (device memory
plumbing), pass raw pointers and torch's current HIP stream, and raise on a
non-zero status.  All arithmetic runs in the library's HIP kernels.  If the
library is missing the import fails loudly: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
import re
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspa.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "spa.h")

SPA_OK = 0
SPA_ERR_INVALID_ARG = -1
SPA_ERR_UNSUPPORTED = -2
SPA_ERR_WORKSPACE = -3
SPA_ERR_HIP = -4
SPA_F32 = 0
SPA_BF16 = 1
SPA_SCORE_DECODE = 0
SPA_SCORE_PREFILL_POOLED = 1
SPA_SCORE_PREFILL_TOKENS = 2
SPA_SCORE_DECODE_GROUPED = 3
SPA_ORDER_SLOT = 0
SPA_ORDER_ORIGINAL = 1
SPA_ORDER_KV_ORIGINAL = 2
SPA_DBG_NONE = 0
SPA_DBG_SEQ_LEN = 1
SPA_DBG_COUNT = 2
SPA_DBG_IDX_RANGE = 3
SPA_DBG_IDX_ORDER = 4
SPA_DBG_HEAD_MODE = 5
SPA_DBG_Q_POS = 6
SPA_DBG_K_POS = 7
SPA_DBG_PERM_RANGE = 8
SPA_DBG_PERM_DUP = 9
SPA_DBG_TOK_POS = 10

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t
_i64 = ctypes.c_int64

_SIGS = {
    "spa_status_string": (ctypes.c_char_p, [_i]),
    "spa_last_error": (ctypes.c_char_p, []),
    "spa_version": (_i, []),
    "spa_set_debug_checks": (None, [_i]),
    "spa_debug_checks": (_i, []),
    "spa_debug_error": (_i, []),
    "spa_index_score": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _i, _i, _vp, _vp, _sz, _vp]),
    "spa_index_score_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "spa_select_topk": (_i, [_vp, _i, _i, _i, _i, _vp, _i, _i, _i, _i, _i, _vp, _vp, _i, _vp, _sz, _vp]),
    "spa_select_topp": (_i, [_vp, _i, _i, _i, _i, _vp, _i, _i, _i, _i, _f, _f, _i, _i, _vp, _vp, _i, _vp, _sz, _vp]),
    "spa_select_topk_hist": (_i, [_vp, _i, _i, _i, _i, _vp, _i, _i, _i, _i, _i, _vp, _vp, _i, _vp, _sz, _vp]),
    "spa_select_topp_hist": (_i, [_vp, _i, _i, _i, _i, _vp, _i, _i, _i, _i, _f, _f, _i, _i, _vp, _vp, _i, _vp, _sz,
                                  _vp]),
    "spa_score_select_decode": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _i, _i, _i, _i, _i, _f, _f, _i, _i, _vp,
                                     _vp, _vp, _i, _vp]),
    "spa_sparse_decode_attn": (_i, [_vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _vp, _i, _i, _i, _i, _i, _i, _i, _f,
                                    _vp, _i, _vp, _vp, _sz, _vp]),
    "spa_sparse_decode_attn_grouped": (_i, [_vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _vp, _i, _i, _i, _i, _i, _i, _i,
                                            _f, _vp, _i, _vp, _vp, _sz, _vp]),
    "spa_sparse_decode_attn_workspace_size": (_sz, [_i, _i, _i, _i]),
    "spa_block_sparse_prefill": (_i, [_vp, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f,
                                      _vp, _i, _vp, _i, _vp, _sz, _vp]),
    "spa_segment_permute": (_i, [_vp, _vp, _i64, _i, _sz, _vp, _i, _i, _vp]),
    "spa_quantize_selector_keys": (_i, [_vp, _i64, _i, _vp, _vp, _vp]),
    "spa_index_score_q4": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _i, _i, _vp, _vp]),
    "spa_importance_permutation": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _vp, _i, _f, _i, _vp, _vp, _vp, _sz, _vp]),
    "spa_importance_permutation_workspace_size": (_sz, [_i, _i, _i]),
}

_lib: Optional[ctypes.CDLL] = None


class SpaError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} -> {status} ({detail})")
        self.status = status
        self.detail = detail


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with block_sparse_long_int8_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def declared_symbols():
    """Function names declared in include/spa.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:spa_status|size_t|const char\*|int|void)\s+(spa_\w+)\s*\(", text, re.M)))


def spa_set_debug_checks(on: bool) -> None:
    """Switch the library's device-side checks of index arrays on or off (process-wide)."""
    lib().spa_set_debug_checks(int(bool(on)))


def spa_debug_checks() -> bool:
    return bool(lib().spa_debug_checks())


def spa_debug_error() -> int:
    """SPA_DBG_* code of the last device-side check violation on this thread (SPA_DBG_NONE if none)."""
    return int(lib().spa_debug_error())


def _check(fn: str, status: int):
    if status != SPA_OK:
        raise SpaError(fn, status, lib().spa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _io_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SPA_BF16
    if t.dtype == torch.float32:
        return SPA_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


# ------------------------------------------------------------------ scores --

def spa_index_score_workspace_size(B, H_idx, r, Mq, nKb, mode) -> int:
    return int(lib().spa_index_score_workspace_size(B, H_idx, r, Mq, nKb, mode))


def spa_index_score(qI, kI, w, blk, seq_len=None, mode=SPA_SCORE_DECODE, q_blk0=0, nKb=None, Mq=None,
                    scores=None, ws=None, tok_pos=None) -> torch.Tensor:
    """Block scores (int32).  Layouts as in include/spa.h; returns scores.

    For SPA_SCORE_DECODE_GROUPED, ``Mq`` is the number of groups (required).  With ``tok_pos``
    (SPA_SCORE_PREFILL_TOKENS only) qI and kI hold every token in original order and slot t
    pools row tok_pos[b, t]; Mq defaults to the blocks from q_blk0 to the end.
    """
    _dev(qI, "qI", torch.int8)
    _dev(kI, "kI", torch.int8)
    _dev(w, "w", torch.int8)
    if mode == SPA_SCORE_DECODE:
        B, H, r = qI.shape
        nKb = kI.shape[1]
        Mq = 1
        shape = (B, nKb)
    elif mode == SPA_SCORE_DECODE_GROUPED:
        B, H, r = qI.shape
        nKb = kI.shape[1]
        if Mq is None:
            raise ValueError("grouped decode scoring needs Mq (the number of groups)")
        shape = (B, Mq, nKb)
    else:
        B, _, H, r = qI.shape
        if mode == SPA_SCORE_PREFILL_POOLED:
            Mq = qI.shape[1] if Mq is None else Mq
            nKb = kI.shape[1] if nKb is None else nKb
        else:
            # per-token vectors: whole blocks only (the pooling kernel reads Mq*blk / nKb*blk tokens)
            if qI.shape[1] % blk or kI.shape[1] % blk:
                raise ValueError("per-token indexer inputs must hold a whole number of blocks")
            nKb = kI.shape[1] // blk if nKb is None else nKb
            if Mq is None:
                Mq = nKb - q_blk0 if tok_pos is not None else qI.shape[1] // blk
            q_rows = nKb * blk if tok_pos is not None else Mq * blk
            if q_rows > qI.shape[1] or nKb * blk > kI.shape[1]:
                raise ValueError("Mq/nKb exceed the per-token inputs")
            if tok_pos is not None:
                _dev(tok_pos, "tok_pos", torch.int32)
                if tok_pos.numel() != B * nKb * blk:
                    raise ValueError(f"tok_pos must hold B*nKb*blk = {B * nKb * blk} positions")
        shape = (B, Mq, nKb)
    if seq_len is not None:
        _dev(seq_len, "seq_len", torch.int32)
    if scores is None:
        scores = torch.empty(shape, dtype=torch.int32, device=qI.device)
    need = spa_index_score_workspace_size(B, H, r, Mq, nKb, mode)
    if need and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=qI.device)
    st = lib().spa_index_score(_ptr(qI), _ptr(kI), _ptr(w), B, H, r, Mq, nKb, q_blk0, _ptr(seq_len), _ptr(tok_pos),
                               blk, mode, _ptr(scores), _ptr(ws), 0 if ws is None else ws.numel(), _stream())
    _check("spa_index_score", st)
    return scores


def spa_quantize_selector_keys(kI, codes=None, exps=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """int8 key vectors [..., 16] -> int4 codes [..., 8] uint8 and exponents [...] uint8."""
    _dev(kI, "kI", torch.int8)
    r = kI.shape[-1]
    lead = tuple(kI.shape[:-1])
    if codes is None:
        codes = torch.empty(lead + (r // 2,), dtype=torch.uint8, device=kI.device)
    if exps is None:
        exps = torch.empty(lead, dtype=torch.uint8, device=kI.device)
    st = lib().spa_quantize_selector_keys(_ptr(kI), math.prod(lead), r, _ptr(codes), _ptr(exps), _stream())
    _check("spa_quantize_selector_keys", st)
    return codes, exps


def spa_index_score_q4(qI, codes, exps, w, blk, seq_len, mode=SPA_SCORE_DECODE, Mq=None, scores=None) -> torch.Tensor:
    """Decode scores from the int4 selector cache; Mq is the number of groups in grouped mode."""
    _dev(qI, "qI", torch.int8)
    _dev(codes, "codes", torch.uint8)
    _dev(exps, "exps", torch.uint8)
    _dev(w, "w", torch.int8)
    _dev(seq_len, "seq_len", torch.int32)
    B, H, r = qI.shape
    nKb = codes.shape[1]
    if codes.shape != (B, nKb, H, r // 2) or exps.shape != (B, nKb, H):
        raise ValueError("codes must be [B, nKb, H_idx, r/2] and exps [B, nKb, H_idx]")
    Mq = 1 if mode == SPA_SCORE_DECODE else Mq
    if Mq is None:
        raise ValueError("grouped decode scoring needs Mq (the number of groups)")
    if scores is None:
        scores = torch.empty((B, nKb) if mode == SPA_SCORE_DECODE else (B, Mq, nKb), dtype=torch.int32,
                             device=qI.device)
    st = lib().spa_index_score_q4(_ptr(qI), _ptr(codes), _ptr(exps), _ptr(w), B, H, r, Mq, nKb, _ptr(seq_len), blk,
                                  mode, _ptr(scores), _stream())
    _check("spa_index_score_q4", st)
    return scores


# --------------------------------------------------------------- selection --

def _sel_out(scores, cap, idx, count):
    B = scores.shape[0]
    M = 1 if scores.dim() == 2 else scores.shape[1]
    if idx is None:
        idx = torch.empty((B, M, cap) if scores.dim() == 3 else (B, cap), dtype=torch.int32, device=scores.device)
    if count is None:
        count = torch.empty((B, M) if scores.dim() == 3 else (B,), dtype=torch.int32, device=scores.device)
    return B, M, idx, count


def spa_select_topk(scores, blk, n_sink, n_local, k, cap, seq_len=None, prefill=False, q_blk0=0,
                    idx=None, count=None, algo="sort") -> Tuple[torch.Tensor, torch.Tensor]:
    """algo "sort" calls spa_select_topk, "hist" spa_select_topk_hist (same result)."""
    _dev(scores, "scores", torch.int32)
    B, M, idx, count = _sel_out(scores, cap, idx, count)
    nKb = scores.shape[-1]
    name = _sel_name("spa_select_topk", algo)
    st = getattr(lib(), name)(_ptr(scores), B, M, nKb, q_blk0, _ptr(seq_len), blk, n_sink, n_local, int(prefill),
                              k, _ptr(idx), _ptr(count), cap, None, 0, _stream())
    _check(name, st)
    return idx, count


def _sel_name(base, algo):
    if algo not in ("sort", "hist"):
        raise ValueError(f"algo must be 'sort' or 'hist', not {algo!r}")
    return base if algo == "sort" else base + "_hist"


def spa_select_topp(scores, blk, n_sink, n_local, beta, p, k_min, k_max, cap, seq_len=None, prefill=False,
                    q_blk0=0, idx=None, count=None, algo="sort") -> Tuple[torch.Tensor, torch.Tensor]:
    """algo "sort" calls spa_select_topp, "hist" spa_select_topp_hist."""
    _dev(scores, "scores", torch.int32)
    B, M, idx, count = _sel_out(scores, cap, idx, count)
    nKb = scores.shape[-1]
    name = _sel_name("spa_select_topp", algo)
    st = getattr(lib(), name)(_ptr(scores), B, M, nKb, q_blk0, _ptr(seq_len), blk, n_sink, n_local, int(prefill),
                              float(beta), float(p), k_min, k_max, _ptr(idx), _ptr(count), cap, None, 0, _stream())
    _check(name, st)
    return idx, count


def spa_score_select_decode(qI, kI, w, seq_len, blk, n_sink, n_local, cap, mode="topp", k=0, beta=1.0, p=0.9,
                            k_min=0, k_max=0, scores_out=None, idx=None, count=None):
    """Fused decode scoring + selection; returns (idx, count)."""
    _dev(qI, "qI", torch.int8)
    _dev(kI, "kI", torch.int8)
    _dev(w, "w", torch.int8)
    _dev(seq_len, "seq_len", torch.int32)
    B, H, r = qI.shape
    nKb = kI.shape[1]
    if idx is None:
        idx = torch.empty((B, cap), dtype=torch.int32, device=qI.device)
    if count is None:
        count = torch.empty((B,), dtype=torch.int32, device=qI.device)
    st = lib().spa_score_select_decode(_ptr(qI), _ptr(kI), _ptr(w), B, H, r, nKb, _ptr(seq_len), blk, n_sink,
                                       n_local, 0 if mode == "topk" else 1, k, float(beta), float(p), k_min, k_max,
                                       _ptr(scores_out), _ptr(idx), _ptr(count), cap, _stream())
    _check("spa_score_select_decode", st)
    return idx, count


# ---------------------------------------------------------- decode attention --

def spa_sparse_decode_attn_workspace_size(B, Hq, Hkv, d) -> int:
    return int(lib().spa_sparse_decode_attn_workspace_size(B, Hq, Hkv, d))


def spa_sparse_decode_attn(q, k_cache, v_cache, seq_len, idx, count, blk, head_mode=None, local_sink_tok=0,
                           local_window_tok=0, scale=None, out_dtype=torch.float32, out=None, lse=None, ws=None,
                           want_lse=True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """One block list per sequence: idx [B, cap], count [B]."""
    return _decode_attn("spa_sparse_decode_attn", q, k_cache, v_cache, seq_len, idx, count, blk, head_mode,
                        local_sink_tok, local_window_tok, scale, out_dtype, out, lse, ws, want_lse)


def spa_sparse_decode_attn_grouped(q, k_cache, v_cache, seq_len, idx, count, blk, head_mode=None,
                                   local_sink_tok=0, local_window_tok=0, scale=None, out_dtype=torch.float32,
                                   out=None, lse=None, ws=None,
                                   want_lse=True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """One block list per (sequence, KV head): idx [B, Hkv, cap], count [B, Hkv]."""
    return _decode_attn("spa_sparse_decode_attn_grouped", q, k_cache, v_cache, seq_len, idx, count, blk,
                        head_mode, local_sink_tok, local_window_tok, scale, out_dtype, out, lse, ws, want_lse)


def _decode_attn(name, q, k_cache, v_cache, seq_len, idx, count, blk, head_mode, local_sink_tok, local_window_tok,
                 scale, out_dtype, out, lse, ws, want_lse):
    _dev(q, "q")
    _dev(k_cache, "k_cache", q.dtype)
    _dev(v_cache, "v_cache", q.dtype)
    _dev(seq_len, "seq_len", torch.int32)
    _dev(idx, "idx", torch.int32)
    _dev(count, "count", torch.int32)
    B, Hq, d = q.shape
    _, Hkv, Tcap, _ = k_cache.shape
    cap = idx.shape[-1]
    rows = B * Hkv if name.endswith("_grouped") else B
    if idx.numel() != rows * cap or count.numel() != rows:
        raise ValueError(f"{name}: idx must hold {rows} lists of {cap} and count {rows} entries")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = torch.empty(max(1, spa_sparse_decode_attn_workspace_size(B, Hq, Hkv, d)), dtype=torch.uint8,
                         device=q.device)
    if head_mode is not None:
        _dev(head_mode, "head_mode", torch.uint8)
    st = getattr(lib(), name)(_ptr(q), _ptr(k_cache), _ptr(v_cache), _io_dtype(q), _ptr(seq_len), _ptr(idx),
                              _ptr(count), cap, blk, _ptr(head_mode), local_sink_tok, local_window_tok, B, Hq, Hkv, d,
                              Tcap, float(scale), _ptr(out), _io_dtype(out), _ptr(lse), _ptr(ws), ws.numel(),
                              _stream())
    _check(name, st)
    return out, lse


# ----------------------------------------------------------------- prefill --

def spa_block_sparse_prefill(q, k, v, idx, count, blk, q_pos=None, k_pos=None, q_blk0=0, scale=None,
                             out_dtype=torch.float32, out=None, lse=None, want_lse=True, order="slot",
                             Tq=None, kv_order="slot") -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``order="slot"``: q, out [B, Hq, Tq, d] hold the chunk's slots.  ``order="original"``:
    q, out [B, Hq, T, d] (and lse [B, Hq, T]) in original token order, rows q_pos[b, slot];
    Tq (the chunk length) defaults to T - q_blk0*blk.  ``kv_order="original"``: k, v in
    original order (slot t is row k_pos[b, t])."""
    if kv_order not in ("slot", "original"):
        raise ValueError(f"kv_order must be 'slot' or 'original', not {kv_order!r}")
    _dev(q, "q", torch.bfloat16)
    _dev(k, "k", torch.bfloat16)
    _dev(v, "v", torch.bfloat16)
    _dev(idx, "idx", torch.int32)
    _dev(count, "count", torch.int32)
    if order not in ("slot", "original"):
        raise ValueError(f"order must be 'slot' or 'original', not {order!r}")
    B, Hq, Tr, d = q.shape
    _, Hkv, T, _ = k.shape
    if order == "slot":
        Tq = Tr if Tq is None else Tq
        if Tq != Tr:
            raise ValueError("in slot order q holds exactly the chunk's Tq rows")
    else:
        if Tr != T:
            raise ValueError("in original order q holds the whole sequence (T rows)")
        Tq = T - q_blk0 * blk if Tq is None else Tq
    cap = idx.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, Tr, d), dtype=out_dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Tr), dtype=torch.float32, device=q.device)
    st = lib().spa_block_sparse_prefill(_ptr(q), q_blk0, Tq, _ptr(k), _ptr(v), _ptr(q_pos), _ptr(k_pos), _ptr(idx),
                                        _ptr(count), cap, blk, B, Hq, Hkv, d, T, float(scale), _ptr(out),
                                        _io_dtype(out), _ptr(lse),
                                        (SPA_ORDER_ORIGINAL if order == "original" else SPA_ORDER_SLOT)
                                        | (SPA_ORDER_KV_ORIGINAL if kv_order == "original" else 0), None, 0,
                                        _stream())
    _check("spa_block_sparse_prefill", st)
    return out, lse


# ------------------------------------------------------------- permutation --

def spa_segment_permute(src, perm, seg, dim, inverse=False, dst=None) -> torch.Tensor:
    """Permute ``src`` along ``dim`` (dst[t] = src[perm[t]], or the inverse)."""
    _dev(src, "src")
    _dev(perm, "perm", torch.int32)
    if dst is None:
        dst = torch.empty_like(src)
    outer = math.prod(src.shape[:dim])
    T = src.shape[dim]
    row_bytes = math.prod(src.shape[dim + 1:]) * src.element_size()
    st = lib().spa_segment_permute(_ptr(src), _ptr(dst), outer, T, row_bytes, _ptr(perm), seg, int(inverse),
                                   _stream())
    _check("spa_segment_permute", st)
    return dst


# ------------------------------------------------------ importance permutation --

def spa_importance_permutation_workspace_size(B, Hq, T) -> int:
    return int(lib().spa_importance_permutation_workspace_size(B, Hq, T))


def spa_importance_permutation(q, k, seg, proxy=64, seq_len=None, scale=None, imp=None, perm=None,
                               ws=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Importance of every key from the last ``proxy`` queries and the segment-wise
    descending-importance permutation; q [B, Hq, T, d], k [B, Hkv, T, d] bf16.
    Returns (imp [B, T] fp32, perm [B, T] int32)."""
    _dev(q, "q", torch.bfloat16)
    _dev(k, "k", torch.bfloat16)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, T, d):
        raise ValueError("k must be [B, Hkv, T, d] with q's B, T and d")
    if seq_len is not None:
        _dev(seq_len, "seq_len", torch.int32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if imp is None:
        imp = torch.empty((B, T), dtype=torch.float32, device=q.device)
    if perm is None:
        perm = torch.empty((B, T), dtype=torch.int32, device=q.device)
    if ws is None:
        ws = torch.empty(max(1, spa_importance_permutation_workspace_size(B, Hq, T)), dtype=torch.uint8,
                         device=q.device)
    st = lib().spa_importance_permutation(_ptr(q), _ptr(k), B, Hq, Hkv, T, d, _ptr(seq_len), proxy, float(scale), seg,
                                          _ptr(imp), _ptr(perm), _ptr(ws), ws.numel(), _stream())
    _check("spa_importance_permutation", st)
    return imp, perm
