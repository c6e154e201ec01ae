"""ctypes binding of libspa.so: argument marshalling only.

Every function here has the name of the C entry point it calls (include/spa.h)
and does nothing but check each tensor argument against the layout the entry
point reads (exact shape, dtype, contiguity, one device; ValueError before any
launch), allocate outputs with torch (device memory plumbing), pass raw
pointers and torch's current HIP stream, and raise on a non-zero status.  All
arithmetic runs in the library's HIP kernels.  If the library is missing the
import fails loudly: there is no fallback path.
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
INCLUDE = os.path.join(os.path.dirname(_PKG), "include")
HEADER = os.path.join(INCLUDE, "spa.h")

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
    "spa_sparse_decode_attn_noalloc": (_i, [_vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _vp, _i, _i, _i, _i, _i, _i, _i,
                                            _f, _vp, _i, _vp, _vp]),
    "spa_block_sparse_prefill": (_i, [_vp, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f,
                                      _vp, _i, _vp, _i, _vp, _sz, _vp]),
    "spa_segment_permute": (_i, [_vp, _vp, _i64, _i, _sz, _vp, _i, _i, _vp]),
    "spa_quantize_selector_keys": (_i, [_vp, _i64, _i, _vp, _vp, _vp]),
    "spa_index_score_q4": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _i, _i, _vp, _vp]),
    "spa_importance_permutation": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _vp, _i, _f, _i, _vp, _vp, _vp, _sz, _vp]),
    "spa_importance_permutation_workspace_size": (_sz, [_i, _i, _i]),
    "spa_probe_read": (_i, [_vp, _sz, _i, _vp, _vp]),
    "spa_probe_mfma_bf16": (_i, [_i, _i, _vp, _vp]),
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
    """Function names declared in the headers under include/ (spa.h, spa_probe.h)."""
    text = ""
    for name in sorted(os.listdir(INCLUDE)):
        if name.endswith(".h"):
            with open(os.path.join(INCLUDE, name)) as f:
                text += f.read()
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


def _want(t: Optional[torch.Tensor], name: str, shape=None, dtype=None, optional: bool = False):
    """Check one tensor argument against the layout the C entry point reads: exact
    shape, dtype and contiguity.  Raises ValueError (nothing is launched)."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(int(x) for x in shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _on_device(**tensors):
    """Every given tensor lives on the same GPU (checked after the shapes)."""
    devs = set()
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        devs.add(t.device)
    if len(devs) > 1:
        raise ValueError(f"tensors on different devices: {sorted(str(d) for d in devs)}")


def _ws(ws: Optional[torch.Tensor], need: int, name: str = "ws"):
    """A caller workspace must be a contiguous uint8 tensor of at least ``need`` bytes."""
    if ws is None:
        return None
    _want(ws, name, dtype=torch.uint8)
    if ws.numel() < need:
        raise ValueError(f"{name} holds {ws.numel()} bytes, the call needs {need}")
    return ws


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
    for name, t in (("qI", qI), ("kI", kI), ("w", w)):
        _want(t, name, dtype=torch.int8)
    if mode in (SPA_SCORE_DECODE, SPA_SCORE_DECODE_GROUPED):
        if qI.dim() != 3:
            raise ValueError("decode scoring: qI must be [B, H_idx, r]")
        B, H, r = qI.shape
        nKb = kI.shape[1] if nKb is None else nKb
        if mode == SPA_SCORE_DECODE:
            Mq = 1
            shape = (B, nKb)
        else:
            if Mq is None:
                raise ValueError("grouped decode scoring needs Mq (the number of groups)")
            shape = (B, Mq, nKb)
        _want(kI, "kI", (B, nKb, H, r))
        _want(w, "w", (B, H))
        _want(seq_len, "seq_len", (B,), torch.int32)
        if tok_pos is not None:
            raise ValueError("tok_pos is only for SPA_SCORE_PREFILL_TOKENS")
    elif mode in (SPA_SCORE_PREFILL_POOLED, SPA_SCORE_PREFILL_TOKENS):
        if qI.dim() != 4:
            raise ValueError("prefill scoring: qI must be [B, rows, H_idx, r]")
        B, _, H, r = qI.shape
        if mode == SPA_SCORE_PREFILL_POOLED:
            Mq = qI.shape[1] if Mq is None else Mq
            nKb = kI.shape[1] if nKb is None else nKb
            _want(qI, "qI", (B, Mq, H, r))
            _want(kI, "kI", (B, nKb, H, r))
            if tok_pos is not None:
                raise ValueError("tok_pos is only for SPA_SCORE_PREFILL_TOKENS")
        else:
            # per-token vectors: whole blocks only (the pooling kernel reads Mq*blk / nKb*blk tokens)
            if qI.shape[1] % blk or kI.shape[1] % blk:
                raise ValueError("per-token indexer inputs must hold a whole number of blocks")
            nKb = kI.shape[1] // blk if nKb is None else nKb
            if Mq is None:
                Mq = nKb - q_blk0 if tok_pos is not None else qI.shape[1] // blk
            q_rows = nKb * blk if tok_pos is not None else Mq * blk
            _want(qI, "qI", (B, q_rows, H, r))
            _want(kI, "kI", (B, nKb * blk, H, r))
            _want(tok_pos, "tok_pos", (B, nKb * blk), torch.int32, optional=True)
        _want(w, "w", (B, Mq, H))
        _want(seq_len, "seq_len", (B,), torch.int32, optional=True)
        shape = (B, Mq, nKb)
    else:
        raise ValueError(f"unknown scoring mode {mode}")
    _want(scores, "scores", shape, torch.int32, optional=True)
    need = spa_index_score_workspace_size(B, H, r, Mq, nKb, mode)
    _ws(ws, need)
    _on_device(qI=qI, kI=kI, w=w, seq_len=seq_len, tok_pos=tok_pos, scores=scores, ws=ws)
    if scores is None:
        scores = torch.empty(shape, dtype=torch.int32, device=qI.device)
    if need and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=qI.device)
    st = lib().spa_index_score(_ptr(qI), _ptr(kI), _ptr(w), B, H, r, Mq, nKb, q_blk0, _ptr(seq_len), _ptr(tok_pos),
                               blk, mode, _ptr(scores), _ptr(ws), 0 if ws is None else ws.numel(), _stream())
    _check("spa_index_score", st)
    return scores


def spa_quantize_selector_keys(kI, codes=None, exps=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """int8 key vectors [..., 16] -> int4 codes [..., 8] uint8 and exponents [...] uint8."""
    _want(kI, "kI", dtype=torch.int8)
    r = kI.shape[-1]
    lead = tuple(kI.shape[:-1])
    _want(codes, "codes", lead + (r // 2,), torch.uint8, optional=True)
    _want(exps, "exps", lead, torch.uint8, optional=True)
    _on_device(kI=kI, codes=codes, exps=exps)
    if codes is None:
        codes = torch.empty(lead + (r // 2,), dtype=torch.uint8, device=kI.device)
    if exps is None:
        exps = torch.empty(lead, dtype=torch.uint8, device=kI.device)
    st = lib().spa_quantize_selector_keys(_ptr(kI), math.prod(lead), r, _ptr(codes), _ptr(exps), _stream())
    _check("spa_quantize_selector_keys", st)
    return codes, exps


def spa_index_score_q4(qI, codes, exps, w, blk, seq_len, mode=SPA_SCORE_DECODE, Mq=None, scores=None) -> torch.Tensor:
    """Decode scores from the int4 selector cache; Mq is the number of groups in grouped mode."""
    _want(qI, "qI", dtype=torch.int8)
    if qI.dim() != 3:
        raise ValueError("qI must be [B, H_idx, r]")
    B, H, r = qI.shape
    _want(codes, "codes", dtype=torch.uint8)
    nKb = codes.shape[1] if codes.dim() == 4 else -1
    if codes.shape != (B, nKb, H, r // 2) or tuple(exps.shape) != (B, nKb, H):
        raise ValueError("codes must be [B, nKb, H_idx, r/2] and exps [B, nKb, H_idx]")
    _want(exps, "exps", (B, nKb, H), torch.uint8)
    _want(w, "w", (B, H), torch.int8)
    _want(seq_len, "seq_len", (B,), torch.int32)
    Mq = 1 if mode == SPA_SCORE_DECODE else Mq
    if Mq is None:
        raise ValueError("grouped decode scoring needs Mq (the number of groups)")
    shape = (B, nKb) if mode == SPA_SCORE_DECODE else (B, Mq, nKb)
    _want(scores, "scores", shape, torch.int32, optional=True)
    _on_device(qI=qI, codes=codes, exps=exps, w=w, seq_len=seq_len, scores=scores)
    if scores is None:
        scores = torch.empty(shape, dtype=torch.int32, device=qI.device)
    st = lib().spa_index_score_q4(_ptr(qI), _ptr(codes), _ptr(exps), _ptr(w), B, H, r, Mq, nKb, _ptr(seq_len), blk,
                                  mode, _ptr(scores), _stream())
    _check("spa_index_score_q4", st)
    return scores


# --------------------------------------------------------------- selection --

def _sel_out(scores, cap, idx, count, seq_len, prefill):
    """Check the selection tensors (scores [B, nKb] or [B, M, nKb]; idx, count to match) and
    allocate the missing outputs."""
    _want(scores, "scores", dtype=torch.int32)
    if scores.dim() not in (2, 3):
        raise ValueError("scores must be [B, nKb] or [B, M, nKb]")
    B = scores.shape[0]
    M = 1 if scores.dim() == 2 else scores.shape[1]
    rows = (B,) if scores.dim() == 2 else (B, M)
    _want(idx, "idx", rows + (cap,), torch.int32, optional=True)
    _want(count, "count", rows, torch.int32, optional=True)
    _want(seq_len, "seq_len", (B,), torch.int32, optional=prefill)
    _on_device(scores=scores, idx=idx, count=count, seq_len=seq_len)
    if idx is None:
        idx = torch.empty(rows + (cap,), dtype=torch.int32, device=scores.device)
    if count is None:
        count = torch.empty(rows, dtype=torch.int32, device=scores.device)
    return B, M, idx, count


def spa_select_topk(scores, blk, n_sink, n_local, k, cap, seq_len=None, prefill=False, q_blk0=0,
                    idx=None, count=None, algo="sort") -> Tuple[torch.Tensor, torch.Tensor]:
    """algo "sort" calls spa_select_topk, "hist" spa_select_topk_hist (same result)."""
    name = _sel_name("spa_select_topk", algo)
    B, M, idx, count = _sel_out(scores, cap, idx, count, seq_len, prefill)
    nKb = scores.shape[-1]
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
    name = _sel_name("spa_select_topp", algo)
    B, M, idx, count = _sel_out(scores, cap, idx, count, seq_len, prefill)
    nKb = scores.shape[-1]
    st = getattr(lib(), name)(_ptr(scores), B, M, nKb, q_blk0, _ptr(seq_len), blk, n_sink, n_local, int(prefill),
                              float(beta), float(p), k_min, k_max, _ptr(idx), _ptr(count), cap, None, 0, _stream())
    _check(name, st)
    return idx, count


def spa_score_select_decode(qI, kI, w, seq_len, blk, n_sink, n_local, cap, mode="topp", k=0, beta=1.0, p=0.9,
                            k_min=0, k_max=0, scores_out=None, idx=None, count=None):
    """Fused decode scoring + selection; returns (idx, count)."""
    if mode not in ("topk", "topp"):
        raise ValueError(f"mode must be 'topk' or 'topp', not {mode!r}")
    _want(qI, "qI", dtype=torch.int8)
    if qI.dim() != 3:
        raise ValueError("qI must be [B, H_idx, r]")
    B, H, r = qI.shape
    nKb = kI.shape[1] if kI.dim() == 4 else -1
    _want(kI, "kI", (B, nKb, H, r), torch.int8)
    _want(w, "w", (B, H), torch.int8)
    _want(seq_len, "seq_len", (B,), torch.int32)
    _want(scores_out, "scores_out", (B, nKb), torch.int32, optional=True)
    _want(idx, "idx", (B, cap), torch.int32, optional=True)
    _want(count, "count", (B,), torch.int32, optional=True)
    _on_device(qI=qI, kI=kI, w=w, seq_len=seq_len, scores_out=scores_out, idx=idx, count=count)
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


def spa_sparse_decode_attn_noalloc(q, k_cache, v_cache, seq_len, idx, count, blk, head_mode=None, local_sink_tok=0,
                                   local_window_tok=0, scale=None, out_dtype=torch.float32, out=None, lse=None,
                                   want_lse=True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """spa_sparse_decode_attn on the library's own workspace (no workspace argument; the library
    allocates nothing).  Pass ``out`` (and ``lse``) to keep torch from allocating them."""
    return _decode_attn("spa_sparse_decode_attn_noalloc", q, k_cache, v_cache, seq_len, idx, count, blk, head_mode,
                        local_sink_tok, local_window_tok, scale, out_dtype, out, lse, None, want_lse)


def _decode_attn(name, q, k_cache, v_cache, seq_len, idx, count, blk, head_mode, local_sink_tok, local_window_tok,
                 scale, out_dtype, out, lse, ws, want_lse):
    _want(q, "q")
    if q.dim() != 3:
        raise ValueError(f"{name}: q must be [B, Hq, d]")
    io = _io_dtype(q)
    B, Hq, d = q.shape
    if k_cache.dim() != 4:
        raise ValueError(f"{name}: k_cache must be [B, Hkv, Tcap, d]")
    Hkv, Tcap = k_cache.shape[1], k_cache.shape[2]
    _want(k_cache, "k_cache", (B, Hkv, Tcap, d), q.dtype)
    _want(v_cache, "v_cache", (B, Hkv, Tcap, d), q.dtype)
    _want(seq_len, "seq_len", (B,), torch.int32)
    rows = (B, Hkv) if name.endswith("_grouped") else (B,)
    cap = idx.shape[-1]
    _want(idx, "idx", rows + (cap,), torch.int32)
    _want(count, "count", rows, torch.int32)
    _want(head_mode, "head_mode", (Hkv,), torch.uint8, optional=True)
    if out is not None:
        out_dtype = out.dtype
    _io_dtype(torch.empty(0, dtype=out_dtype))
    _want(out, "out", (B, Hq, d), out_dtype, optional=True)
    _want(lse, "lse", (B, Hq), torch.float32, optional=True)
    noalloc = name.endswith("_noalloc")
    need = spa_sparse_decode_attn_workspace_size(B, Hq, Hkv, d)
    _ws(ws, need)
    _on_device(q=q, k_cache=k_cache, v_cache=v_cache, seq_len=seq_len, idx=idx, count=count, head_mode=head_mode,
               out=out, lse=lse, ws=ws)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if ws is None and not noalloc:
        ws = torch.empty(max(1, need), dtype=torch.uint8, device=q.device)
    tail = () if noalloc else (_ptr(ws), ws.numel())
    st = getattr(lib(), name)(_ptr(q), _ptr(k_cache), _ptr(v_cache), io, _ptr(seq_len), _ptr(idx),
                              _ptr(count), cap, blk, _ptr(head_mode), local_sink_tok, local_window_tok, B, Hq, Hkv, d,
                              Tcap, float(scale), _ptr(out), _io_dtype(out), _ptr(lse), *tail, _stream())
    _check(name, st)
    return out, lse


# ----------------------------------------------------------------- prefill --

def spa_block_sparse_prefill(q, k, v, idx, count, blk, q_pos=None, k_pos=None, q_blk0=0, scale=None,
                             out_dtype=torch.float32, out=None, lse=None, want_lse=True, order="slot",
                             Tq=None, kv_order="slot") -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``order="slot"``: q, out [B, Hq, Tq, d] hold the chunk's slots.  ``order="original"``:
    q, out [B, Hq, T, d] (and lse [B, Hq, T]) in original token order, rows q_pos[b, slot];
    Tq (the chunk length) defaults to T - q_blk0*blk.  ``kv_order="original"``: k, v in
    original order (slot t is row k_pos[b, t]).  idx [B, ceil(Tq/blk), cap], count
    [B, ceil(Tq/blk)]; q_pos, k_pos [B, T] int32."""
    if kv_order not in ("slot", "original"):
        raise ValueError(f"kv_order must be 'slot' or 'original', not {kv_order!r}")
    if order not in ("slot", "original"):
        raise ValueError(f"order must be 'slot' or 'original', not {order!r}")
    _want(q, "q", dtype=torch.bfloat16)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, Hq, rows, d] and k, v [B, Hkv, T, d]")
    B, Hq, Tr, d = q.shape
    Hkv, T = k.shape[1], k.shape[2]
    _want(k, "k", (B, Hkv, T, d), torch.bfloat16)
    _want(v, "v", (B, Hkv, T, d), torch.bfloat16)
    if order == "slot":
        Tq = Tr if Tq is None else Tq
        if Tq != Tr:
            raise ValueError("in slot order q holds exactly the chunk's Tq rows")
    else:
        if Tr != T:
            raise ValueError("in original order q holds the whole sequence (T rows)")
        Tq = T - q_blk0 * blk if Tq is None else Tq
    if q_blk0 < 0 or Tq < 0 or q_blk0 * blk + Tq > T:
        raise ValueError(f"chunk [{q_blk0 * blk}, {q_blk0 * blk + Tq}) exceeds the {T} key slots")
    Mq = -(-Tq // blk)
    cap = idx.shape[-1]
    _want(idx, "idx", (B, Mq, cap), torch.int32)
    _want(count, "count", (B, Mq), torch.int32)
    _want(q_pos, "q_pos", (B, T), torch.int32, optional=order == "slot")
    _want(k_pos, "k_pos", (B, T), torch.int32, optional=kv_order == "slot")
    if out is not None:
        out_dtype = out.dtype
    _io_dtype(torch.empty(0, dtype=out_dtype))
    _want(out, "out", (B, Hq, Tr, d), out_dtype, optional=True)
    _want(lse, "lse", (B, Hq, Tr), torch.float32, optional=True)
    _on_device(q=q, k=k, v=v, idx=idx, count=count, q_pos=q_pos, k_pos=k_pos, out=out, lse=lse)
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
    """Permute ``src`` along ``dim`` (dst[t] = src[perm[t]], or the inverse); perm [T] int32."""
    _want(src, "src")
    T = src.shape[dim]
    _want(perm, "perm", (T,), torch.int32)
    _want(dst, "dst", tuple(src.shape), src.dtype, optional=True)
    _on_device(src=src, perm=perm, dst=dst)
    if dst is None:
        dst = torch.empty_like(src)
    outer = math.prod(src.shape[:dim])
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
    _want(q, "q", dtype=torch.bfloat16)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, Hq, T, d] and k [B, Hkv, T, d]")
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, T, d):
        raise ValueError("k must be [B, Hkv, T, d] with q's B, T and d")
    _want(k, "k", (B, Hkv, T, d), torch.bfloat16)
    _want(seq_len, "seq_len", (B,), torch.int32, optional=True)
    _want(imp, "imp", (B, T), torch.float32, optional=True)
    _want(perm, "perm", (B, T), torch.int32, optional=True)
    need = spa_importance_permutation_workspace_size(B, Hq, T)
    _ws(ws, need)
    _on_device(q=q, k=k, seq_len=seq_len, imp=imp, perm=perm, ws=ws)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if imp is None:
        imp = torch.empty((B, T), dtype=torch.float32, device=q.device)
    if perm is None:
        perm = torch.empty((B, T), dtype=torch.int32, device=q.device)
    if ws is None:
        ws = torch.empty(max(1, need), dtype=torch.uint8, device=q.device)
    st = lib().spa_importance_permutation(_ptr(q), _ptr(k), B, Hq, Hkv, T, d, _ptr(seq_len), proxy, float(scale), seg,
                                          _ptr(imp), _ptr(perm), _ptr(ws), ws.numel(), _stream())
    _check("spa_importance_permutation", st)
    return imp, perm


# ---- rate probes of the device (include/spa_probe.h) -------------------------

PROBE_MFMA_FLOPS_PER_WAVE_ROUND = 131072  # four 32x32x16 bf16 products


def spa_probe_read(buf: torch.Tensor, workgroups: int, sink: torch.Tensor) -> None:
    """Read all of buf (a contiguous device tensor, a multiple of 16 bytes) once; asynchronous."""
    _want(buf, "buf")
    _want(sink, "sink", (1,), torch.int32)
    _on_device(buf=buf, sink=sink)
    nbytes = buf.numel() * buf.element_size()
    _check("spa_probe_read", lib().spa_probe_read(_ptr(buf), nbytes, int(workgroups), _ptr(sink), _stream()))


def spa_probe_mfma_bf16(workgroups: int, iters: int, sink: torch.Tensor) -> int:
    """Run the bf16 MFMA loop; asynchronous.  Returns the flops the call performs."""
    _want(sink, "sink", (1,), torch.float32)
    _on_device(sink=sink)
    _check("spa_probe_mfma_bf16", lib().spa_probe_mfma_bf16(int(workgroups), int(iters), _ptr(sink), _stream()))
    return int(workgroups) * 4 * int(iters) * PROBE_MFMA_FLOPS_PER_WAVE_ROUND
