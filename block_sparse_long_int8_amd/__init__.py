"""Block-sparse long-context attention with an int8 indexer, for MI355X (gfx950).

The library (libspa.so, HIP kernels behind a C ABI declared in include/spa.h)
does all the work; this package is its thin ctypes binding plus the two hot
paths wired as sequences of calls.  The same library carries two rate probes
of the device (include/spa_probe.h) that the measurements compare against.
"""
from ._lib import (SPA_BF16, SPA_ERR_HIP, SPA_ERR_INVALID_ARG, SPA_ERR_UNSUPPORTED, SPA_ERR_WORKSPACE, SPA_F32,
                   SPA_OK, SPA_SCORE_DECODE, SPA_SCORE_PREFILL_POOLED, SPA_SCORE_PREFILL_TOKENS, SPA_SCORE_DECODE_GROUPED,
                   SPA_ORDER_KV_ORIGINAL, SPA_ORDER_ORIGINAL, SPA_ORDER_SLOT,
                   SPA_DBG_NONE, SPA_DBG_SEQ_LEN, SPA_DBG_COUNT, SPA_DBG_IDX_RANGE, SPA_DBG_IDX_ORDER, SPA_DBG_HEAD_MODE,
                   SPA_DBG_Q_POS, SPA_DBG_K_POS, SPA_DBG_PERM_RANGE, SPA_DBG_PERM_DUP, SPA_DBG_TOK_POS,
                   spa_set_debug_checks, spa_debug_checks, spa_debug_error,
                   LIB_PATH,
                   SpaError, declared_symbols, lib, spa_block_sparse_prefill, spa_index_score,
                   spa_index_score_workspace_size, spa_score_select_decode, spa_segment_permute, spa_select_topk,
                   spa_select_topp,
                   spa_sparse_decode_attn, spa_sparse_decode_attn_grouped, spa_sparse_decode_attn_workspace_size,
                   spa_sparse_decode_attn_noalloc,
                   spa_importance_permutation, spa_importance_permutation_workspace_size, spa_quantize_selector_keys,
                   spa_index_score_q4, spa_probe_read, spa_probe_mfma_bf16, PROBE_MFMA_FLOPS_PER_WAVE_ROUND)
from .pipeline import DecodeSpec, DecodeStep, PrefillSpec, PrefillStep

__all__ = [n for n in dir() if not n.startswith("_")]
