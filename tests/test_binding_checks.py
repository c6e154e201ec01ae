"""The Python binding refuses misshaped tensor arguments before anything is launched.

Every check runs on the host.  The tensors here live on the CPU: a correctly
shaped call gets past the layout checks and stops at the device check, and a
misshaped one must be refused by the layout check first, naming the argument.
No GPU needed (the library is loaded only for its workspace-size queries).
"""
import pytest
import torch

import block_sparse_long_int8_amd as S

i8, i32, u8, f32, bf16 = torch.int8, torch.int32, torch.uint8, torch.float32, torch.bfloat16


def z(*shape, dtype=i32):
    return torch.zeros(shape, dtype=dtype)


def refused(name, fn, *args, **kw):
    with pytest.raises(ValueError) as e:
        fn(*args, **kw)
    assert name in str(e.value), str(e.value)
    assert "device tensor" not in str(e.value), "the layout check let a misshaped argument through"


def reaches_device_check(fn, *args, **kw):
    with pytest.raises(ValueError) as e:
        fn(*args, **kw)
    assert "device tensor" in str(e.value), str(e.value)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    S.lib()


# -------------------------------------------------------------- prefill ----

def _prefill(B=2, Hq=4, Hkv=2, T=256, d=128, blk=64, cap=5):
    nb = T // blk
    return dict(q=z(B, Hq, T, d, dtype=bf16), k=z(B, Hkv, T, d, dtype=bf16), v=z(B, Hkv, T, d, dtype=bf16),
                idx=z(B, nb, cap), count=z(B, nb), pos=z(B, T)), blk


def test_prefill_positions_must_be_per_sequence():
    t, blk = _prefill()
    args = (t["q"], t["k"], t["v"], t["idx"], t["count"], blk)
    reaches_device_check(S.spa_block_sparse_prefill, *args, q_pos=t["pos"], k_pos=t["pos"], order="original",
                         kv_order="original")
    # a [T] permutation shared by the batch is the spa_segment_permute form, not this call's [B, T]
    refused("q_pos", S.spa_block_sparse_prefill, *args, q_pos=t["pos"][0], k_pos=t["pos"], order="original",
            kv_order="original")
    refused("k_pos", S.spa_block_sparse_prefill, *args, q_pos=t["pos"], k_pos=t["pos"][0], order="original",
            kv_order="original")
    refused("q_pos", S.spa_block_sparse_prefill, *args, k_pos=t["pos"], order="original", kv_order="original")
    refused("k_pos", S.spa_block_sparse_prefill, *args, q_pos=t["pos"], order="original", kv_order="original")


def test_prefill_lists_outputs_and_chunk():
    t, blk = _prefill()
    base = (t["q"], t["k"], t["v"])
    refused("idx", S.spa_block_sparse_prefill, *base, z(2, 3, 5), t["count"], blk)
    refused("count", S.spa_block_sparse_prefill, *base, t["idx"], z(2, 3), blk)
    refused("idx", S.spa_block_sparse_prefill, *base, t["idx"].to(torch.int64), t["count"], blk)
    refused("out", S.spa_block_sparse_prefill, *base, t["idx"], t["count"], blk, out=z(2, 4, 255, 128, dtype=f32))
    refused("lse", S.spa_block_sparse_prefill, *base, t["idx"], t["count"], blk, lse=z(2, 4, 256, dtype=f32)[:, :2])
    refused("v", S.spa_block_sparse_prefill, t["q"], t["k"], z(2, 2, 128, 128, dtype=bf16), t["idx"], t["count"], blk)
    # a chunk of two query blocks takes two list rows
    refused("idx", S.spa_block_sparse_prefill, t["q"], t["k"], t["v"], t["idx"], t["count"], blk, q_pos=t["pos"],
            k_pos=t["pos"], q_blk0=2, Tq=128, order="original", kv_order="original")
    reaches_device_check(S.spa_block_sparse_prefill, t["q"], t["k"], t["v"], z(2, 2, 5), z(2, 2), blk,
                         q_pos=t["pos"], k_pos=t["pos"], q_blk0=2, Tq=128, order="original", kv_order="original")
    with pytest.raises(ValueError, match="exceeds"):
        S.spa_block_sparse_prefill(t["q"], t["k"], t["v"], z(2, 2, 5), z(2, 2), blk, q_pos=t["pos"], k_pos=t["pos"],
                                   q_blk0=3, Tq=128, order="original", kv_order="original")


# --------------------------------------------------------------- decode ----

def _decode(B=2, Hq=8, Hkv=2, Tcap=512, d=128, cap=9):
    return dict(q=z(B, Hq, d, dtype=bf16), k=z(B, Hkv, Tcap, d, dtype=bf16), v=z(B, Hkv, Tcap, d, dtype=bf16),
                seq_len=z(B), idx=z(B, cap), count=z(B), gidx=z(B, Hkv, cap), gcount=z(B, Hkv))


def test_decode_attention_arguments():
    t = _decode()
    args = (t["q"], t["k"], t["v"], t["seq_len"], t["idx"], t["count"], 64)
    reaches_device_check(S.spa_sparse_decode_attn, *args)
    refused("seq_len", S.spa_sparse_decode_attn, t["q"], t["k"], t["v"], z(3), t["idx"], t["count"], 64)
    refused("count", S.spa_sparse_decode_attn, t["q"], t["k"], t["v"], t["seq_len"], t["idx"], z(3), 64)
    refused("idx", S.spa_sparse_decode_attn, t["q"], t["k"], t["v"], t["seq_len"], t["gidx"], t["count"], 64)
    refused("head_mode", S.spa_sparse_decode_attn, *args, head_mode=z(3, dtype=u8))
    refused("head_mode", S.spa_sparse_decode_attn, *args, head_mode=z(2, dtype=i32))
    refused("out", S.spa_sparse_decode_attn, *args, out=z(2, 8, 64, dtype=f32))
    refused("lse", S.spa_sparse_decode_attn, *args, lse=z(2, 4, dtype=f32))
    refused("k_cache", S.spa_sparse_decode_attn, t["q"], z(2, 2, 512, 128, dtype=f32), t["v"], t["seq_len"],
            t["idx"], t["count"], 64)
    refused("v_cache", S.spa_sparse_decode_attn, t["q"], t["k"], z(2, 2, 256, 128, dtype=bf16), t["seq_len"],
            t["idx"], t["count"], 64)
    refused("ws", S.spa_sparse_decode_attn, *args, ws=z(16, dtype=u8))
    # grouped lists are one per (sequence, KV head)
    reaches_device_check(S.spa_sparse_decode_attn_grouped, t["q"], t["k"], t["v"], t["seq_len"], t["gidx"],
                         t["gcount"], 64)
    refused("idx", S.spa_sparse_decode_attn_grouped, t["q"], t["k"], t["v"], t["seq_len"], t["idx"], t["gcount"], 64)
    refused("count", S.spa_sparse_decode_attn_grouped, t["q"], t["k"], t["v"], t["seq_len"], t["gidx"], t["count"],
            64)


def test_selection_arguments():
    scores = z(3, 100)
    reaches_device_check(S.spa_select_topk, scores, 64, 1, 4, 8, 13, seq_len=z(3))
    refused("seq_len", S.spa_select_topk, scores, 64, 1, 4, 8, 13)          # decode rows need seq_len
    refused("seq_len", S.spa_select_topk, scores, 64, 1, 4, 8, 13, seq_len=z(2))
    refused("idx", S.spa_select_topk, scores, 64, 1, 4, 8, 13, seq_len=z(3), idx=z(3, 12))
    refused("count", S.spa_select_topp, scores, 64, 1, 4, 0.1, 0.9, 4, 8, 13, seq_len=z(3), count=z(3, 1))
    refused("scores", S.spa_select_topk, z(3, 100, dtype=torch.int64), 64, 1, 4, 8, 13, seq_len=z(3))
    # per-group rows: idx [B, M, cap]; prefill rows need no seq_len
    reaches_device_check(S.spa_select_topk, z(2, 4, 50), 64, 1, 0, 8, 10, prefill=True)
    refused("idx", S.spa_select_topk, z(2, 4, 50), 64, 1, 0, 8, 10, prefill=True, idx=z(2, 10))


def test_scoring_arguments():
    B, H, r, nKb, blk = 2, 8, 16, 40, 64
    qI, kI, w, L = z(B, H, r, dtype=i8), z(B, nKb, H, r, dtype=i8), z(B, H, dtype=i8), z(B)
    reaches_device_check(S.spa_index_score, qI, kI, w, blk, seq_len=L)
    refused("seq_len", S.spa_index_score, qI, kI, w, blk)
    refused("w", S.spa_index_score, qI, kI, z(B, H + 1, dtype=i8), blk, seq_len=L)
    refused("kI", S.spa_index_score, qI, z(B, nKb, H, r + 4, dtype=i8), w, blk, seq_len=L)
    refused("scores", S.spa_index_score, qI, kI, w, blk, seq_len=L, scores=z(B, nKb - 1))
    refused("scores", S.spa_index_score, qI, kI, w, blk, seq_len=L, mode=S.SPA_SCORE_DECODE_GROUPED, Mq=4,
            scores=z(B, nKb))
    # prefill, per-token vectors in original order gathered through tok_pos [B, nKb*blk]
    T = 8 * blk
    x = z(B, T, H, r, dtype=i8)
    wp = z(B, 8, H, dtype=i8)
    reaches_device_check(S.spa_index_score, x, x, wp, blk, mode=S.SPA_SCORE_PREFILL_TOKENS, tok_pos=z(B, T))
    refused("tok_pos", S.spa_index_score, x, x, wp, blk, mode=S.SPA_SCORE_PREFILL_TOKENS, tok_pos=z(T))
    refused("w", S.spa_index_score, x, x, z(B, 7, H, dtype=i8), blk, mode=S.SPA_SCORE_PREFILL_TOKENS,
            tok_pos=z(B, T))
    reaches_device_check(S.spa_index_score, x, x, z(B, 3, H, dtype=i8), blk, mode=S.SPA_SCORE_PREFILL_TOKENS,
                         tok_pos=z(B, T), q_blk0=5, Mq=3)
    refused("ws", S.spa_index_score, x, x, wp, blk, mode=S.SPA_SCORE_PREFILL_TOKENS, tok_pos=z(B, T),
            ws=z(1, dtype=u8))


def test_int4_and_permutation_arguments():
    B, nKb, H = 2, 30, 8
    reaches_device_check(S.spa_index_score_q4, z(B, H, 16, dtype=i8), z(B, nKb, H, 8, dtype=u8),
                         z(B, nKb, H, dtype=u8), z(B, H, dtype=i8), 64, z(B))
    refused("seq_len", S.spa_index_score_q4, z(B, H, 16, dtype=i8), z(B, nKb, H, 8, dtype=u8),
            z(B, nKb, H, dtype=u8), z(B, H, dtype=i8), 64, z(B + 1))
    refused("codes", S.spa_quantize_selector_keys, z(B, nKb, H, 16, dtype=i8), codes=z(B, nKb, H, 16, dtype=u8))
    src = z(3, 100, 16, dtype=i8)
    reaches_device_check(S.spa_segment_permute, src, z(100), 50, dim=1)
    refused("perm", S.spa_segment_permute, src, z(2, 100), 50, dim=1)
    refused("perm", S.spa_segment_permute, src, z(99), 50, dim=1)
    refused("dst", S.spa_segment_permute, src, z(100), 50, dim=1, dst=z(3, 100, 8, dtype=i8))
    q, k = z(1, 4, 128, 128, dtype=bf16), z(1, 2, 128, 128, dtype=bf16)
    reaches_device_check(S.spa_importance_permutation, q, k, 64)
    refused("perm", S.spa_importance_permutation, q, k, 64, perm=z(128))
    refused("seq_len", S.spa_importance_permutation, q, k, 64, seq_len=z(2))


def test_prefill_step_chunks():
    import dataclasses
    spec = S.PrefillSpec(B=1, T=8192, Hq=2, Hkv=1, d=128, blk=64, H_idx=8, r=16, k=32, n_sink=1, n_local=0,
                         seg=1024, chunk=2048)
    st = S.PrefillStep(spec, device="cpu")
    assert st.chunks == [(0, 32), (32, 32), (64, 32), (96, 32)]
    assert tuple(st.idx.shape) == (1, 128, spec.cap) and tuple(st.scores.shape) == (1, 128, 128)
    assert S.PrefillStep(dataclasses.replace(spec, chunk=0), device="cpu").chunks == [(0, 128)]
    with pytest.raises(ValueError, match="segments"):
        S.PrefillStep(dataclasses.replace(spec, chunk=1536), device="cpu")   # half a segment per chunk
