"""bench.py's contract and the algorithmic counts its rooflines divide by, checked on the host
against hand counts of tiny cases (no GPU): the decode attention's HBM bytes, the scoring and
selection bytes, the attended (query, key) pairs of a permuted prefill, and the refusal of more
than one GPU.
"""
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _cfg(**kw):
    base = dict(dtype="bf16", d=4, blk=8, B=2, Hkv=2, Hq=4, local_sink_tok=0, local_window_tok=0, r=16, H_idx=2,
                selector_q4=False)
    base.update(kw)
    return SimpleNamespace(**base)


def test_decode_attn_bytes_hand_count():
    # sequence 0 (20 tokens) selects blocks 0 and 2: 8 + 4 tokens (block 2 is clipped at the end);
    # sequence 1 (9 tokens) selects block 1: 1 token.  Two KV groups read them each, K and V rows of
    # d = 4 bf16 (8 bytes): (12 + 12 + 1 + 1) * 2 * 8 = 416 bytes.  Q 2*4*4*2 = 64, O (fp32)
    # 2*4*4*4 = 128, lse 2*4*4 = 32, lists 3 entries + 2 counts + 2 lengths = 28 bytes.
    cfg = _cfg()
    idx = np.array([[0, 2, -1], [1, -1, -1]], dtype=np.int32)
    counts = np.array([2, 1], dtype=np.int32)
    seq_len = np.array([20, 9])
    assert bench.decode_attn_bytes(cfg, idx, counts, seq_len, [0, 0]) == 416 + 64 + 128 + 32 + 28
    # group 0 local (2 sink tokens + a 4-token window = 6 tokens of each sequence), group 1 retrieval:
    # (6 + 12 + 6 + 1) rows * 16 bytes = 400
    cfg = _cfg(local_sink_tok=2, local_window_tok=4)
    assert bench.decode_attn_bytes(cfg, idx, counts, seq_len, [1, 0]) == 400 + 64 + 128 + 32 + 28
    # fp32 inputs double the K, V and Q bytes
    cfg = _cfg(dtype="f32")
    assert bench.decode_attn_bytes(cfg, idx, counts, seq_len, [0, 0]) == 832 + 128 + 128 + 32 + 28


def test_decode_attn_bytes_per_group_lists():
    # one list per (sequence, KV group): group 0 of sequence 0 takes block 0, group 1 blocks 0 and 1
    cfg = _cfg(B=1)
    idx = np.array([[[0, -1], [0, 1]]], dtype=np.int32)
    counts = np.array([[1, 2]], dtype=np.int32)
    kv = (8 + 16) * 2 * 8
    assert bench.decode_attn_bytes(cfg, idx, counts, np.array([16]), [0, 0]) == kv + 32 + 64 + 16 + (3 + 2 + 1) * 4


def test_decode_index_bytes_hand_count():
    # 3 + 2 valid blocks, 2 indexer heads of 16 int8 values; qI (16) and w (1) per head and sequence;
    # one length per sequence
    cfg = _cfg()
    assert bench.decode_index_bytes(cfg, [20, 9]) == 5 * 2 * 16 + 2 * 2 * 17 + 2 * 4
    # int4 cache: 8 bytes of codes and one exponent byte per key vector
    cfg = _cfg(selector_q4=True)
    assert bench.decode_index_bytes(cfg, [20, 9]) == 5 * 2 * 9 + 2 * 2 * 17 + 2 * 4


def test_prefill_pairs_hand_count():
    # two 4-token blocks, segments of 4: slots hold original positions 3 1 2 0 | 7 5 4 6
    perm = np.array([3, 1, 2, 0, 7, 5, 4, 6])
    # every causal block selected: all T (T + 1) / 2 = 36 pairs
    idx = np.array([[0, -1], [0, 1]], dtype=np.int32)
    assert bench.prefill_pairs(perm, idx, np.array([1, 2]), 4) == 36
    # query block 1 attends block 1 only: positions 7, 5, 4, 6 see 4, 2, 1 and 3 keys at or below them
    idx = np.array([[0, -1], [1, -1]], dtype=np.int32)
    assert bench.prefill_pairs(perm, idx, np.array([1, 1]), 4) == 10 + 10


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
