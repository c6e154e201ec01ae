"""Pins for the CPU oracle: hand-worked fixtures, closed forms, invariants,
library special cases and brute force on tiny inputs.  No GPU needed.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O
from gen import f32_to_bf16_bits

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- scores ----

def test_score_golden():
    g = gold("score_tiny.json")
    qI = np.array(g["qI"], dtype=np.int8)[None]
    kI = np.array(g["kI"], dtype=np.int8)[None]
    w = np.array(g["w"], dtype=np.int8)[None]
    s = O.score_decode(qI, kI, w, np.array([g["seq_len"]]), g["blk"])
    assert s[0].tolist() == g["expected"]
    s = O.score_decode(qI, kI, w, np.array([g["seq_len_ragged"]]), g["blk"])
    assert s[0].tolist() == g["expected_ragged"]


def _rand_idx(rng, B, nb, H, r, lo=-8, hi=7):
    qI = rng.integers(lo, hi + 1, size=(B, H, r), dtype=np.int8)
    kI = rng.integers(lo, hi + 1, size=(B, nb, H, r), dtype=np.int8)
    w = rng.integers(1, 5, size=(B, H), dtype=np.int8)
    return qI, kI, w


def test_score_copy_closed_form():
    # kI = qI makes every head dot a squared norm: s = sum_h w_h ||qI_h||^2
    rng = np.random.default_rng(1)
    qI, kI, w = _rand_idx(rng, 3, 9, 8, 16, -128, 127)
    kI[:] = qI[:, None]
    s = O.score_decode(qI, kI, w, np.array([9 * 64] * 3), 64)
    norms = np.linalg.norm(qI.astype(np.float64), axis=2) ** 2          # [B, H]
    expect = np.rint((norms * w).sum(axis=1)).astype(np.int64)
    assert np.array_equal(s, np.repeat(expect[:, None], 9, axis=1))


def test_score_relu_split_identity():
    # ReLU(x) + ReLU(-x) = |x| per head: s(k) + s(-k) = sum_h w_h |q_h . k_h|
    rng = np.random.default_rng(2)
    qI, kI, w = _rand_idx(rng, 2, 17, 4, 16, -100, 100)
    L = np.array([17 * 16] * 2)
    sp = O.score_decode(qI, kI, w, L, 16)
    sm = O.score_decode(qI, (-kI.astype(np.int16)).astype(np.int8), w, L, 16)
    # matmul over r per head: kI [B,nb,H,1,r] x qI [B,1,H,r,1] -> [B,nb,H]
    absdot = np.abs(np.matmul(kI.astype(np.float64)[..., None, :], qI.astype(np.float64)[:, None, :, :, None])[..., 0, 0])
    expect = np.rint((absdot * w[:, None, :]).sum(-1)).astype(np.int64)
    assert np.array_equal(sp + sm, expect)
    assert (sp >= 0).all() and (sm >= 0).all()


def test_score_linear_in_w_and_invariances():
    rng = np.random.default_rng(3)
    qI, kI, w = _rand_idx(rng, 2, 11, 8, 16)
    L = np.array([11 * 64, 11 * 64])
    s = O.score_decode(qI, kI, w, L, 64)
    assert np.array_equal(O.score_decode(qI, kI, (2 * w).astype(np.int8), L, 64), 2 * s)
    perm_r = rng.permutation(16)
    assert np.array_equal(O.score_decode(qI[..., perm_r], kI[..., perm_r], w, L, 64), s)
    perm_h = rng.permutation(8)
    assert np.array_equal(O.score_decode(qI[:, perm_h], kI[:, :, perm_h], w[:, perm_h], L, 64), s)
    # one-hot head weight isolates one head: the ReLU of a plain dot product
    w1 = np.zeros_like(w)
    w1[:, 5] = 1
    s1 = O.score_decode(qI, kI, w1, L, 64)
    for b in range(2):
        for j in range(11):
            assert s1[b, j] == max(0, int(np.dot(qI[b, 5].astype(np.int64), kI[b, j, 5].astype(np.int64))))


def test_score_prefill_matches_decode_rows_and_mask():
    rng = np.random.default_rng(4)
    qIb = rng.integers(-128, 128, size=(1, 6, 3, 16), dtype=np.int8)
    kIb = rng.integers(-128, 128, size=(1, 6, 3, 16), dtype=np.int8)
    w = rng.integers(1, 5, size=(1, 6, 3), dtype=np.int8)
    S = O.score_prefill(qIb, kIb, w)
    for i in range(6):
        ref = O.score_decode(qIb[:, i], kIb, w[:, i], np.array([6 * 8]), 8)
        assert np.array_equal(S[0, i, :i], ref[0, :i])
        assert (S[0, i, i:] == O.INT32_MIN).all()
    # chunked rows agree with the one-shot rows
    S2 = O.score_prefill(qIb[:, 3:], kIb, w[:, 3:], q_blk0=3)
    assert np.array_equal(S2, S[:, 3:])


def test_score_grouped_golden():
    g = gold("score_tiny.json")["grouped"]
    qI = np.array(g["qI"], dtype=np.int8)[None]
    kI = np.array(g["kI"], dtype=np.int8)[None]
    w = np.array(g["w"], dtype=np.int8)[None]
    for groups in (1, 2, 4):
        s = O.score_decode_grouped(qI, kI, w, np.array([g["seq_len"]]), g["blk"], groups)
        assert s[0].tolist() == g[f"expected_groups{groups}"], groups
    # ragged: the second block lies past a 16-token sequence
    s = O.score_decode_grouped(qI, kI, w, np.array([16]), g["blk"], 2)
    assert s[0].tolist() == [[9, O.INT32_MIN], [4, O.INT32_MIN]]


def test_score_grouped_partitions_the_shared_score():
    # the groups partition the indexer heads, so their scores add up to the
    # shared score, and a single group is the shared score itself
    rng = np.random.default_rng(14)
    qI, kI, w = _rand_idx(rng, 3, 21, 8, 16, -128, 127)
    L = np.array([21 * 32, 400, 33])
    shared = O.score_decode(qI, kI, w, L, 32)
    assert np.array_equal(O.score_decode_grouped(qI, kI, w, L, 32, 1)[:, 0], shared)
    for groups in (2, 4, 8):
        s = O.score_decode_grouped(qI, kI, w, L, 32, groups)
        valid = shared != O.INT32_MIN
        for b in range(3):
            v = valid[b]
            assert np.array_equal(s[b][:, v].sum(axis=0), shared[b][v])
            assert (s[b][:, ~v] == O.INT32_MIN).all()


def test_score_grouped_finds_each_groups_planted_blocks():
    # blocks planted into one group's indexer heads rank first in that group
    # and carry no signal for the others
    from gen import SMALL_DECODE_PERGROUP, make_decode_index
    cfg = SMALL_DECODE_PERGROUP
    inp = make_decode_index(cfg, seed=0)
    s = O.score_decode_grouped(inp["qI"], inp["kI"], inp["w"], inp["seq_len"], cfg.blk, cfg.Hkv)
    sel, _ = O.select_decode_grouped(s, inp["seq_len"], cfg.blk, cfg.n_sink, cfg.n_local, "topk", k=cfg.k)
    for b in range(cfg.B):
        for g in range(cfg.Hkv):
            mine = set(int(x) for x in inp["planted_g"][b][g])
            assert mine and mine <= set(int(x) for x in sel[b][g]), (b, g)
            others = set().union(*(set(int(x) for x in inp["planted_g"][b][o]) for o in range(cfg.Hkv) if o != g))
            lo = min(int(s[b, g, j]) for j in mine)
            assert all(int(s[b, g, j]) < lo for j in others - mine), (b, g)


def test_int4_quantization_golden():
    g = gold("int4_tiny.json")
    codes, exps = O.quantize_selector_keys(np.array(g["kI"], dtype=np.int8))
    assert exps.tolist() == g["exps"]
    assert codes.tolist() == g["codes"]
    assert O.pack_int4(codes)[0].tolist() == g["packed_row0"]


def test_int4_quantization_bounds_minimality_and_packing():
    rng = np.random.default_rng(31)
    kI = rng.integers(-128, 128, size=(500, 16), dtype=np.int8)
    kI[:50] = rng.integers(-8, 8, size=(50, 16))           # already int4: exact
    kI[50:100] = rng.integers(-30, 31, size=(50, 16))
    codes, exps = O.quantize_selector_keys(kI)
    x = kI.astype(np.int64)
    e = exps.astype(np.int64)[:, None]
    deq = O.dequantize_selector_keys(codes, exps).astype(np.int64)
    assert (codes >= -8).all() and (codes <= 7).all()
    # round to nearest: within half a step, ties upward
    assert (np.abs(deq - x) * 2 <= (1 << e)).all()
    assert ((2 * (deq - x) == (1 << e)) | (np.abs(deq - x) * 2 < (1 << e)) | (e == 0)).all()
    assert (exps[:50] == 0).all() and np.array_equal(deq[:50], x[:50])
    # minimal: one exponent less overflows the int4 range for some element
    for i in np.nonzero(exps > 0)[0]:
        e1 = int(exps[i]) - 1
        c = [math.floor(v / 2 ** e1 + 0.5) for v in x[i]]
        assert min(c) < -8 or max(c) > 7
    # packing: low nibble = even element, high nibble = odd element, 4-bit two's complement
    p = O.pack_int4(codes).astype(np.int64)
    lo = ((p & 0xF) ^ 8) - 8
    hi = ((p >> 4) ^ 8) - 8
    assert np.array_equal(lo, codes[:, 0::2]) and np.array_equal(hi, codes[:, 1::2])


def test_int4_scores_equal_int8_scores_when_keys_fit():
    # keys already in the int4 range quantise exactly, so the scores are unchanged
    rng = np.random.default_rng(32)
    qI, kI, w = _rand_idx(rng, 2, 30, 8, 16, -8, 7)
    codes, exps = O.quantize_selector_keys(kI)
    L = np.array([30 * 64, 1000])
    assert np.array_equal(O.score_decode(qI, O.dequantize_selector_keys(codes, exps), w, L, 64),
                          O.score_decode(qI, kI, w, L, 64))


def test_pool_golden():
    g = gold("pool_tiny.json")
    toks = np.array([b["tokens"] for b in g["blocks"]], dtype=np.int8).reshape(1, -1, 1, 1)
    pooled = O.pool_blocks(toks, g["blk"])
    assert pooled[0, :, 0, 0].tolist() == [b["expected"] for b in g["blocks"]]


def test_pool_constant_block_and_ragged():
    rng = np.random.default_rng(5)
    c = rng.integers(-128, 128, size=(2, 5, 3, 16), dtype=np.int8)
    toks = np.repeat(c, 64, axis=1)                       # each block constant
    assert np.array_equal(O.pool_blocks(toks, 64), c)
    # ragged last block of 10 tokens averages only those tokens
    t2 = np.repeat(c, 64, axis=1)[:, :4 * 64 + 10]
    assert np.array_equal(O.pool_blocks(t2, 64), c)
    # brute-force rounding against exact rationals
    x = rng.integers(-128, 128, size=(1, 3 * 64, 2, 4), dtype=np.int8)
    p = O.pool_blocks(x, 64)
    from fractions import Fraction
    for j in range(3):
        for h in range(2):
            for c_ in range(4):
                m = Fraction(int(x[0, j * 64:(j + 1) * 64, h, c_].astype(np.int64).sum()), 64)
                assert p[0, j, h, c_] == math.floor(m + Fraction(1, 2))


# ------------------------------------------------------------- selection ----

def test_topk_golden():
    g = gold("select_tiny.json")
    s = np.array(g["scores"])
    res, cand = O.decode_sets(g["seq_len"], g["blk"], g["n_sink"], g["n_local"])
    assert O.select_row_topk(res, cand, s, g["topk"]["k"]) == g["topk"]["expected"]
    assert O.select_row_topk(res, cand, s, g["topk_all"]["k"]) == g["topk_all"]["expected"]


def test_topp_golden():
    g = gold("select_tiny.json")["topp"]
    s = np.array(g["scores"])
    res, cand = O.decode_sets(g["seq_len"], g["blk"], g["n_sink"], g["n_local"])
    for c in g["cases"]:
        sel, info = O.select_row_topp(res, cand, s, g["beta"], c["p"], c["k_min"], c["k_max"])
        assert info["kp"] == c["kp"], c
        assert sel == c["expected"], c
    g = gold("select_tiny.json")["topp_exact"]
    res, cand = O.decode_sets(g["seq_len"], g["blk"], g["n_sink"], g["n_local"])
    sel, info = O.select_row_topp(res, cand, np.array(g["scores"]), g["beta"], g["p"], 0, 99)
    assert info["kp"] == g["kp"] and sel == g["expected"]


def _topk_characterisation(chosen, cand, s, k):
    chosen = set(chosen)
    assert len(chosen) == min(k, len(cand))
    rest = set(cand) - chosen
    for a in chosen:
        for b in rest:
            assert s[a] > s[b] or (s[a] == s[b] and a < b)


@pytest.mark.parametrize("seed", range(20))
def test_topk_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    nb = int(rng.integers(1, 40))
    s = rng.integers(0, 6, size=nb)           # many ties on purpose
    k = int(rng.integers(0, 12))
    ns, nl = int(rng.integers(0, 3)), int(rng.integers(0, 3))
    res, cand = O.decode_sets(nb * 16, 16, ns, nl)
    out = O.select_row_topk(res, cand, s, k)
    assert out == sorted(set(out))
    assert set(res) <= set(out)
    _topk_characterisation(set(out) - set(res), cand, s, k)
    # exhaustive: among all k-subsets, the chosen one is the lexicographically best
    # list of (score desc, index asc) keys
    kk = min(k, len(cand))
    if len(cand) <= 10:
        best = max(itertools.combinations(cand, kk),
                   key=lambda c: sorted([(int(s[j]), -j) for j in c], reverse=True))
        assert set(best) == set(out) - set(res)


def test_topk_all_equal_and_large_k():
    s = np.full(50, 7)
    res, cand = O.decode_sets(50 * 64, 64, 1, 4)
    assert O.select_row_topk(res, cand, s, 5) == sorted(set(res) | {1, 2, 3, 4, 5})
    assert O.select_row_topk(res, cand, s, 1000) == list(range(50))


def test_prefill_sets():
    res, cand = O.prefill_sets(0, 1, 0)
    assert res == [0] and cand == []
    res, cand = O.prefill_sets(5, 1, 0)
    assert res == [0, 5] and cand == [1, 2, 3, 4]
    res, cand = O.prefill_sets(5, 1, 2)
    assert res == [0, 3, 4, 5] and cand == [1, 2]


@pytest.mark.parametrize("seed", range(30))
def test_topp_minimality_brute_force(seed):
    # the greedy prefix is a smallest set whose softmax mass reaches p
    rng = np.random.default_rng(200 + seed)
    n = int(rng.integers(1, 11))
    s = rng.integers(-20, 21, size=n)
    beta = float(rng.choice([0.125, 0.3, 1.0]))
    p = float(rng.choice([0.5, 0.8, 0.9, 0.95]))
    cand = list(range(n))
    order = O.rank_order(cand, s)
    kp, M = O.topp_count(order, s, beta, p)
    mass = scipy.special.softmax(beta * s.astype(np.float64))       # library softmax
    assert np.allclose(np.sort(mass)[::-1], O.topp_masses(order, s, beta), rtol=1e-12, atol=1e-15)
    best = min(len(c) for r in range(1, n + 1) for c in itertools.combinations(range(n), r)
               if mass[list(c)].sum() >= p - 1e-12)
    assert kp == best
    assert M[kp - 1] >= p - 1e-12
    if kp > 1:
        assert M[kp - 2] < p


def test_topp_special_cases():
    res, cand = O.decode_sets(40 * 64, 64, 1, 4)
    s = np.zeros(40, dtype=np.int64)
    s[17] = 10000                                         # one-hot mass
    sel, info = O.select_row_topp(res, cand, s, 0.125, 0.9, 16, 512)
    assert info["kp"] == 1 and info["k"] == 16 and 17 in sel
    # n equal planted blocks dominating -> kp = ceil(p n) (n not a multiple of 10)
    for n in (1, 3, 7, 13, 19, 23):
        s = np.zeros(40, dtype=np.int64)
        s[np.arange(5, 5 + n)] = 20000
        sel, info = O.select_row_topp(res, cand, s, 0.125, 0.9, 0, 512)
        assert info["kp"] == math.ceil(0.9 * n)
    # p = 1 takes every candidate
    s = np.arange(40)
    sel, info = O.select_row_topp(res, cand, s, 0.01, 1.0, 0, 512)
    assert sel == list(range(40))
    # K_max caps the nucleus, reserved come on top
    sel, info = O.select_row_topp(res, cand, s, 0.0, 0.99, 0, 3)
    assert len(sel) == len(res) + 3


# ------------------------------------------------------------- attention ----

def test_attention_golden():
    g = gold("attn_tiny.json")
    for key in ("single_key", "equal_logits", "ln3_gap"):
        c = g[key]
        o, lse = O.softmax_attend(np.array(c["q"]), np.array(c["K"]), np.array(c["V"]), 1.0)
        assert np.allclose(o, c["o"], atol=1e-14), key
        assert abs(lse - c["lse"]) < 1e-14, key


def _sdpa(q, k, v, scale, mask=None, causal=False):
    # library special case: torch's scaled_dot_product_attention in float64 on CPU
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=None if mask is None else torch.from_numpy(mask), is_causal=causal, scale=scale).numpy()


def test_decode_all_blocks_equals_dense():
    rng = np.random.default_rng(7)
    B, Hq, Hkv, d, T, blk = 2, 6, 2, 32, 200, 16
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    L = np.array([200, 77])
    sel = [list(range(-(-int(x) // blk))) for x in L]
    o, lse = O.decode_attention(q, k, v, "f32", L, sel, blk)
    for b in range(B):
        G = Hq // Hkv
        kk = np.repeat(k[b, :, :L[b]], G, axis=0)
        vv = np.repeat(v[b, :, :L[b]], G, axis=0)
        ref = _sdpa(q[b][:, None], kk, vv, 1 / math.sqrt(d))[:, 0]
        assert np.allclose(o[b], ref, atol=1e-12)
        x = np.einsum("hd,htd->ht", q[b], kk) / math.sqrt(d)
        assert np.allclose(lse[b], scipy.special.logsumexp(x, axis=1), atol=1e-12)


def test_decode_gather_equals_masked_dense_and_set_semantics():
    rng = np.random.default_rng(8)
    B, Hq, Hkv, d, T, blk = 1, 4, 1, 16, 160, 16
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    sel = [[0, 3, 4, 9]]
    o, _ = O.decode_attention(q, k, v, "f32", np.array([150]), sel, blk)
    mask = np.full((1, T), -np.inf)
    for j in sel[0]:
        mask[0, j * blk:min((j + 1) * blk, 150)] = 0.0
    ref = _sdpa(q[0][:, None], np.repeat(k[0], Hq, 0), np.repeat(v[0], Hq, 0), 1 / 4.0, mask=mask)[:, 0]
    assert np.allclose(o[0], ref, atol=1e-12)
    o2, _ = O.decode_attention(q, k, v, "f32", np.array([150]), [[9, 0, 4, 3]], blk)
    assert np.allclose(o, o2, atol=1e-13)


def test_decode_per_group_lists_route_by_kv_head():
    # each query head attends over its own KV group's list: equal to masked
    # dense attention with that group's blocks; identical lists give the
    # shared-list result
    rng = np.random.default_rng(15)
    B, Hq, Hkv, d, T, blk = 2, 6, 3, 16, 160, 16
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    L = np.array([160, 101])
    sel = [[[0, 2, 9], [1, 5], [0, 3, 4, 6]], [[6], [0, 1, 2], [2, 4]]]
    o, lse = O.decode_attention(q, k, v, "f32", L, sel, blk, per_group=True)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            g = h // G
            mask = np.full((1, T), -np.inf)
            for j in sel[b][g]:
                mask[0, j * blk:min((j + 1) * blk, int(L[b]))] = 0.0
            ref = _sdpa(q[b, h][None, None], k[b, g][None], v[b, g][None], 1 / 4.0, mask=mask[None])[0, 0]
            assert np.allclose(o[b, h], ref, atol=1e-12), (b, h)
    same = [[s0[1]] * Hkv for s0 in sel]
    o1, l1 = O.decode_attention(q, k, v, "f32", L, same, blk, per_group=True)
    o2, l2 = O.decode_attention(q, k, v, "f32", L, [s0[1] for s0 in sel], blk)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_kv_permutation_invariance():
    # PBS-Attn §1: permuting key/value pairs together leaves the output unchanged
    rng = np.random.default_rng(9)
    qv = rng.standard_normal(24)
    K = rng.standard_normal((50, 24))
    V = rng.standard_normal((50, 24))
    pi = rng.permutation(50)
    o1, l1 = O.softmax_attend(qv, K, V, 0.3)
    o2, l2 = O.softmax_attend(qv, K[pi], V[pi], 0.3)
    assert np.allclose(o1, o2, atol=1e-13) and abs(l1 - l2) < 1e-12
    o3, _ = O.softmax_attend(qv, K, V[pi], 0.3)               # broken pairing changes it
    assert not np.allclose(o1, o3, atol=1e-6)


def test_local_heads_window_covers_all_equals_dense():
    rng = np.random.default_rng(10)
    B, Hq, Hkv, d, T = 1, 4, 2, 16, 100
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    hm = np.array([1, 1], dtype=np.uint8)
    o, _ = O.decode_attention(q, k, v, "f32", np.array([90]), [[]], 16, hm, 0, 1000)
    ref = _sdpa(q[0][:, None], np.repeat(k[0, :, :90], 2, 0), np.repeat(v[0, :, :90], 2, 0), 0.25)[:, 0]
    assert np.allclose(o[0], ref, atol=1e-12)
    toks = O.decode_tokens([], 90, 16, 1, 4, 10)
    assert toks.tolist() == [0, 1, 2, 3] + list(range(80, 90))
    toks = O.decode_tokens([], 12, 16, 1, 4, 10)           # sink and window overlap
    assert toks.tolist() == list(range(12))


def test_prefill_all_blocks_equals_dense_causal():
    rng = np.random.default_rng(11)
    B, Hq, Hkv, d, T, blk = 1, 4, 2, 16, 80, 16
    q = rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    pos = np.arange(T)
    sel = [[list(range(i + 1)) for i in range(5)]]
    o, _ = O.prefill_attention(q, k, v, "f32", pos, pos, sel, blk)
    ref = _sdpa(q[0], np.repeat(k[0], 2, 0), np.repeat(v[0], 2, 0), 0.25, causal=True)
    assert np.allclose(o[0], ref, atol=1e-12)
    # a later chunk computed alone matches
    oc, _ = O.prefill_attention(q[:, :, 48:], k, v, "f32", pos, pos, [sel[0][3:]], blk, q_blk0=3)
    assert np.allclose(oc, o[:, :, 48:], atol=0)


def test_permuted_pipeline_all_blocks_equals_unpermuted_dense():
    # PBS-Attn §1-§2: permute Q,K,V within segments, causal mask on original
    # positions, inverse-permute O -> the unpermuted dense causal result
    rng = np.random.default_rng(12)
    B, Hq, Hkv, d, T, blk, seg = 1, 2, 1, 8, 96, 16, 32
    q = rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    perm = np.concatenate([s + rng.permutation(seg) for s in range(0, T, seg)])
    assert O.check_segment_perm(perm, seg)
    qp, kp, vp = (O.segment_permute(x, perm, axis=2) for x in (q, k, v))
    # every block up to the end of the query block's segment can hold a causal key
    sel = [[list(range(((i * blk) // seg + 1) * seg // blk)) for i in range(T // blk)]]
    op, _ = O.prefill_attention(qp, kp, vp, "f32", perm, perm, sel, blk)
    o = O.segment_permute(op, perm, axis=2, inverse=True)
    ref = _sdpa(q[0], np.repeat(k[0], 2, 0), np.repeat(v[0], 2, 0), 1 / math.sqrt(d), causal=True)
    assert np.allclose(o[0], ref, atol=1e-12)


def test_permute_golden_and_inverse():
    g = gold("permute_tiny.json")
    perm = np.array(g["perm"])
    src = np.array(g["src"])
    assert O.check_segment_perm(perm, g["seg"])
    assert not O.check_segment_perm(np.array(g["not_segment_closed"]), g["seg"])
    assert O.segment_permute(src, perm, 0).tolist() == g["forward"]
    assert O.segment_permute(src, perm, 0, inverse=True).tolist() == g["inverse_of_src"]
    rng = np.random.default_rng(13)
    x = rng.standard_normal((3, 64, 5))
    pr = np.concatenate([s + rng.permutation(16) for s in range(0, 64, 16)])
    y = O.segment_permute(O.segment_permute(x, pr, 1), pr, 1, inverse=True)
    assert np.array_equal(x, y)


def test_importance_permutation_golden():
    g = gold("permute_tiny.json")["importance"]
    perm = O.importance_permutation(np.array([g["imp"]]), np.array([g["seq_len"]]), g["seg"])
    assert perm[0].tolist() == g["perm"]
    assert O.check_segment_perm(perm[0], g["seg"])


def _importance_inputs(rng, B, Hq, Hkv, T, d):
    q = rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    return q, k


def test_key_importance_is_mean_of_sdpa_probabilities():
    # library special case: attention with V = identity returns the probability rows
    rng = np.random.default_rng(21)
    B, Hq, Hkv, T, d, proxy = 2, 6, 2, 150, 16, 24
    q, k = _importance_inputs(rng, B, Hq, Hkv, T, d)
    L = np.array([150, 97])
    imp = O.key_importance(q, k, "f32", L, proxy, scale=0.3)
    G = Hq // Hkv
    for b in range(B):
        n = min(proxy, int(L[b]))
        u0 = int(L[b]) - n
        mask = np.where(np.arange(L[b])[None, :] <= (u0 + np.arange(n))[:, None], 0.0, -np.inf)
        P = _sdpa(q[b, :, u0:L[b]], np.repeat(k[b, :, :L[b]], G, axis=0), np.broadcast_to(np.eye(L[b]), (Hq, L[b], L[b])).copy(),
                  0.3, mask=mask)
        assert np.allclose(imp[b, :L[b]], P.mean(axis=(0, 1)), atol=1e-14)
        assert (imp[b, L[b]:] == 0).all()
        assert abs(imp[b].sum() - 1.0) < 1e-12


def test_key_importance_uniform_keys_closed_form():
    # equal keys: proxy row i (position u0 + i) spreads 1/(u0 + i + 1) over keys 0 .. u0 + i
    rng = np.random.default_rng(22)
    T, proxy = 40, 8
    q = rng.standard_normal((1, 4, T, 8))
    k = np.broadcast_to(rng.standard_normal(8), (1, 2, T, 8)).copy()
    imp = O.key_importance(q, k, "f32", np.array([T]), proxy)
    u0 = T - proxy
    expect = np.array([sum(1.0 / (u0 + i + 1) for i in range(proxy) if t <= u0 + i) / proxy for t in range(T)])
    assert np.allclose(imp[0], expect, atol=1e-14)


def test_importance_permutation_properties_and_heavy_hitters():
    from gen import SMALL_PREFILL_IMPORTANCE, make
    cfg = SMALL_PREFILL_IMPORTANCE
    inp = make(cfg)
    imp = O.key_importance(inp["q"], inp["k"], cfg.dtype, inp["seq_len"], cfg.proxy)
    perm = O.importance_permutation(imp, inp["seq_len"], cfg.seg)
    assert O.check_segment_perm(perm[0], cfg.seg)
    for s0 in range(0, cfg.T, cfg.seg):
        v = imp[0, perm[0, s0:s0 + cfg.seg]]
        assert (np.diff(v) <= 0).all()
        # each segment's heavy hitters lead it
        hh = set(int(t) for t in inp["hh"][0] if s0 <= t < s0 + cfg.seg)
        assert set(perm[0, s0:s0 + len(hh)].tolist()) == hh
    # ragged: keys past seq_len stay in place at the segment's end
    L = np.array([cfg.T - 100])
    imp2 = O.key_importance(inp["q"], inp["k"], cfg.dtype, L, cfg.proxy)
    perm2 = O.importance_permutation(imp2, L, cfg.seg)
    assert perm2[0, L[0]:].tolist() == list(range(L[0], cfg.T))
    assert O.check_segment_perm(perm2[0], cfg.seg)


def test_prefill_block_mass_and_coverage():
    rng = np.random.default_rng(23)
    Hq, Hkv, T, d, blk = 4, 2, 96, 8, 16
    qp = rng.standard_normal((Hq, T, d))
    kp = rng.standard_normal((Hkv, T, d))
    pos = np.concatenate([s + rng.permutation(48) for s in (0, 48)])
    m = O.prefill_block_mass(qp, kp, "f32", pos, pos, blk, [0, 3, 5])
    assert np.allclose(m.sum(axis=1), 1.0, atol=1e-12)
    # library: attention onto one-hot block indicators gives the block masses
    ind = np.zeros((T, T // blk))
    ind[np.arange(T), np.arange(T) // blk] = 1.0
    G = Hq // Hkv
    for n, i in enumerate([0, 3, 5]):
        rows = np.arange(i * blk, (i + 1) * blk)
        mask = np.where(pos[None, :] <= pos[rows][:, None], 0.0, -np.inf)
        P = _sdpa(qp[:, rows], np.repeat(kp, G, axis=0), np.broadcast_to(ind, (Hq, T, T // blk)).copy(),
                  1 / math.sqrt(d), mask=mask)
        assert np.allclose(m[n], P.mean(axis=(0, 1)), atol=1e-13)
    assert O.blocks_for_coverage(np.array([0.5, 0.1, 0.3, 0.1]), 0.8) == 2
    assert O.blocks_for_coverage(np.array([0.5, 0.1, 0.3, 0.1]), 0.81) == 3
    assert O.blocks_for_coverage(np.array([0.25, 0.25, 0.25, 0.25]), 1.0) == 4


def test_bf16_widening_and_rounding_golden():
    g = gold("bf16_tiny.json")
    for c in g["cases"]:
        bits = f32_to_bf16_bits(np.array([c["x"]], dtype=np.float32))
        assert int(bits[0]) == c["bits"], c
    assert O.bf16_to_f64(np.array([16256, 49152], dtype=np.uint16)).tolist() == [1.0, -2.0]
