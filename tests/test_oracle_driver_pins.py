"""Pins for the oracle's whole-path drivers: decode_step, prefill_front,
prefill_step and dense_mass.

Every full-size GPU parity test compares against these drivers, so their
wiring (which scores feed which selection, which permutation feeds which
tensor, which lists feed which heads) is pinned here against hand-worked
fixtures and library routines, independently of the functions they compose.
No GPU needed.
"""
import json
import math
import os

import numpy as np
import scipy.special
import torch

import oracle as O
from gen import DecodeConfig, PrefillConfig

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _sdpa(q, k, v, scale, mask=None, causal=False):
    # library special case: torch's scaled_dot_product_attention in float64 on CPU
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=None if mask is None else torch.from_numpy(mask), is_causal=causal, scale=scale).numpy()


def _masked_ref(qv, K, V, toks, scale):
    """Attention of one query over the listed token rows: SDPA with -inf outside them, and the lse."""
    mask = np.full((1, K.shape[0]), -np.inf)
    mask[0, toks] = 0.0
    o = _sdpa(qv[None, None], K[None], V[None], scale, mask=mask[None])[0, 0]
    lse = scipy.special.logsumexp((K[toks] @ qv) * scale)
    return o, lse


# ------------------------------------------------------------ decode_step ----

def _decode_case(g, name, seed):
    c = g["cases"][name]
    H, Hq, Hkv = c["heads"], c["Hq"], c["Hkv"]
    blk, Tcap, L = g["blk"], g["Tcap"], g["seq_len"]
    d = 4
    cfg = DecodeConfig(
        name=name, cfg_id=900, B=1, Hq=Hq, Hkv=Hkv, d=d, T=Tcap, blk=blk, H_idx=H, r=2, dtype="f32",
        n_sink=g["n_sink"], n_local=g["n_local"], select=c["select"], k=c.get("k", 0), p=c.get("p", 0.0),
        beta=math.log(2.0) if c.get("beta_ln2") else 1.0, k_min=c.get("k_min", 0), k_max=c.get("k_max", 0),
        local_sink_tok=c.get("local_sink_tok", 0), local_window_tok=c.get("local_window_tok", 0),
        per_group=c["per_group"], selector_q4=c["q4"])
    qI = np.zeros((1, H, 2), dtype=np.int8)
    kI = np.zeros((1, 8, H, 2), dtype=np.int8)
    qI[0, 0, 0] = 1
    kI[0, :, 0, 0] = g["c"]
    if H == 2:
        qI[0, 1, 1] = 1
        kI[0, :, 1, 1] = g["e"]
    rng = np.random.default_rng(seed)
    inp = dict(cfg=cfg, qI=qI, kI=kI, w=np.array([c["w"]], dtype=np.int8),
               seq_len=np.array([L], dtype=np.int32),
               head_mode=np.array(c.get("head_mode", [0] * Hkv), dtype=np.uint8),
               q=rng.standard_normal((1, Hq, d)).astype(np.float32),
               k=rng.standard_normal((1, Hkv, Tcap, d)).astype(np.float32),
               v=rng.standard_normal((1, Hkv, Tcap, d)).astype(np.float32))
    return cfg, c, inp


def _tokens_of(blocks, blk, L):
    return [t for j in blocks for t in range(j * blk, min((j + 1) * blk, L))]


def _check_decode_attention(g, cfg, c, inp, res):
    G = cfg.Hq // cfg.Hkv
    for h in range(cfg.Hq):
        gi = h // G
        if "tokens" in c:
            toks = c["tokens"][gi]
        else:
            sel = c["sel"][gi] if cfg.per_group else c["sel"]
            toks = _tokens_of(sel, g["blk"], g["seq_len"])
        o, lse = _masked_ref(inp["q"][0, h].astype(np.float64), inp["k"][0, gi].astype(np.float64),
                             inp["v"][0, gi].astype(np.float64), toks, 1 / math.sqrt(cfg.d))
        assert np.allclose(res["o"][0, h], o, atol=1e-12), h
        assert abs(res["lse"][0, h] - lse) < 1e-12, h


def test_decode_step_shared_topk_int8_and_int4():
    g = gold("decode_step_tiny.json")
    for i, name in enumerate(("shared_topk_int8", "shared_topk_int4")):
        cfg, c, inp = _decode_case(g, name, 40 + i)
        res = O.decode_step(inp)
        assert res["scores"][0].tolist() == c["scores"], name
        assert res["sel"] == [c["sel"]], name
        _check_decode_attention(g, cfg, c, inp, res)


def test_decode_step_shared_topp():
    g = gold("decode_step_tiny.json")
    cfg, c, inp = _decode_case(g, "shared_topp", 42)
    res = O.decode_step(inp)
    assert res["scores"][0].tolist() == c["scores"]
    assert res["sel"] == [c["sel"]]
    assert res["info"][0]["kp"] == 3
    _check_decode_attention(g, cfg, c, inp, res)


def test_decode_step_per_group_topk_and_topp():
    g = gold("decode_step_tiny.json")
    for i, name in enumerate(("per_group_topk", "per_group_topp")):
        cfg, c, inp = _decode_case(g, name, 43 + i)
        res = O.decode_step(inp)
        assert res["scores"][0].tolist() == c["scores"], name
        assert res["sel"] == [c["sel"]], name
        _check_decode_attention(g, cfg, c, inp, res)


def test_decode_step_local_heads():
    g = gold("decode_step_tiny.json")
    cfg, c, inp = _decode_case(g, "local_heads", 45)
    res = O.decode_step(inp)
    assert res["scores"][0].tolist() == c["scores"]
    assert res["sel"] == [c["sel"]]
    _check_decode_attention(g, cfg, c, inp, res)


def test_decode_step_head_and_batch_subsets_match_full_run():
    g = gold("decode_step_tiny.json")
    cfg, c, inp = _decode_case(g, "local_heads", 46)
    full = O.decode_step(inp)
    part = O.decode_step(inp, heads=[3])
    assert np.array_equal(part["o"][0, 3], full["o"][0, 3])
    assert np.isnan(part["o"][0, :3]).all()


# ----------------------------------------------------------- prefill_front ----

def _prefill_front_case():
    g = gold("prefill_front_tiny.json")
    T = g["T"]
    cfg = PrefillConfig(name="front_tiny", cfg_id=901, B=1, T=T, Hq=2, Hkv=1, d=4, blk=g["blk"], H_idx=1, r=2,
                        k=g["k"], n_sink=g["n_sink"], n_local=g["n_local"], seg=g["seg"], dtype="f32")
    t = np.arange(T)
    qI_tok = np.stack([np.ones(T), 8 - 2 * t], axis=1).astype(np.int8)[None, :, None, :]
    kI_tok = np.stack([t, np.ones(T)], axis=1).astype(np.int8)[None, :, None, :]
    inp = dict(cfg=cfg, qI_tok=qI_tok, kI_tok=kI_tok, w=np.array(g["w"], dtype=np.int8).reshape(1, 4, 1),
               perm=np.array(g["perm"], dtype=np.int32))
    return g, cfg, inp


def test_prefill_front_golden_two_segments():
    g, cfg, inp = _prefill_front_case()
    f = O.prefill_front(inp)
    assert f["kIb"][0, :, 0].tolist() == g["kIb"]
    assert f["qIb"][0, :, 0].tolist() == g["qIb"]
    expect = [[O.INT32_MIN if v is None else v for v in row] for row in g["scores"]]
    assert f["scores"][0].tolist() == expect
    assert f["sel"] == [g["sel"]]
    assert f["pos"].tolist() == g["perm"]


# ------------------------------------------------------------ prefill_step ----

def _prefill_inputs(rng, B, Hq, Hkv, T, d, blk, seg, k, H_idx=2, r=4):
    cfg = PrefillConfig(name="step_pin", cfg_id=902, B=B, T=T, Hq=Hq, Hkv=Hkv, d=d, blk=blk, H_idx=H_idx, r=r, k=k,
                        n_sink=1, n_local=0, seg=seg, dtype="f32")
    perm = np.concatenate([s + rng.permutation(seg) for s in range(0, T, seg)]).astype(np.int32)
    nb = T // blk
    return dict(cfg=cfg, q=rng.standard_normal((B, Hq, T, d)), k=rng.standard_normal((B, Hkv, T, d)),
                v=rng.standard_normal((B, Hkv, T, d)),
                qI_tok=rng.integers(-128, 128, size=(B, T, H_idx, r), dtype=np.int8),
                kI_tok=rng.integers(-128, 128, size=(B, T, H_idx, r), dtype=np.int8),
                w=rng.integers(1, 5, size=(B, nb, H_idx), dtype=np.int8), perm=perm)


def _dense_causal(inp):
    """Unpermuted causal attention in the original order (library routine) and its lse."""
    q, k, v = inp["q"], inp["k"], inp["v"]
    B, Hq, T, d = q.shape
    G = Hq // k.shape[1]
    o = np.empty_like(q)
    lse = np.empty((B, Hq, T))
    causal = np.tril(np.ones((T, T), dtype=bool))
    for b in range(B):
        kk = np.repeat(k[b], G, axis=0)
        o[b] = _sdpa(q[b], kk, np.repeat(v[b], G, axis=0), 1 / math.sqrt(d), causal=True)
        x = np.einsum("htd,hsd->hts", q[b], kk) / math.sqrt(d)
        lse[b] = scipy.special.logsumexp(np.where(causal, x, -np.inf), axis=2)
    return o, lse


def test_prefill_step_segment_blocks_equal_unpermuted_dense_causal():
    # PBS-Attn §1-§2: with every block up to the end of the query block's
    # segment listed, the driver's permuted pipeline (positions from its own
    # front end, inverse permutation of O and lse) is dense causal attention
    rng = np.random.default_rng(50)
    inp = _prefill_inputs(rng, B=2, Hq=4, Hkv=2, T=96, d=8, blk=16, seg=32, k=2)
    cfg = inp["cfg"]
    front = O.prefill_front(inp)
    nb = cfg.T // cfg.blk
    spb = cfg.seg // cfg.blk
    front["sel"] = [[list(range((i // spb + 1) * spb)) for i in range(nb)] for _ in range(cfg.B)]
    res = O.prefill_step(inp, front=front)
    o, lse = _dense_causal(inp)
    assert np.allclose(res["o"], o, atol=1e-12)
    assert np.allclose(res["lse"], lse, atol=1e-12)


def test_prefill_step_own_front_with_block_segments_is_dense_causal():
    # segments of one block: the permutation never moves a token across a
    # block, so a budget above the block count makes the driver's own
    # selection (sink, diagonal and every past block) dense causal
    rng = np.random.default_rng(51)
    inp = _prefill_inputs(rng, B=1, Hq=4, Hkv=1, T=80, d=8, blk=16, seg=16, k=10)
    res = O.prefill_step(inp)
    assert res["sel"][0] == [list(range(i + 1)) for i in range(5)]
    o, lse = _dense_causal(inp)
    assert np.allclose(res["o"], o, atol=1e-12)
    assert np.allclose(res["lse"], lse, atol=1e-12)


def test_prefill_step_sparse_rows_follow_their_lists():
    # a sparse selection: every query row equals masked SDPA over the original
    # positions of the listed blocks' tokens that do not follow it
    rng = np.random.default_rng(52)
    inp = _prefill_inputs(rng, B=1, Hq=2, Hkv=1, T=64, d=8, blk=8, seg=32, k=1)
    res = O.prefill_step(inp)
    perm = inp["perm"]
    q, k, v = inp["q"][0], inp["k"][0, 0], inp["v"][0, 0]
    for slot in range(64):
        i = slot // 8
        pos_u = int(perm[slot])
        toks = [int(perm[t]) for j in res["sel"][0][i] for t in range(j * 8, (j + 1) * 8) if perm[t] <= pos_u]
        for h in range(2):
            o, lse = _masked_ref(q[h, pos_u], k, v, toks, 1 / math.sqrt(8))
            assert np.allclose(res["o"][0, h, pos_u], o, atol=1e-12), (slot, h)
            assert abs(res["lse"][0, h, pos_u] - lse) < 1e-12, (slot, h)


def test_prefill_step_block_subset_matches_full_run():
    rng = np.random.default_rng(53)
    inp = _prefill_inputs(rng, B=1, Hq=2, Hkv=1, T=64, d=8, blk=8, seg=32, k=2)
    full = O.prefill_step(inp)
    front = {key: full[key] for key in ("qIb", "kIb", "scores", "sel", "pos")}
    part = O.prefill_step(inp, front=front, blocks=[2, 5], heads=[1])
    assert "o" not in part
    for i in (2, 5):
        assert np.array_equal(part["o_slot"][0, 1, 8 * i:8 * i + 8], full["o_slot"][0, 1, 8 * i:8 * i + 8])
    assert np.isnan(part["o_slot"][0, 0]).all()


# -------------------------------------------------------------- dense_mass ----

def test_dense_mass_equals_attention_onto_an_indicator():
    # library special case: attention with V = indicator of the token set
    # returns the set's share of the softmax mass over [0, seq_len)
    rng = np.random.default_rng(54)
    Hq, Hkv, T, d, L = 6, 2, 120, 16, 101
    q = rng.standard_normal((Hq, d))
    k = rng.standard_normal((Hkv, T, d))
    toks = np.array([0, 3, 4, 50, 77, 100])
    m = O.dense_mass(q, k, "f32", L, toks)
    ind = np.zeros((L, 1))
    ind[toks] = 1.0
    for h in range(Hq):
        ref = _sdpa(q[h][None, None], k[h // 3, :L][None], ind[None], 1 / math.sqrt(d))[0, 0, 0]
        assert abs(m[h] - ref) < 1e-13, h
    assert np.allclose(O.dense_mass(q, k, "f32", L, np.arange(L)), 1.0, atol=1e-13)
    assert np.array_equal(O.dense_mass(q, k, "f32", L, toks, heads=[4]), m[4:5])
