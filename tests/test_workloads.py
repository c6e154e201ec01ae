"""The seeded workloads: determinism, planted structure and the measured
properties the configurations promise (planted mass, query-dependent top-p
budgets, segment-closed permutations).  CPU only.
"""
import numpy as np
import pytest

import gen
import oracle as O


def test_deterministic_and_thread_independent():
    a = gen.make(gen.SMALL_DECODE_TOPK, seed=0, threads=1)
    b = gen.make(gen.SMALL_DECODE_TOPK, seed=0, threads=4)
    for key in ("q", "k", "v", "qI", "kI", "w", "seq_len", "head_mode"):
        assert np.array_equal(a[key], b[key]), key
    c = gen.make(gen.SMALL_DECODE_TOPK, seed=1)
    assert not np.array_equal(a["k"], c["k"])


def test_planted_blocks_avoid_reserved_and_rank_first():
    for cfg in (gen.TINY_DECODE, gen.SMALL_DECODE_TOPK, gen.SMALL_DECODE_HEADSPLIT):
        inp = gen.make(cfg)
        s = O.score_decode(inp["qI"], inp["kI"], inp["w"], inp["seq_len"], cfg.blk)
        for b in range(cfg.B):
            res, cand = O.decode_sets(inp["seq_len"][b], cfg.blk, cfg.n_sink, cfg.n_local)
            pl = set(inp["planted"][b].tolist())
            assert pl <= set(cand)
            top = set(O.topk_choose(cand, s[b], len(pl)))
            assert top == pl, (cfg.name, b)


def test_copy_planting_ties_exactly():
    inp = gen.make(gen.SMALL_DECODE_TOPP)
    s = O.score_decode(inp["qI"], inp["kI"], inp["w"], inp["seq_len"], 64)
    for b in range(inp["cfg"].B):
        vals = set(int(s[b, j]) for j in inp["planted"][b])
        assert len(vals) == 1
        expect = int((inp["w"][b].astype(np.int64) * (inp["qI"][b].astype(np.int64) ** 2).sum(-1)).sum())
        assert vals == {expect}


def test_planted_mass_32k_about_sixty_percent():
    inp = gen.make(gen.DECODE_32K)
    toks = np.concatenate([np.arange(j * 64, (j + 1) * 64) for j in inp["planted"][0]])
    m = O.dense_mass(inp["q"][0], inp["k"][0], "bf16", 32768, toks)
    assert 0.55 <= m.mean() <= 0.65, m.mean()


def test_topp_budget_varies_by_query():
    # the 128K top-p workload's indexer streams at full size, drawn as gen.synth
    # draws them (the 8 GiB K/V cache is not needed for selection)
    cfg = gen.DECODE_128K_TOPP
    idx = gen.make_decode_index(cfg)
    qI, kI, w, B = idx["qI"], idx["kI"], idx["w"], cfg.B
    n_pl = [len(p) for p in idx["planted"]]
    L = np.full(B, cfg.T)
    s = O.score_decode(qI, kI, w, L, cfg.blk)
    sel, info = O.select_decode(s, L, cfg.blk, cfg.n_sink, cfg.n_local, "topp", beta=cfg.beta, p=cfg.p,
                                k_min=cfg.k_min, k_max=cfg.k_max)
    counts = [len(x) for x in sel]
    assert min(counts) >= 5 + 16 and max(counts) <= 5 + 512
    assert len(set(counts)) > 8                      # the budget follows the query
    for n, i in zip(n_pl, info):
        if n > 17:
            assert abs(i["kp"] - np.ceil(0.9 * n)) <= 1


def test_prefill_permutation_is_segment_closed():
    inp = gen.make(gen.SMALL_PREFILL)
    assert O.check_segment_perm(inp["perm"], gen.SMALL_PREFILL.seg)
    assert not np.array_equal(inp["perm"], np.arange(len(inp["perm"])))


def test_importance_permutation_needs_fewer_blocks_for_coverage():
    """PBS-Attn "Resultados Clave": importance-sorted segments need fewer key
    blocks for the same attention coverage than an arbitrary order.  On the
    heavy-hitter workload at 16K tokens (sampled query blocks, dense fp64 mass),
    the importance order needs fewer blocks for 97.5 % coverage, and the
    indexer's top-k blocks capture more of the mass."""
    import dataclasses
    import oracle as O
    cfg = dataclasses.replace(gen.SMALL_PREFILL_IMPORTANCE, T=16384, seg=4096, k=32)
    inp = gen.make(cfg)
    imp = O.key_importance(inp["q"], inp["k"], cfg.dtype, inp["seq_len"], cfg.proxy)
    perms = {"random": inp["perm"].astype(np.int64),
             "importance": O.importance_permutation(imp, inp["seq_len"], cfg.seg)[0]}
    qb = [40, 100, 160, 230]
    res = {}
    for name, perm in perms.items():
        qp = O.segment_permute(inp["q"][0], perm, 1)
        kp = O.segment_permute(inp["k"][0], perm, 1)
        m = O.prefill_block_mass(qp, kp, cfg.dtype, perm, perm, cfg.blk, qb)
        sel = O.prefill_front(dict(inp, perm=perm.astype(np.int32)))["sel"][0]
        res[name] = (np.mean([O.blocks_for_coverage(m[n], 0.975) for n in range(len(qb))]),
                     np.mean([m[n, sel[i]].sum() for n, i in enumerate(qb)]))
    assert res["importance"][0] < 0.95 * res["random"][0], res
    assert res["importance"][1] > res["random"][1] + 0.2, res


def test_int4_selector_cache_keeps_the_selection():
    """SpotAttention §4: the int4 selector cache costs no measurable accuracy.  On
    the small top-p workload the selections from int4 keys equal those from
    the int8 keys, sequence by sequence."""
    import dataclasses
    import oracle as O
    cfg = gen.SMALL_DECODE_TOPP_Q4
    inp = gen.make(cfg)
    r4 = O.decode_step(inp)
    r8 = O.decode_step(dict(inp, cfg=dataclasses.replace(cfg, selector_q4=False)))
    for b in range(cfg.B):
        assert r4["sel"][b] == r8["sel"][b], b
