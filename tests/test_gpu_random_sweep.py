"""Seeded random sweeps of decode, prefill and importance-permutation shapes against the CPU oracle.

Each case draws one configuration that the named workloads do not cover
together: block size, GQA ratio, indexer heads, reserved blocks, top-k or dual
top-p budgets, ragged sequence lengths, local-window heads, fp32 or bf16, and
the selection path (separate sorted, separate sort-free, or fused).  Every
fourth case of the decode, prefill and variant sweeps runs with the library's
device-side checks on, which must accept every input and change no result.
The parity bars are the suite's: scores and top-k lists bit-exact, top-p lists by
the set rule, attention within max |diff| <= 1e-2 and relative L2 <= 2e-3.
"""
import contextlib
import dataclasses

import numpy as np
import pytest
import torch

import gen
import oracle as O
from gpu_util import attn_close, check_importance_perm, check_topp_row, dev, imp_close, sel_lists

pytestmark = pytest.mark.gpu

S = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global S
    import block_sparse_long_int8_amd as mod
    mod.lib()
    S = mod
    yield


PATHS = ("separate", "fused", "separate-hist")


@contextlib.contextmanager
def _checks(seed: int):
    """Every fourth seed runs with the device-side checks on."""
    on = seed % 4 == 3
    if on:
        S.spa_set_debug_checks(True)
    try:
        yield
    finally:
        if on:
            assert S.spa_debug_error() == S.SPA_DBG_NONE
            S.spa_set_debug_checks(False)


def _draw(seed: int):
    """One decode configuration and selection path, from a seeded generator."""
    g = np.random.default_rng(1000 + seed)
    f32 = g.random() < 0.25
    d = int(g.choice([64, 128]))  # bf16 and fp32 both take d 64 and 128
    blk = int(g.choice([16, 32, 64, 128]))
    Hkv = int(g.choice([1, 2, 4]))
    G = int(g.choice([1, 2, 3, 4, 8, 16] if Hkv == 1 else [1, 2, 3, 4, 8]))
    B = int(g.integers(1, 6))
    nb = int(g.integers(6, 81))
    T = nb * blk
    H_idx = int(g.choice([1, 2, 4, 8]))
    n_sink = int(g.integers(0, 3))
    n_local = int(g.integers(0, 5))
    kw = {}
    if g.random() < 0.5:
        kw.update(select="topk", k=int(g.integers(0, nb + 1)))
    else:
        k_min = min(int(g.integers(0, 9)), nb)
        kw.update(select="topp", p=float(g.choice([0.5, 0.8, 0.95])), beta=float(g.choice([0.125, 0.5, 1.0])),
                  k_min=k_min, k_max=int(g.integers(max(k_min, 1), nb + 1)))
    seq_lens = tuple(int(x) for x in g.integers(1, T + 1, size=B))
    n_ret = None
    if Hkv > 1 and g.random() < 0.5:
        n_ret = int(g.integers(0, Hkv + 1))
        kw.update(local_sink_tok=int(g.integers(0, 2 * blk)), local_window_tok=int(g.integers(0, 8 * blk)))
    cfg = dataclasses.replace(
        gen.DECODE_128K_TOPP, name=f"random_decode_{seed}", cfg_id=200 + seed, B=B, Hq=G * Hkv, Hkv=Hkv, d=d, T=T,
        blk=blk, H_idx=H_idx, r=16, dtype="f32" if f32 else "bf16", n_sink=n_sink, n_local=n_local,
        plant_kind="copy", n_plant=(0, min(6, nb)), plant_boost=1.5, plant_mass=0.0, n_retrieval_groups=n_ret,
        seq_lens=seq_lens, **kw)
    return cfg, PATHS[seed % len(PATHS)]


@pytest.mark.parametrize("seed", range(200))
def test_decode_random_sweep(seed):
    cfg, path = _draw(seed)
    print(f"[random decode] seed {seed} {path}: B={cfg.B} Hq={cfg.Hq} Hkv={cfg.Hkv} d={cfg.d} T={cfg.T} blk={cfg.blk} "
          f"H_idx={cfg.H_idx} {cfg.select} k={cfg.k} p={cfg.p} beta={cfg.beta} kmin={cfg.k_min} kmax={cfg.k_max} "
          f"sink={cfg.n_sink} local={cfg.n_local} ret={cfg.n_retrieval_groups} lens={cfg.seq_lens} {cfg.dtype}",
          flush=True)
    inp = gen.make(cfg)
    t = dict(q=dev(inp["q"], cfg.dtype), k=dev(inp["k"], cfg.dtype), v=dev(inp["v"], cfg.dtype),
             qI=dev(inp["qI"]), kI=dev(inp["kI"]), w=dev(inp["w"]), seq_len=dev(inp["seq_len"]),
             head_mode=dev(inp["head_mode"]))
    spec = S.DecodeSpec(B=cfg.B, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d, Tcap=cfg.T, blk=cfg.blk, H_idx=cfg.H_idx, r=cfg.r,
                        n_sink=cfg.n_sink, n_local=cfg.n_local, select=cfg.select, k=cfg.k, beta=cfg.beta, p=cfg.p,
                        k_min=cfg.k_min, k_max=cfg.k_max, local_sink_tok=cfg.local_sink_tok,
                        local_window_tok=cfg.local_window_tok,
                        select_algo="hist" if path.endswith("hist") else "sort")
    step = S.DecodeStep(spec, fused=path == "fused")
    with _checks(seed):
        step(t["q"], t["k"], t["v"], t["qI"], t["kI"], t["w"], t["seq_len"], t["head_mode"], keep_scores=True)
    torch.cuda.synchronize()
    ref = O.decode_step(inp)
    assert np.array_equal(step.scores.cpu().numpy().astype(np.int64), ref["scores"])
    gsel = sel_lists(step.idx, step.count)
    idx_h = step.idx.cpu().numpy()
    for b in range(cfg.B):
        assert (idx_h[b, len(gsel[b]):] == -1).all(), "padding after count must be -1"
    if cfg.select == "topk":
        assert gsel == ref["sel"]
    else:
        for b in range(cfg.B):
            check_topp_row(gsel[b], ref["info"][b], cfg.k_min, cfg.k_max, cfg.p)
    o_ref, lse_ref = O.decode_attention(inp["q"], inp["k"], inp["v"], cfg.dtype, inp["seq_len"], gsel, cfg.blk,
                                        inp["head_mode"], cfg.local_sink_tok, cfg.local_window_tok)
    attn_close(step.out.cpu().numpy(), o_ref)
    lse = step.lse.cpu().numpy()
    fin = np.isfinite(lse_ref)
    assert (np.isfinite(lse) == fin).all()
    assert np.allclose(lse[fin], lse_ref[fin], atol=1e-4, rtol=1e-5)


def _draw_prefill(seed: int):
    """One permuted block-sparse prefill configuration, from a seeded generator."""
    g = np.random.default_rng(2000 + seed)
    Hkv = int(g.choice([1, 2]))
    G = int(g.choice([1, 2, 3, 4, 5, 8]))
    T = 64 * int(g.integers(4, 41))  # whole 64-token blocks, as the per-token indexer inputs must be
    seg = int(g.choice([64, 128, 192, 256, 512, T]))
    return dataclasses.replace(
        gen.SMALL_PREFILL, name=f"random_prefill_{seed}", cfg_id=300 + seed, B=int(g.integers(1, 3)), T=T,
        Hq=G * Hkv, Hkv=Hkv, H_idx=int(g.choice([1, 2, 4, 8])), k=int(g.integers(0, 13)),
        n_sink=int(g.integers(0, 3)), n_local=int(g.integers(0, 3)), seg=seg)


@pytest.mark.parametrize("seed", range(60))
def test_prefill_random_sweep(seed):
    cfg = _draw_prefill(seed)
    print(f"[random prefill] seed {seed}: B={cfg.B} T={cfg.T} Hq={cfg.Hq} Hkv={cfg.Hkv} H_idx={cfg.H_idx} k={cfg.k} "
          f"sink={cfg.n_sink} local={cfg.n_local} seg={cfg.seg}", flush=True)
    inp = gen.make(cfg)
    t = dict(q=dev(inp["q"], "bf16"), k=dev(inp["k"], "bf16"), v=dev(inp["v"], "bf16"), qI=dev(inp["qI_tok"]),
             kI=dev(inp["kI_tok"]), w=dev(inp["w"]), perm=dev(inp["perm"]))
    step = S.PrefillStep(S.PrefillSpec(B=cfg.B, T=cfg.T, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d, blk=cfg.blk,
                                       H_idx=cfg.H_idx, r=cfg.r, k=cfg.k, n_sink=cfg.n_sink, n_local=cfg.n_local,
                                       seg=cfg.seg))
    with _checks(seed):
        out = step(t["q"], t["k"], t["v"], t["qI"], t["kI"], t["w"], t["perm"])
    torch.cuda.synchronize()
    if seed % 2:
        # K and V copied into slot order first, then read in slot order: bit for bit the in-kernel gather
        pos = step.pos
        kp = torch.stack([S.spa_segment_permute(t["k"][b], pos[b].contiguous(), cfg.seg, dim=1) for b in range(cfg.B)])
        vp = torch.stack([S.spa_segment_permute(t["v"][b], pos[b].contiguous(), cfg.seg, dim=1) for b in range(cfg.B)])
        o2, l2 = S.spa_block_sparse_prefill(t["q"], kp, vp, step.idx, step.count, cfg.blk, q_pos=pos, k_pos=pos,
                                            order="original", kv_order="slot")
        torch.cuda.synchronize()
        assert torch.equal(o2, out)
        assert torch.equal(l2, step.lse)
    front = O.prefill_front(inp)
    assert np.array_equal(step.scores.cpu().numpy().astype(np.int64), front["scores"])
    assert sel_lists(step.idx, step.count) == front["sel"]
    ref = O.prefill_step(inp, front=front)
    attn_close(out.cpu().numpy(), ref["o"])
    lse = step.lse.cpu().numpy()
    fin = np.isfinite(ref["lse"])
    assert (np.isfinite(lse) == fin).all()
    assert np.allclose(lse[fin], ref["lse"][fin], atol=1e-4, rtol=1e-5)


def _draw_variant(seed: int):
    """A decode configuration with per-KV-group selection and/or the int4 selector cache."""
    g = np.random.default_rng(3000 + seed)
    per_group = bool(seed % 3 != 1)
    q4 = bool(seed % 3 != 0)
    base, _ = _draw(500 + seed)
    Hkv = int(g.choice([1, 2, 4, 8]))
    hpg = int(g.choice([1, 2, 4])) if per_group else 1
    H_idx = min(32, Hkv * hpg) if per_group else int(g.choice([1, 2, 4, 8, 16, 32]))
    G = int(g.choice([1, 2, 4]))
    cfg = dataclasses.replace(base, name=f"random_variant_{seed}", cfg_id=400 + seed, Hkv=Hkv, Hq=G * Hkv, H_idx=H_idx,
                              per_group=per_group, selector_q4=q4, n_retrieval_groups=None, local_sink_tok=0,
                              local_window_tok=0)
    return cfg, ("separate-hist" if seed % 2 else "separate")


@pytest.mark.parametrize("seed", range(40))
def test_decode_variant_random_sweep(seed):
    cfg, path = _draw_variant(seed)
    print(f"[random decode variant] seed {seed} {path}: per_group={cfg.per_group} q4={cfg.selector_q4} B={cfg.B} "
          f"Hq={cfg.Hq} Hkv={cfg.Hkv} H_idx={cfg.H_idx} T={cfg.T} blk={cfg.blk} {cfg.select} k={cfg.k} p={cfg.p} "
          f"kmin={cfg.k_min} kmax={cfg.k_max} sink={cfg.n_sink} local={cfg.n_local} lens={cfg.seq_lens} {cfg.dtype}",
          flush=True)
    inp = gen.make(cfg)
    t = dict(q=dev(inp["q"], cfg.dtype), k=dev(inp["k"], cfg.dtype), v=dev(inp["v"], cfg.dtype),
             qI=dev(inp["qI"]), kI=dev(inp["kI"]), w=dev(inp["w"]), seq_len=dev(inp["seq_len"]),
             head_mode=dev(inp["head_mode"]))
    spec = S.DecodeSpec(B=cfg.B, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d, Tcap=cfg.T, blk=cfg.blk, H_idx=cfg.H_idx, r=cfg.r,
                        n_sink=cfg.n_sink, n_local=cfg.n_local, select=cfg.select, k=cfg.k, beta=cfg.beta, p=cfg.p,
                        k_min=cfg.k_min, k_max=cfg.k_max, per_group=cfg.per_group, selector_q4=cfg.selector_q4,
                        select_algo="hist" if path.endswith("hist") else "sort")
    step = S.DecodeStep(spec)
    kI = step.quantize_selector(t["kI"]) if cfg.selector_q4 else t["kI"]
    with _checks(seed):
        step(t["q"], t["k"], t["v"], t["qI"], kI, t["w"], t["seq_len"], t["head_mode"], keep_scores=True)
    torch.cuda.synchronize()
    ref = O.decode_step(inp)
    assert np.array_equal(step.scores.cpu().numpy().astype(np.int64), ref["scores"])
    gsel = sel_lists(step.idx, step.count)
    rows = [(b, None) for b in range(cfg.B)] if not cfg.per_group else \
        [(b, g) for b in range(cfg.B) for g in range(cfg.Hkv)]
    for b, g in rows:
        mine = gsel[b] if g is None else gsel[b][g]
        theirs = ref["sel"][b] if g is None else ref["sel"][b][g]
        info = ref["info"][b] if g is None else ref["info"][b][g]
        if cfg.select == "topk":
            assert mine == theirs, (b, g)
        else:
            check_topp_row(mine, info, cfg.k_min, cfg.k_max, cfg.p)
    o_ref, lse_ref = O.decode_attention(inp["q"], inp["k"], inp["v"], cfg.dtype, inp["seq_len"], gsel, cfg.blk,
                                        inp["head_mode"], 0, 0, per_group=cfg.per_group)
    attn_close(step.out.cpu().numpy(), o_ref)
    lse = step.lse.cpu().numpy()
    fin = np.isfinite(lse_ref)
    assert (np.isfinite(lse) == fin).all()
    assert np.allclose(lse[fin], lse_ref[fin], atol=1e-4, rtol=1e-5)


@pytest.mark.parametrize("seed", range(10))
def test_importance_permutation_random_sweep(seed):
    g = np.random.default_rng(4000 + seed)
    B = int(g.integers(1, 4))
    Hkv = int(g.choice([1, 2, 4]))
    Hq = Hkv * int(g.choice([1, 2, 3, 4]))
    T = int(g.integers(64, 3001))
    seg = int(g.choice([64, 100, 256, 1000, 4096]))
    proxy = int(g.integers(1, 65))
    lens = tuple(int(x) for x in g.integers(1, T + 1, size=B)) if g.random() < 0.5 else None
    print(f"[random importance] seed {seed}: B={B} Hq={Hq} Hkv={Hkv} T={T} seg={seg} proxy={proxy} lens={lens}",
          flush=True)
    q = gen.f32_to_bf16_bits(g.standard_normal((B, Hq, T, 128), dtype=np.float32))
    k = gen.f32_to_bf16_bits(g.standard_normal((B, Hkv, T, 128), dtype=np.float32))
    L = np.array(lens if lens else [T] * B, dtype=np.int32)
    imp, perm = S.spa_importance_permutation(dev(q, "bf16"), dev(k, "bf16"), seg, proxy=proxy,
                                             seq_len=None if lens is None else dev(L))
    torch.cuda.synchronize()
    ref = O.key_importance(q, k, "bf16", L, proxy)
    imp_h, perm_h = imp.cpu().numpy(), perm.cpu().numpy()
    imp_close(imp_h, ref)
    for b in range(B):
        assert abs(float(imp_h[b].astype(np.float64).sum()) - 1.0) < 1e-4
        check_importance_perm(perm_h[b], imp_h[b], ref[b], L[b], seg)


@pytest.mark.parametrize("seed", range(10))
def test_scores_random_sweep(seed):
    """Decode scores for random indexer shapes (any rank r that is a multiple of 4, any head count): both kernels."""
    g = np.random.default_rng(5000 + seed)
    H = int(g.integers(1, 17))
    r = 4 * int(g.integers(1, 9))
    if H * r > 1024:
        r = 4 * max(1, 1024 // (4 * H))
    groups = int(g.choice([d for d in range(1, H + 1) if H % d == 0]))
    B, nKb, blk = int(g.integers(1, 5)), int(g.integers(1, 700)), int(g.choice([16, 32, 64, 128]))
    lo = int(g.choice([-128, -8]))
    qI = g.integers(lo, -lo, size=(B, H, r), dtype=np.int8)
    kI = g.integers(lo, -lo, size=(B, nKb, H, r), dtype=np.int8)
    w = g.integers(1, 5, size=(B, H), dtype=np.int8)
    L = g.integers(1, nKb * blk + 1, size=B).astype(np.int32)
    print(f"[random scores] seed {seed}: B={B} H={H} r={r} groups={groups} nKb={nKb} blk={blk}", flush=True)
    got = S.spa_index_score(dev(qI), dev(kI), dev(w), blk, seq_len=dev(L), mode=S.SPA_SCORE_DECODE_GROUPED, Mq=groups)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().astype(np.int64), O.score_decode_grouped(qI, kI, w, L, blk, groups))
    got1 = S.spa_index_score(dev(qI), dev(kI), dev(w), blk, seq_len=dev(L))
    torch.cuda.synchronize()
    assert np.array_equal(got1.cpu().numpy().astype(np.int64), O.score_decode(qI, kI, w, L, blk))


@pytest.mark.parametrize("algo", ["sort", "hist"])
@pytest.mark.parametrize("seed", range(8))
def test_select_ties_random_sweep(seed, algo):
    """Selection on heavily tied scores (a few distinct values): top-k lists exact, top-p by the set rule."""
    g = np.random.default_rng(6000 + seed)
    B, nb, blk = int(g.integers(1, 5)), int(g.integers(8, 2049)), 64
    levels = int(g.choice([1, 2, 3, 5, 17]))
    s = (g.integers(0, levels, size=(B, nb)) * int(g.choice([1, 100, 40000]))).astype(np.int32)
    L = g.integers(1, nb * blk + 1, size=B).astype(np.int32)
    n_sink, n_local = int(g.integers(0, 3)), int(g.integers(0, 5))
    k = int(g.integers(0, nb + 1))
    print(f"[random ties] seed {seed} {algo}: B={B} nb={nb} levels={levels} k={k} sink={n_sink} local={n_local}",
          flush=True)
    idx, cnt = S.spa_select_topk(dev(s), blk, n_sink, n_local, k, max(1, min(nb, n_sink + n_local + k)),
                                 seq_len=dev(L), algo=algo)
    ref, _ = O.select_decode(s.astype(np.int64), L, blk, n_sink, n_local, "topk", k=k)
    assert sel_lists(idx, cnt) == ref
    k_min = int(g.integers(0, 9))
    k_max = int(g.integers(max(1, k_min), nb + 1))
    p, beta = float(g.choice([0.3, 0.9, 1.0])), float(g.choice([0.0, 0.01, 0.125]))
    idx, cnt = S.spa_select_topp(dev(s), blk, n_sink, n_local, beta, p, k_min, k_max,
                                 max(1, min(nb, n_sink + n_local + k_max)), seq_len=dev(L), algo=algo)
    gsel = sel_lists(idx, cnt)
    _, info = O.select_decode(s.astype(np.int64), L, blk, n_sink, n_local, "topp", beta=beta, p=p, k_min=k_min,
                              k_max=k_max)
    for b in range(B):
        check_topp_row(gsel[b], info[b], k_min, k_max, p)


@pytest.mark.parametrize("seed", range(10))
def test_segment_permute_random_sweep(seed):
    """Segment permutation and its inverse on random row sizes (16-byte, 4-byte and byte paths), lengths and segments."""
    g = np.random.default_rng(7000 + seed)
    T = int(g.integers(1, 5001))
    seg = int(g.integers(1, T + 1)) if g.random() < 0.7 else int(g.choice([64, 4096]))
    perm = np.concatenate([s0 + g.permutation(min(seg, T - s0)) for s0 in range(0, T, seg)]).astype(np.int32)
    dt = (np.int8, np.int16, np.float32)[int(g.integers(3))]
    tails = ((128,), (8, 16), (3,), (5, 7), (1,), (33,))
    tail = tails[int(g.integers(len(tails)))]
    outer = tuple(int(x) for x in g.integers(1, 4, size=int(g.integers(0, 3))))
    shape = outer + (T,) + tail
    x = g.integers(-100, 100, size=shape).astype(dt)
    dim = len(outer)
    print(f"[random permute] seed {seed}: shape={shape} dtype={np.dtype(dt).name} seg={seg}", flush=True)
    y = S.spa_segment_permute(dev(x), dev(perm), seg, dim)
    z = S.spa_segment_permute(y, dev(perm), seg, dim, inverse=True)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), O.segment_permute(x, perm, dim))
    assert np.array_equal(z.cpu().numpy(), x)


@pytest.mark.parametrize("seed", range(10))
def test_scores_prefill_random_sweep(seed):
    """Prefill block-pair scores from pooled block vectors (a chunk of query blocks at q_blk0) and from per-token
    vectors with ragged sequence lengths."""
    g = np.random.default_rng(8000 + seed)
    B, H, blk = int(g.integers(1, 4)), int(g.integers(1, 17)), 64
    nKb = int(g.integers(1, 120))
    q_blk0 = int(g.integers(0, nKb))
    M = int(g.integers(1, nKb - q_blk0 + 1))
    lo = int(g.choice([-128, -8]))
    qIb = g.integers(lo, -lo, size=(B, M, H, 16), dtype=np.int8)
    kIb = g.integers(lo, -lo, size=(B, nKb, H, 16), dtype=np.int8)
    w = g.integers(1, 5, size=(B, M, H), dtype=np.int8)
    print(f"[random prefill scores] seed {seed}: B={B} H={H} nKb={nKb} q_blk0={q_blk0} M={M}", flush=True)
    got = S.spa_index_score(dev(qIb), dev(kIb), dev(w), blk, mode=S.SPA_SCORE_PREFILL_POOLED, q_blk0=q_blk0)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().astype(np.int64), O.score_prefill(qIb, kIb, w, q_blk0=q_blk0))
    # per-token vectors of whole blocks, pooled by the library; ragged lengths pool the tokens each block has
    T = nKb * blk
    x = g.integers(lo, -lo, size=(B, T, H, 16), dtype=np.int8)
    wt = g.integers(1, 5, size=(B, nKb, H), dtype=np.int8)
    L = g.integers(1, T + 1, size=B).astype(np.int32)
    s = S.spa_index_score(dev(x), dev(x), dev(wt), blk, seq_len=dev(L), mode=S.SPA_SCORE_PREFILL_TOKENS)
    torch.cuda.synchronize()
    sh = s.cpu().numpy()
    for b in range(B):
        pooled = O.pool_blocks(x[b:b + 1, :L[b]], blk)
        nb = pooled.shape[1]
        ref = O.score_prefill(pooled, pooled, wt[b:b + 1, :nb])
        assert np.array_equal(sh[b:b + 1, :nb, :nb].astype(np.int64), ref)
