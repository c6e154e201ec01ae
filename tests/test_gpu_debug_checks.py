"""Device-side checks of the values inside device arrays (spa_set_debug_checks).

With the checks on, every call validates its block lists, sequence lengths,
positions, head modes and permutations on the device before its own kernels
run, and returns SPA_ERR_INVALID_ARG (launching nothing else) on a violation.
Every corrupted input here is chosen so that, even if a check missed it, the
call's kernels would still read and write inside the test's buffers: blocks
that exist in the cache, rows that fall in the next (sequence, head) slab of a
batch of two, values within [0, T).
"""
import dataclasses

import numpy as np
import pytest
import torch

import gen
from gpu_util import dev

pytestmark = pytest.mark.gpu

S = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global S
    import block_sparse_long_int8_amd as mod
    mod.lib()
    S = mod
    yield


@pytest.fixture()
def checks():
    S.spa_set_debug_checks(True)
    try:
        yield
    finally:
        S.spa_set_debug_checks(False)


def _expect(code, fn, *args, **kw):
    with pytest.raises(S.SpaError) as e:
        fn(*args, **kw)
    torch.cuda.synchronize()
    assert e.value.status == S.SPA_ERR_INVALID_ARG, e.value
    assert "device-side check" in e.value.detail, e.value.detail
    assert S.spa_debug_error() == code, (S.spa_debug_error(), e.value.detail)


def _decode_setup():
    cfg = gen.SMALL_DECODE_HEADSPLIT  # B 2, Hkv 4, Tcap 8192, seq_len (8192, 5001), two local KV heads
    inp = gen.make(cfg)
    t = dict(q=dev(inp["q"], cfg.dtype), k=dev(inp["k"], cfg.dtype), v=dev(inp["v"], cfg.dtype),
             qI=dev(inp["qI"]), kI=dev(inp["kI"]), w=dev(inp["w"]), seq_len=dev(inp["seq_len"]),
             head_mode=dev(inp["head_mode"]))
    spec = S.DecodeSpec(B=cfg.B, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d, Tcap=cfg.T, blk=cfg.blk, H_idx=cfg.H_idx, r=cfg.r,
                        n_sink=cfg.n_sink, n_local=cfg.n_local, select=cfg.select, k=cfg.k, beta=cfg.beta, p=cfg.p,
                        k_min=cfg.k_min, k_max=cfg.k_max, local_sink_tok=cfg.local_sink_tok,
                        local_window_tok=cfg.local_window_tok)
    return cfg, inp, t, spec


def _attn(cfg, t, idx, count, seq_len=None, head_mode=None, grouped=False, out=None):
    f = S.spa_sparse_decode_attn_grouped if grouped else S.spa_sparse_decode_attn
    return f(t["q"], t["k"], t["v"], t["seq_len"] if seq_len is None else seq_len, idx, count, cfg.blk,
             head_mode=t["head_mode"] if head_mode is None else head_mode, local_sink_tok=cfg.local_sink_tok,
             local_window_tok=cfg.local_window_tok, out=out)


def test_valid_calls_pass_and_match_unchecked():
    cfg, inp, t, spec = _decode_setup()
    args = (t["q"], t["k"], t["v"], t["qI"], t["kI"], t["w"], t["seq_len"], t["head_mode"])
    step = S.DecodeStep(spec)
    step(*args)
    torch.cuda.synchronize()
    ref = step.out.clone()
    S.spa_set_debug_checks(True)
    try:
        step(*args)
        torch.cuda.synchronize()
        assert S.spa_debug_error() == S.SPA_DBG_NONE
        assert torch.equal(step.out, ref)
        pcfg = gen.SMALL_PREFILL
        pin = gen.make(pcfg)
        pt = [dev(pin["q"], "bf16"), dev(pin["k"], "bf16"), dev(pin["v"], "bf16"), dev(pin["qI_tok"]),
              dev(pin["kI_tok"]), dev(pin["w"]), dev(pin["perm"])]
        pstep = S.PrefillStep(S.PrefillSpec(B=pcfg.B, T=pcfg.T, Hq=pcfg.Hq, Hkv=pcfg.Hkv, d=pcfg.d, blk=pcfg.blk,
                                            H_idx=pcfg.H_idx, r=pcfg.r, k=pcfg.k, n_sink=pcfg.n_sink,
                                            n_local=pcfg.n_local, seg=pcfg.seg))
        checked = pstep(*pt).clone()
    finally:
        S.spa_set_debug_checks(False)
    unchecked = pstep(*pt)
    torch.cuda.synchronize()
    assert torch.equal(checked, unchecked)


def test_decode_list_violations(checks):
    cfg, inp, t, spec = _decode_setup()
    step = S.DecodeStep(spec)
    step(t["q"], t["k"], t["v"], t["qI"], t["kI"], t["w"], t["seq_len"], t["head_mode"])
    torch.cuda.synchronize()
    idx, count = step.idx.clone(), step.count.clone()
    cnt = count.cpu().numpy()
    out = torch.full((cfg.B, cfg.Hq, cfg.d), float("nan"), device="cuda")
    # block 79 is one past the last block of sequence 1 (5001 tokens), still inside the cache
    bad = idx.clone()
    last = int(cnt[1]) - 1
    assert int(bad[1, last]) == 78
    bad[1, last] = 79
    _expect(S.SPA_DBG_IDX_RANGE, _attn, cfg, t, bad, count, out=out)
    assert torch.isnan(out).all(), "nothing may run after a failed check"
    # two entries swapped
    bad = idx.clone()
    bad[0, 0], bad[0, 1] = idx[0, 1], idx[0, 0]
    _expect(S.SPA_DBG_IDX_ORDER, _attn, cfg, t, bad, count, out=out)
    # a sequence length past the cache (sequence 0: a window past its end lies in the next slab)
    sl = t["seq_len"].clone()
    sl[0] = cfg.T + 1
    _expect(S.SPA_DBG_SEQ_LEN, _attn, cfg, t, idx, count, seq_len=sl, out=out)
    hm = t["head_mode"].clone()
    hm[1] = 2
    _expect(S.SPA_DBG_HEAD_MODE, _attn, cfg, t, idx, count, head_mode=hm, out=out)
    # a valid call clears the code and runs
    _attn(cfg, t, idx, count, out=out)
    torch.cuda.synchronize()
    assert S.spa_debug_error() == S.SPA_DBG_NONE
    assert torch.isfinite(out).all()
    # count above cap on row 0 (its extra entries would be row 1's valid blocks)
    bad_c = count.clone()
    bad_c[0] = idx.shape[1] + 1
    out.fill_(float("nan"))
    _expect(S.SPA_DBG_COUNT, _attn, cfg, t, idx, bad_c, out=out)
    assert torch.isnan(out).all()


def test_grouped_rows_use_their_sequence(checks):
    cfg, inp, t, spec = _decode_setup()
    step = S.DecodeStep(spec)
    step(t["q"], t["k"], t["v"], t["qI"], t["kI"], t["w"], t["seq_len"], t["head_mode"])
    torch.cuda.synchronize()
    g_idx = step.idx[:, None, :].expand(cfg.B, cfg.Hkv, -1).contiguous()
    g_cnt = step.count[:, None].expand(cfg.B, cfg.Hkv).contiguous()
    _attn(cfg, t, g_idx, g_cnt, grouped=True)
    torch.cuda.synchronize()
    assert S.spa_debug_error() == S.SPA_DBG_NONE
    # row (1, 3) is sequence 1's: block 79 is past its 5001 tokens though below sequence 0's length
    bad = g_idx.clone()
    last = int(g_cnt[1, 3]) - 1
    bad[1, 3, last] = 79
    _expect(S.SPA_DBG_IDX_RANGE, _attn, cfg, t, bad, g_cnt, grouped=True)


def test_score_and_select_seq_len(checks):
    cfg = gen.SMALL_DECODE_TOPP  # B 4, nKb 128
    inp = gen.make(cfg)
    qI, kI, w = dev(inp["qI"]), dev(inp["kI"]), dev(inp["w"])
    sl = dev(inp["seq_len"])
    scores = S.spa_index_score(qI, kI, w, cfg.blk, seq_len=sl)
    torch.cuda.synchronize()
    bad = sl.clone()
    bad[0] = cfg.T + 1
    _expect(S.SPA_DBG_SEQ_LEN, S.spa_index_score, qI, kI, w, cfg.blk, seq_len=bad)
    cap = cfg.n_sink + cfg.n_local + cfg.k_max
    S.spa_select_topp(scores, cfg.blk, cfg.n_sink, cfg.n_local, cfg.beta, cfg.p, cfg.k_min, cfg.k_max, cap,
                      seq_len=sl)
    torch.cuda.synchronize()
    _expect(S.SPA_DBG_SEQ_LEN, S.spa_select_topp, scores, cfg.blk, cfg.n_sink, cfg.n_local, cfg.beta, cfg.p,
            cfg.k_min, cfg.k_max, cap, seq_len=bad)


def test_prefill_positions_and_lists(checks):
    cfg = dataclasses.replace(gen.SMALL_PREFILL, name="small_prefill_b2_bf16", cfg_id=61, B=2)
    inp = gen.make(cfg)
    q, k, v = dev(inp["q"], "bf16"), dev(inp["k"], "bf16"), dev(inp["v"], "bf16")
    perm = dev(inp["perm"])
    step = S.PrefillStep(S.PrefillSpec(B=cfg.B, T=cfg.T, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d, blk=cfg.blk,
                                       H_idx=cfg.H_idx, r=cfg.r, k=cfg.k, n_sink=cfg.n_sink, n_local=cfg.n_local,
                                       seg=cfg.seg))
    step(q, k, v, dev(inp["qI_tok"]), dev(inp["kI_tok"]), dev(inp["w"]), perm)
    torch.cuda.synchronize()
    pos, idx, count = step.pos, step.idx, step.count
    T = cfg.T

    def call(qp=pos, kp=pos, ix=idx, order="original", kv_order="original"):
        return S.spa_block_sparse_prefill(q, k, v, ix, count, cfg.blk, q_pos=qp, k_pos=kp, order=order,
                                          kv_order=kv_order)

    bad = pos.clone()
    bad[0, 5] = T  # row T of sequence 0 is the first row of the next slab
    _expect(S.SPA_DBG_K_POS, call, kp=bad, qp=pos.clone())
    _expect(S.SPA_DBG_Q_POS, call, qp=bad, kp=pos.clone())
    # in slot order the positions only mask: not row numbers, not checked
    call(qp=pos, kp=bad, order="slot", kv_order="slot")
    torch.cuda.synchronize()
    assert S.spa_debug_error() == S.SPA_DBG_NONE
    bad_i = idx.clone()
    nb = cfg.nb
    last = int(count[0, nb - 1]) - 1
    assert int(bad_i[0, nb - 1, last]) == nb - 1
    bad_i[0, nb - 1, last] = nb  # one past the last key block (the kernel clamps rows to T-1)
    _expect(S.SPA_DBG_IDX_RANGE, call, ix=bad_i)


def test_permutation_violations(checks):
    T, seg = 2048, 512
    src = torch.arange(T * 8, dtype=torch.int32, device="cuda").reshape(1, T, 8)
    g = np.random.default_rng(5)
    perm = np.concatenate([s0 + g.permutation(seg) for s0 in range(0, T, seg)]).astype(np.int32)
    out = S.spa_segment_permute(src, dev(perm), seg, dim=1)
    torch.cuda.synchronize()
    assert S.spa_debug_error() == S.SPA_DBG_NONE
    assert torch.equal(out[0].cpu(), src[0].cpu()[torch.from_numpy(perm).long()])
    bad = perm.copy()
    bad[600] = 10  # a row of segment 0 placed in segment 1
    _expect(S.SPA_DBG_PERM_RANGE, S.spa_segment_permute, src, dev(bad), seg, dim=1)
    bad = perm.copy()
    bad[1030] = bad[1031]  # a repeat inside segment 2
    _expect(S.SPA_DBG_PERM_DUP, S.spa_segment_permute, src, dev(bad), seg, dim=1)


def test_checked_call_refuses_graph_capture(checks):
    cfg, inp, t, spec = _decode_setup()
    step = S.DecodeStep(spec)
    step(t["q"], t["k"], t["v"], t["qI"], t["kI"], t["w"], t["seq_len"], t["head_mode"])
    torch.cuda.synchronize()
    out = torch.empty((cfg.B, cfg.Hq, cfg.d), device="cuda")
    lse = torch.empty((cfg.B, cfg.Hq), device="cuda")
    ws = torch.empty(S.spa_sparse_decode_attn_workspace_size(cfg.B, cfg.Hq, cfg.Hkv, cfg.d), dtype=torch.uint8,
                     device="cuda")
    g = torch.cuda.CUDAGraph()
    with pytest.raises(S.SpaError) as e:
        with torch.cuda.graph(g):
            S.spa_sparse_decode_attn(t["q"], t["k"], t["v"], t["seq_len"], step.idx, step.count, cfg.blk,
                                     head_mode=t["head_mode"], local_sink_tok=cfg.local_sink_tok,
                                     local_window_tok=cfg.local_window_tok, out=out, lse=lse, ws=ws)
    assert e.value.status == S.SPA_ERR_INVALID_ARG
    assert "captured" in e.value.detail
    torch.cuda.synchronize()


def test_pooling_positions(checks):
    # tok_pos gathers the per-token indexer vectors; row T of sequence 0 is row 0 of sequence 1
    rng = np.random.default_rng(3)
    B, nb, blk, H = 2, 8, 64, 8
    T = nb * blk
    x = dev(rng.integers(-128, 128, size=(B, T, H, 16), dtype=np.int8))
    w = dev(rng.integers(1, 5, size=(B, nb, H), dtype=np.int8))
    pos = np.tile(np.arange(T, dtype=np.int32), (B, 1))
    S.spa_index_score(x, x, w, blk, mode=S.SPA_SCORE_PREFILL_TOKENS, tok_pos=dev(pos))
    torch.cuda.synchronize()
    assert S.spa_debug_error() == S.SPA_DBG_NONE
    bad = pos.copy()
    bad[0, 100] = T
    _expect(S.SPA_DBG_TOK_POS, S.spa_index_score, x, x, w, blk, mode=S.SPA_SCORE_PREFILL_TOKENS, tok_pos=dev(bad))
