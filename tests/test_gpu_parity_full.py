"""GPU parity at the named workloads' full sizes, in the launch
configuration the benchmark uses.  Decode workloads are checked in full
(the oracle finishes them in seconds); the 64K permuted prefill is checked
bit-exactly on every score and every selected block list, on the first and
last query block of every 4096-token segment for the attention output, and,
run in 8192-token chunks, bit for bit against the one-shot run.
"""
import numpy as np
import pytest
import torch

import gen
import oracle as O
from gpu_util import attn_close, check_importance_perm, check_topp_row, dev, imp_close, sel_lists

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    import block_sparse_long_int8_amd as mod
    mod.lib()
    return mod


def segment_ends(cfg):
    """The first and the last query block of every permutation segment."""
    spb = cfg.seg // cfg.blk
    return sorted({b for s0 in range(0, cfg.nb, spb) for b in (s0, min(cfg.nb, s0 + spb) - 1)})


FULL_DECODE = [gen.TINY_DECODE, gen.DECODE_32K, gen.DECODE_64K_HEADSPLIT, gen.DECODE_128K_TOPP]


@pytest.mark.parametrize("cfg", FULL_DECODE, ids=[c.name for c in FULL_DECODE])
def test_full_decode_parity(S, cfg):
    print(f"[full decode parity] {cfg.name}: generating", flush=True)
    inp = gen.make(cfg)
    spec = S.DecodeSpec(B=cfg.B, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d, Tcap=cfg.T, blk=cfg.blk, H_idx=cfg.H_idx, r=cfg.r,
                        n_sink=cfg.n_sink, n_local=cfg.n_local, select=cfg.select, k=cfg.k, beta=cfg.beta, p=cfg.p,
                        k_min=cfg.k_min, k_max=cfg.k_max, local_sink_tok=cfg.local_sink_tok,
                        local_window_tok=cfg.local_window_tok)
    step = S.DecodeStep(spec)
    q, k, v = dev(inp["q"], cfg.dtype), dev(inp["k"], cfg.dtype), dev(inp["v"], cfg.dtype)
    step(q, k, v, dev(inp["qI"]), dev(inp["kI"]), dev(inp["w"]), dev(inp["seq_len"]), dev(inp["head_mode"]),
         keep_scores=True)
    torch.cuda.synchronize()
    print(f"[full decode parity] {cfg.name}: oracle", flush=True)
    ref = O.decode_step(inp)
    assert np.array_equal(step.scores.cpu().numpy().astype(np.int64), ref["scores"])
    gsel = sel_lists(step.idx, step.count)
    if cfg.select == "topk":
        assert gsel == ref["sel"]
    else:
        for b in range(cfg.B):
            check_topp_row(gsel[b], ref["info"][b], cfg.k_min, cfg.k_max, cfg.p)
    o_ref, lse_ref = O.decode_attention(inp["q"], inp["k"], inp["v"], cfg.dtype, inp["seq_len"], gsel, cfg.blk,
                                        inp["head_mode"], cfg.local_sink_tok, cfg.local_window_tok)
    ma, rl = attn_close(step.out.cpu().numpy(), o_ref)
    print(f"[full decode parity] {cfg.name}: max|d| {ma:.2e} rel-L2 {rl:.2e}", flush=True)
    assert np.allclose(step.lse.cpu().numpy(), lse_ref, atol=1e-4, rtol=1e-5)
    # the same workload with the K/V cache at another address (the benchmark's rotation) is bit-identical
    out0 = step.out.clone()
    step.attend(q, k.clone(), v.clone(), dev(inp["seq_len"]), dev(inp["head_mode"]))
    torch.cuda.synchronize()
    assert torch.equal(out0, step.out)
    # the sort-free selection on the same scores
    if cfg.select == "topk":
        hidx, hcnt = S.spa_select_topk(step.scores, cfg.blk, cfg.n_sink, cfg.n_local, cfg.k, spec.cap,
                                       seq_len=dev(inp["seq_len"]), algo="hist")
        assert sel_lists(hidx, hcnt) == ref["sel"]
    else:
        hidx, hcnt = S.spa_select_topp(step.scores, cfg.blk, cfg.n_sink, cfg.n_local, cfg.beta, cfg.p, cfg.k_min,
                                       cfg.k_max, spec.cap, seq_len=dev(inp["seq_len"]), algo="hist")
        hsel = sel_lists(hidx, hcnt)
        for b in range(cfg.B):
            check_topp_row(hsel[b], ref["info"][b], cfg.k_min, cfg.k_max, cfg.p)
    # the fused scoring + selection launch gives the same scores and selection
    fus = S.DecodeStep(spec, fused=True)
    fus.score_select(dev(inp["qI"]), dev(inp["kI"]), dev(inp["w"]), dev(inp["seq_len"]), keep_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(fus.scores, step.scores)
    assert torch.equal(fus.idx, step.idx) and torch.equal(fus.count, step.count)


def test_full_decode_128k_per_group_parity(S):
    cfg = gen.DECODE_128K_PERGROUP
    print(f"[full decode parity] {cfg.name}: generating", flush=True)
    inp = gen.make(cfg)
    spec = S.DecodeSpec(B=cfg.B, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d, Tcap=cfg.T, blk=cfg.blk, H_idx=cfg.H_idx, r=cfg.r,
                        n_sink=cfg.n_sink, n_local=cfg.n_local, select=cfg.select, k=cfg.k, per_group=True)
    step = S.DecodeStep(spec)
    step(dev(inp["q"], cfg.dtype), dev(inp["k"], cfg.dtype), dev(inp["v"], cfg.dtype), dev(inp["qI"]),
         dev(inp["kI"]), dev(inp["w"]), dev(inp["seq_len"]), dev(inp["head_mode"]))
    torch.cuda.synchronize()
    print(f"[full decode parity] {cfg.name}: oracle", flush=True)
    ref = O.decode_step(inp)
    assert np.array_equal(step.scores.cpu().numpy().astype(np.int64), ref["scores"])
    gsel = sel_lists(step.idx, step.count)
    assert gsel == ref["sel"]
    o_ref, lse_ref = O.decode_attention(inp["q"], inp["k"], inp["v"], cfg.dtype, inp["seq_len"], gsel, cfg.blk,
                                        inp["head_mode"], per_group=True)
    ma, rl = attn_close(step.out.cpu().numpy(), o_ref)
    print(f"[full decode parity] {cfg.name}: max|d| {ma:.2e} rel-L2 {rl:.2e}", flush=True)
    assert np.allclose(step.lse.cpu().numpy(), lse_ref, atol=1e-4, rtol=1e-5)
    # the sort-free selection on the same grouped scores
    hidx, hcnt = S.spa_select_topk(step.scores, cfg.blk, cfg.n_sink, cfg.n_local, cfg.k, spec.cap,
                                   seq_len=dev(inp["seq_len"]), algo="hist")
    assert sel_lists(hidx, hcnt) == ref["sel"]


def test_full_decode_128k_q4_parity(S):
    """The 128K top-p step with the int4 selector cache: quantisation and scores
    bit-exact, selection by the top-p rule, attention on the GPU's lists."""
    cfg = gen.DECODE_128K_TOPP_Q4
    print(f"[full decode parity] {cfg.name}: generating", flush=True)
    inp = gen.make(cfg)
    spec = S.DecodeSpec(B=cfg.B, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d, Tcap=cfg.T, blk=cfg.blk, H_idx=cfg.H_idx, r=cfg.r,
                        n_sink=cfg.n_sink, n_local=cfg.n_local, select=cfg.select, k=cfg.k, beta=cfg.beta, p=cfg.p,
                        k_min=cfg.k_min, k_max=cfg.k_max, selector_q4=True)
    step = S.DecodeStep(spec)
    codes, exps = step.quantize_selector(dev(inp["kI"]))
    step(dev(inp["q"], cfg.dtype), dev(inp["k"], cfg.dtype), dev(inp["v"], cfg.dtype), dev(inp["qI"]),
         (codes, exps), dev(inp["w"]), dev(inp["seq_len"]), dev(inp["head_mode"]))
    torch.cuda.synchronize()
    print(f"[full decode parity] {cfg.name}: oracle", flush=True)
    c_ref, e_ref = O.quantize_selector_keys(inp["kI"])
    assert np.array_equal(exps.cpu().numpy(), e_ref)
    assert np.array_equal(codes.cpu().numpy(), O.pack_int4(c_ref))
    ref = O.decode_step(inp)
    assert np.array_equal(step.scores.cpu().numpy().astype(np.int64), ref["scores"])
    gsel = sel_lists(step.idx, step.count)
    for b in range(cfg.B):
        check_topp_row(gsel[b], ref["info"][b], cfg.k_min, cfg.k_max, cfg.p)
    o_ref, _ = O.decode_attention(inp["q"], inp["k"], inp["v"], cfg.dtype, inp["seq_len"], gsel, cfg.blk,
                                  inp["head_mode"])
    attn_close(step.out.cpu().numpy(), o_ref)


def test_full_prefill_64k_parity(S):
    cfg = gen.PREFILL_64K
    print(f"[full prefill parity] {cfg.name}: generating", flush=True)
    inp = gen.make(cfg)
    step = S.PrefillStep(S.PrefillSpec(B=cfg.B, T=cfg.T, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d, blk=cfg.blk,
                                       H_idx=cfg.H_idx, r=cfg.r, k=cfg.k, n_sink=cfg.n_sink, n_local=cfg.n_local,
                                       seg=cfg.seg))
    out = step(dev(inp["q"], "bf16"), dev(inp["k"], "bf16"), dev(inp["v"], "bf16"), dev(inp["qI_tok"]),
               dev(inp["kI_tok"]), dev(inp["w"]), dev(inp["perm"]))
    torch.cuda.synchronize()
    perm = inp["perm"]
    # the segment permutation at full size: sampled slots of permuted K are the source rows perm[t]
    rows = np.array([0, 1, 4095, 4096, 30000, 65535])
    kp = S.spa_segment_permute(dev(inp["k"], "bf16"), dev(perm), cfg.seg, dim=2)
    torch.cuda.synchronize()
    kp = kp[:, :, rows].cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(kp, inp["k"][:, :, perm[rows]])
    del kp
    print(f"[full prefill parity] {cfg.name}: oracle front end", flush=True)
    front = O.prefill_front(inp)
    assert np.array_equal(step.scores.cpu().numpy().astype(np.int64), front["scores"])
    assert sel_lists(step.idx, step.count) == front["sel"]
    blocks = segment_ends(cfg)
    print(f"[full prefill parity] {cfg.name}: oracle attention on {len(blocks)} blocks (each segment's first and "
          f"last)", flush=True)
    ref = O.prefill_step(inp, front=front, blocks=blocks)
    slots = np.concatenate([np.arange(i * cfg.blk, (i + 1) * cfg.blk) for i in blocks])
    # the query in slot t is written at its original position perm[t]
    o_g = out[:, :, torch.from_numpy(perm[slots]).long().cuda()].cpu().numpy()
    attn_close(o_g, ref["o_slot"][:, :, slots])
    lse_g = step.lse[:, :, torch.from_numpy(perm[slots]).long().cuda()].cpu().numpy()
    assert np.allclose(lse_g, ref["lse_slot"][:, :, slots], atol=1e-4, rtol=1e-5)


def test_full_prefill_64k_importance_parity(S):
    """The importance-permuted 64K prefill: importances against fp64, the
    permutation by the near-tie rule, then every score and block list, and
    sampled attention blocks, downstream of that permutation."""
    cfg = gen.PREFILL_64K_IMPORTANCE
    print(f"[full prefill parity] {cfg.name}: generating", flush=True)
    inp = gen.make(cfg)
    step = S.PrefillStep(S.PrefillSpec(B=cfg.B, T=cfg.T, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d, blk=cfg.blk,
                                       H_idx=cfg.H_idx, r=cfg.r, k=cfg.k, n_sink=cfg.n_sink, n_local=cfg.n_local,
                                       seg=cfg.seg, perm_kind="importance", proxy=cfg.proxy))
    out = step(dev(inp["q"], "bf16"), dev(inp["k"], "bf16"), dev(inp["v"], "bf16"), dev(inp["qI_tok"]),
               dev(inp["kI_tok"]), dev(inp["w"]))
    torch.cuda.synchronize()
    print(f"[full prefill parity] {cfg.name}: oracle importance", flush=True)
    imp_ref = O.key_importance(inp["q"], inp["k"], cfg.dtype, inp["seq_len"], cfg.proxy)
    imp_g = step.imp.cpu().numpy()
    imp_close(imp_g, imp_ref)
    perm_g = step.perm.cpu().numpy()[0]
    differ = check_importance_perm(perm_g, imp_g[0], imp_ref[0], cfg.T, cfg.seg)
    perm_ref = O.importance_permutation(imp_ref, inp["seq_len"], cfg.seg)[0]
    print(f"[full prefill parity] {cfg.name}: {differ} positions differ from the oracle order", flush=True)
    use = perm_ref if differ == 0 else perm_g
    inp2 = dict(inp, perm=use.astype(np.int32))
    print(f"[full prefill parity] {cfg.name}: oracle front end", flush=True)
    front = O.prefill_front(inp2)
    assert np.array_equal(step.scores.cpu().numpy().astype(np.int64), front["scores"])
    assert sel_lists(step.idx, step.count) == front["sel"]
    blocks = segment_ends(cfg)
    print(f"[full prefill parity] {cfg.name}: oracle attention on {len(blocks)} blocks", flush=True)
    ref = O.prefill_step(inp2, front=front, blocks=blocks)
    slots = np.concatenate([np.arange(i * cfg.blk, (i + 1) * cfg.blk) for i in blocks])
    rows = torch.from_numpy(use[slots].astype(np.int64)).cuda()
    attn_close(out[:, :, rows].cpu().numpy(), ref["o_slot"][:, :, slots])
    assert np.allclose(step.lse[:, :, rows].cpu().numpy(), ref["lse_slot"][:, :, slots], atol=1e-4, rtol=1e-5)


def test_full_prefill_64k_chunked_equals_one_shot(S):
    """The 64K permuted prefill run as a chunked prefill, 8 chunks of 8192 tokens (each chunk
    scores, selects and attends its query blocks against the key blocks before them),
    equals the one-shot run bit for bit: scores, block lists, O and lse."""
    cfg = gen.PREFILL_64K
    print(f"[full prefill chunked] {cfg.name}: generating", flush=True)
    inp = gen.make(cfg)
    t = [dev(inp["q"], "bf16"), dev(inp["k"], "bf16"), dev(inp["v"], "bf16"), dev(inp["qI_tok"]),
         dev(inp["kI_tok"]), dev(inp["w"]), dev(inp["perm"])]

    def spec(chunk):
        return S.PrefillSpec(B=cfg.B, T=cfg.T, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d, blk=cfg.blk, H_idx=cfg.H_idx, r=cfg.r,
                             k=cfg.k, n_sink=cfg.n_sink, n_local=cfg.n_local, seg=cfg.seg, chunk=chunk)
    one = S.PrefillStep(spec(0))
    one(*t)
    torch.cuda.synchronize()
    print(f"[full prefill chunked] {cfg.name}: one shot done, 8 chunks next", flush=True)
    ch = S.PrefillStep(spec(8192))
    assert len(ch.chunks) == 8
    ch(*t)
    torch.cuda.synchronize()
    assert torch.equal(ch.scores, one.scores)
    assert torch.equal(ch.idx, one.idx) and torch.equal(ch.count, one.count)
    assert torch.equal(ch.out, one.out)
    assert torch.equal(ch.lse, one.lse)
