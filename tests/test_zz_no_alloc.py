"""spa_sparse_decode_attn_noalloc: the decode attention on the library's own scratch array.

Checked through the C ABI against spa_sparse_decode_attn with a caller workspace on the same
inputs: two calls in a row, the second on a smaller batch (the scratch array keeps the first
call's contents), then an fp32 d = 64 call, each bit-identical to the workspace call (same
kernels, same split) and within the attention tolerance of the fp64 oracle; and a shape whose
workspace exceeds the scratch array is refused before anything is launched.
"""
import numpy as np
import pytest
import torch

import gen
import oracle as O
from gpu_util import attn_close, dev, sel_lists

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    import block_sparse_long_int8_amd as mod
    mod.lib()
    return mod


def _selected(S, cfg, inp, B):
    spec = S.DecodeSpec(B=B, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d, Tcap=cfg.T, blk=cfg.blk, H_idx=cfg.H_idx, r=cfg.r,
                        n_sink=cfg.n_sink, n_local=cfg.n_local, select=cfg.select, k=cfg.k, beta=cfg.beta, p=cfg.p,
                        k_min=cfg.k_min, k_max=cfg.k_max, local_sink_tok=cfg.local_sink_tok,
                        local_window_tok=cfg.local_window_tok)
    step = S.DecodeStep(spec)
    t = dict(q=dev(inp["q"][:B], cfg.dtype), k=dev(inp["k"][:B], cfg.dtype), v=dev(inp["v"][:B], cfg.dtype),
             seq_len=dev(inp["seq_len"][:B]), head_mode=dev(inp["head_mode"]))
    step(t["q"], t["k"], t["v"], dev(inp["qI"][:B]), dev(inp["kI"][:B]), dev(inp["w"][:B]), t["seq_len"],
         t["head_mode"])
    torch.cuda.synchronize()
    return step, t


def _both(S, cfg, inp, B):
    print(f"[no-alloc] {cfg.name}: B={B}", flush=True)
    step, t = _selected(S, cfg, inp, B)
    kw = dict(head_mode=t["head_mode"], local_sink_tok=cfg.local_sink_tok, local_window_tok=cfg.local_window_tok)
    ref, ref_lse = step.out.clone(), step.lse.clone()
    out = torch.full_like(ref, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    S.spa_sparse_decode_attn_noalloc(t["q"], t["k"], t["v"], t["seq_len"], step.idx, step.count, cfg.blk, out=out,
                                     lse=lse, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), "no-alloc output differs from the workspace call"
    assert torch.equal(lse, ref_lse), "no-alloc lse differs from the workspace call"
    sel = sel_lists(step.idx, step.count)
    o_ref, _ = O.decode_attention(inp["q"][:B], inp["k"][:B], inp["v"][:B], cfg.dtype, inp["seq_len"][:B], sel,
                                  cfg.blk, inp["head_mode"], cfg.local_sink_tok, cfg.local_window_tok)
    attn_close(out.cpu().numpy(), o_ref)


def test_no_alloc_matches_workspace_call_twice_then_smaller(S):
    cfg = gen.SMALL_DECODE_TOPP      # B 4, 16 query / 2 KV heads, 8192 tokens, ragged lengths, top-p
    inp = gen.make(cfg)
    _both(S, cfg, inp, cfg.B)
    _both(S, cfg, inp, 2)           # a smaller batch on the scratch the first call filled
    tiny = gen.TINY_DECODE           # fp32, d = 64: the other kernel pair
    _both(S, tiny, gen.make(tiny), tiny.B)


def test_no_alloc_refuses_shapes_beyond_its_scratch(S):
    B, Hq, Hkv, d, Tcap = 256, 64, 8, 128, 64
    assert S.spa_sparse_decode_attn_workspace_size(B, Hq, Hkv, d) > 16 << 20
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((B, Hkv, Tcap, d), dtype=torch.bfloat16, device="cuda")
    seq_len = torch.full((B,), Tcap, dtype=torch.int32, device="cuda")
    idx = torch.zeros((B, 1), dtype=torch.int32, device="cuda")
    count = torch.ones((B,), dtype=torch.int32, device="cuda")
    out = torch.full((B, Hq, d), 7.0, device="cuda")
    with pytest.raises(S.SpaError) as e:
        S.spa_sparse_decode_attn_noalloc(q, kv, kv, seq_len, idx, count, 64, out=out)
    assert e.value.status == S.SPA_ERR_UNSUPPORTED and "scratch" in e.value.detail
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a refused call wrote its output"
