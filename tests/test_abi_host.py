"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects invalid arguments before touching the GPU.  No GPU needed.
"""
import ctypes

import pytest

import torch

import block_sparse_long_int8_amd as S

# These calls pass fake host addresses that must be rejected before any launch.
# They are host-logic tests: never run them where a GPU could execute a launch.
pytestmark = pytest.mark.skipif(torch.cuda.is_available(), reason="fake-pointer rejection tests are host-only")

L = S.lib()
N = None


def test_exports_every_declared_symbol():
    names = S.declared_symbols()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    assert L.spa_status_string(0) == b"SPA_OK"
    assert L.spa_status_string(-1) == b"SPA_ERR_INVALID_ARG"
    assert L.spa_status_string(-4) == b"SPA_ERR_HIP"
    assert L.spa_version() >= 100


def _fake(n=1):
    # aligned non-null host addresses: validation must fail before any dereference
    return ctypes.c_void_p(0x1000 * n)


def test_index_score_rejections():
    f = L.spa_index_score
    assert f(_fake(), _fake(2), _fake(3), 1, 8, 16, 1, 10, 0, _fake(4), N, 64, 7, _fake(5), N, 0, N) == S.SPA_ERR_INVALID_ARG
    assert b"unknown mode" in L.spa_last_error()
    assert f(_fake(), _fake(2), _fake(3), 1, 8, 15, 1, 10, 0, _fake(4), N, 64, 0, _fake(5), N, 0, N) == S.SPA_ERR_INVALID_ARG
    assert f(_fake(), _fake(2), _fake(3), 1, 128, 16, 1, 10, 0, _fake(4), N, 64, 0, _fake(5), N, 0, N) == S.SPA_ERR_INVALID_ARG
    assert f(_fake(), _fake(2), _fake(3), 1, 8, 16, 2, 10, 0, _fake(4), N, 64, 0, _fake(5), N, 0, N) == S.SPA_ERR_INVALID_ARG
    assert f(N, _fake(2), _fake(3), 1, 8, 16, 1, 10, 0, _fake(4), N, 64, 0, _fake(5), N, 0, N) == S.SPA_ERR_INVALID_ARG
    assert f(_fake(), _fake(2), _fake(3), 1, 8, 16, 1, 10, 0, N, N, 64, 0, _fake(5), N, 0, N) == S.SPA_ERR_INVALID_ARG
    # misaligned kI
    assert f(_fake(), ctypes.c_void_p(0x2004), _fake(3), 1, 8, 16, 1, 10, 0, _fake(4), N, 64, 0, _fake(5), N, 0, N) == S.SPA_ERR_INVALID_ARG
    # prefill needs r == 16
    assert f(_fake(), _fake(2), _fake(3), 1, 8, 8, 4, 10, 0, N, N, 64, 1, _fake(5), N, 0, N) == S.SPA_ERR_UNSUPPORTED
    # per-token prefill without workspace
    assert f(_fake(), _fake(2), _fake(3), 1, 8, 16, 4, 10, 0, N, N, 64, 2, _fake(5), N, 0, N) == S.SPA_ERR_WORKSPACE
    # grouped decode: the groups must divide H_idx
    assert f(_fake(), _fake(2), _fake(3), 1, 8, 16, 3, 10, 0, _fake(4), N, 64, 3, _fake(5), N, 0, N) == S.SPA_ERR_INVALID_ARG
    assert b"groups" in L.spa_last_error()
    assert f(_fake(), _fake(2), _fake(3), 1, 8, 16, 0, 10, 0, _fake(4), N, 64, 3, _fake(5), N, 0, N) == S.SPA_ERR_INVALID_ARG
    assert f(_fake(), _fake(2), _fake(3), 1, 8, 16, 4, 10, 0, N, N, 64, 3, _fake(5), N, 0, N) == S.SPA_ERR_INVALID_ARG
    # empty batch is a valid no-op
    assert f(N, N, N, 0, 8, 16, 1, 10, 0, N, N, 64, 0, N, N, 0, N) == S.SPA_OK
    assert L.spa_index_score_workspace_size(1, 8, 16, 1024, 1024, 2) == 2 * 1024 * 128
    assert L.spa_index_score_workspace_size(1, 8, 16, 1024, 1024, 0) == 0
    # tok_pos: per-token prefill only, without seq_len, chunk inside the key blocks
    assert f(_fake(), _fake(2), _fake(3), 1, 8, 16, 1, 10, 0, _fake(4), _fake(6), 64, 0, _fake(5), N, 0, N) == S.SPA_ERR_INVALID_ARG
    assert b"tok_pos" in L.spa_last_error()
    assert f(_fake(), _fake(2), _fake(3), 1, 8, 16, 4, 10, 0, _fake(4), _fake(6), 64, 2, _fake(5), N, 0, N) == S.SPA_ERR_UNSUPPORTED
    assert f(_fake(), _fake(2), _fake(3), 1, 8, 16, 4, 10, 7, N, _fake(6), 64, 2, _fake(5), N, 0, N) == S.SPA_ERR_INVALID_ARG
    assert b"exceed nKb" in L.spa_last_error()
    assert f(_fake(), _fake(2), _fake(3), 1, 8, 16, 4, 10, 6, N, _fake(6), 64, 2, _fake(5), N, 0, N) == S.SPA_ERR_WORKSPACE


@pytest.mark.parametrize("suffix", ["", "_hist"])
def test_select_rejections(suffix):
    tk = getattr(L, "spa_select_topk" + suffix)
    # cap smaller than reserved + k
    assert tk(_fake(), 1, 1, 100, 0, _fake(2), 64, 1, 4, 0, 64, _fake(3), _fake(4), 68, N, 0, N) == S.SPA_ERR_INVALID_ARG
    assert b"cap" in L.spa_last_error()
    # ... but no row lists more than nKb blocks: with 50 blocks, cap 50 is enough (B = 0: validated, nothing launched)
    assert tk(_fake(), 0, 1, 50, 0, _fake(2), 64, 1, 4, 0, 64, _fake(3), _fake(4), 49, N, 0, N) == S.SPA_ERR_INVALID_ARG
    assert tk(_fake(), 0, 1, 50, 0, _fake(2), 64, 1, 4, 0, 64, _fake(3), _fake(4), 50, N, 0, N) == S.SPA_OK
    # decode rows need seq_len
    assert tk(_fake(), 1, 1, 100, 0, N, 64, 1, 4, 0, 8, _fake(3), _fake(4), 13, N, 0, N) == S.SPA_ERR_INVALID_ARG
    assert tk(_fake(), 1, 8, 100, 0, N, 64, 1, 4, 0, 8, _fake(3), _fake(4), 13, N, 0, N) == S.SPA_ERR_INVALID_ARG
    assert tk(_fake(), 1, 1, 5000, 0, _fake(2), 64, 1, 4, 0, 8, _fake(3), _fake(4), 13, N, 0, N) == S.SPA_ERR_UNSUPPORTED
    assert tk(_fake(), 1, 1, 100, 0, _fake(2), 64, 1, 4, 0, -1, _fake(3), _fake(4), 13, N, 0, N) == S.SPA_ERR_INVALID_ARG
    tp = getattr(L, "spa_select_topp" + suffix)
    assert tp(_fake(), 1, 1, 100, 0, _fake(2), 64, 1, 4, 0, 0.125, 1.5, 16, 512, _fake(3), _fake(4), 517, N, 0, N) == S.SPA_ERR_INVALID_ARG
    assert tp(_fake(), 1, 1, 100, 0, _fake(2), 64, 1, 4, 0, 0.125, 0.9, 32, 16, _fake(3), _fake(4), 517, N, 0, N) == S.SPA_ERR_INVALID_ARG
    assert tp(_fake(), 1, 1, 100, 0, _fake(2), 64, 1, 4, 0, float("nan"), 0.9, 16, 512, _fake(3), _fake(4), 517, N, 0, N) == S.SPA_ERR_INVALID_ARG
    assert tp(_fake(), 1, 1, 1000, 0, _fake(2), 64, 1, 4, 0, 0.125, 0.9, 16, 512, _fake(3), _fake(4), 516, N, 0, N) == S.SPA_ERR_INVALID_ARG
    assert tp(N, 0, 1, 100, 0, N, 64, 1, 4, 0, 0.125, 0.9, 16, 512, N, N, 517, N, 0, N) == S.SPA_OK
    # null scores with a batch to select
    assert tk(N, 1, 1, 100, 0, _fake(2), 64, 1, 4, 0, 8, _fake(3), _fake(4), 13, N, 0, N) == S.SPA_ERR_INVALID_ARG


@pytest.mark.parametrize("name", ["spa_sparse_decode_attn", "spa_sparse_decode_attn_grouped"])
def test_decode_attn_rejections(name):
    f = getattr(L, name)
    args = dict(q=_fake(), k=_fake(2), v=_fake(3), io=S.SPA_BF16, sl=_fake(4), idx=_fake(5), cnt=_fake(6), cap=69,
                blk=64, hm=N, ns=0, nw=0, B=1, Hq=32, Hkv=8, d=128, T=32768, scale=0.088, out=_fake(7),
                od=S.SPA_F32, lse=N, ws=_fake(8), wsb=1 << 30, st=N)

    def call(**kw):
        a = dict(args, **kw)
        return f(*a.values())

    assert call(d=96) == S.SPA_ERR_UNSUPPORTED                 # d in {64, 128}
    assert call(Hq=30) == S.SPA_ERR_INVALID_ARG                # not a multiple of Hkv
    assert call(Hq=8 * 17) == S.SPA_ERR_UNSUPPORTED             # G > 16
    assert call(blk=48) == S.SPA_ERR_UNSUPPORTED
    assert call(io=5) == S.SPA_ERR_INVALID_ARG
    assert call(od=9) == S.SPA_ERR_INVALID_ARG
    assert call(scale=float("inf")) == S.SPA_ERR_INVALID_ARG
    assert call(idx=N) == S.SPA_ERR_INVALID_ARG
    assert call(ws=N) == S.SPA_ERR_WORKSPACE
    assert call(wsb=16) == S.SPA_ERR_WORKSPACE
    assert call(q=ctypes.c_void_p(0x1008)) == S.SPA_ERR_INVALID_ARG
    assert call(B=0) == S.SPA_OK
    assert call(io=S.SPA_F32, d=96) == S.SPA_ERR_UNSUPPORTED


def test_prefill_and_permute_rejections():
    f = L.spa_block_sparse_prefill
    base = [_fake(), 0, 4096, _fake(2), _fake(3), N, N, _fake(4), _fake(5), 34, 64, 1, 32, 8, 128, 4096, 0.088,
            _fake(6), S.SPA_F32, N, S.SPA_ORDER_SLOT, N, 0, N]
    b = list(base); b[20] = 4
    assert f(*b) == S.SPA_ERR_INVALID_ARG                      # unknown row-order flag
    b = list(base); b[20] = -1
    assert f(*b) == S.SPA_ERR_INVALID_ARG
    b = list(base); b[10] = 32
    assert f(*b) == S.SPA_ERR_UNSUPPORTED                      # blk must be 64
    b = list(base); b[14] = 64
    assert f(*b) == S.SPA_ERR_UNSUPPORTED                      # d must be 128
    b = list(base); b[1] = 10
    assert f(*b) == S.SPA_ERR_INVALID_ARG                      # query slots past T
    b = list(base); b[0] = N
    assert f(*b) == S.SPA_ERR_INVALID_ARG
    b = list(base); b[2] = 0
    assert f(*b) == S.SPA_OK                                   # empty chunk
    p = L.spa_segment_permute
    assert p(_fake(), _fake(2), 4, 100, 256, _fake(3), 64, 2, N) == S.SPA_ERR_INVALID_ARG
    assert p(_fake(), _fake(), 4, 100, 256, _fake(3), 64, 0, N) == S.SPA_ERR_INVALID_ARG   # overlap
    assert p(_fake(), _fake(2), 4, 100, 256, N, 64, 0, N) == S.SPA_ERR_INVALID_ARG
    assert p(N, N, 0, 100, 256, N, 64, 0, N) == S.SPA_OK


def test_score_select_rejections():
    f = L.spa_score_select_decode
    base = [_fake(), _fake(2), _fake(3), 1, 8, 16, 100, _fake(4), 64, 1, 4, 1, 0, 0.125, 0.9, 16, 64, N, _fake(5),
            _fake(6), 85, N]
    b = list(base); b[11] = 3
    assert f(*b) == S.SPA_ERR_INVALID_ARG                      # mode
    b = list(base); b[5] = 8
    assert f(*b) == S.SPA_ERR_UNSUPPORTED                      # r must be 16
    b = list(base); b[4] = 65
    assert f(*b) == S.SPA_ERR_UNSUPPORTED                      # H_idx <= 64
    b = list(base); b[20] = 68
    assert f(*b) == S.SPA_ERR_INVALID_ARG                      # cap < 1 + 4 + k_max
    b = list(base); b[1] = N
    assert f(*b) == S.SPA_ERR_INVALID_ARG
    b = list(base); b[7] = N
    assert f(*b) == S.SPA_ERR_INVALID_ARG                      # decode rows need seq_len
    b = list(base); b[3] = 0
    assert f(*b) == S.SPA_OK                                   # empty batch


def test_importance_permutation_rejections():
    f = L.spa_importance_permutation
    base = dict(q=_fake(), k=_fake(2), B=1, Hq=32, Hkv=8, T=4096, d=128, sl=N, proxy=64, scale=0.088, seg=4096,
                imp=_fake(3), perm=_fake(4), ws=_fake(5), wsb=1 << 30, st=N)

    def call(**kw):
        a = dict(base, **kw)
        return f(*a.values())

    assert call(d=64) == S.SPA_ERR_UNSUPPORTED
    assert call(proxy=65) == S.SPA_ERR_UNSUPPORTED
    assert call(proxy=0) == S.SPA_ERR_INVALID_ARG
    assert call(seg=8192) == S.SPA_ERR_UNSUPPORTED
    assert call(seg=0) == S.SPA_ERR_INVALID_ARG
    assert call(Hq=30) == S.SPA_ERR_INVALID_ARG
    assert call(scale=float("nan")) == S.SPA_ERR_INVALID_ARG
    assert call(scale=-0.5) == S.SPA_ERR_INVALID_ARG
    assert call(ws=N) == S.SPA_ERR_WORKSPACE
    assert call(wsb=1024) == S.SPA_ERR_WORKSPACE
    assert call(perm=N) == S.SPA_ERR_INVALID_ARG
    assert call(k=ctypes.c_void_p(0x2008)) == S.SPA_ERR_INVALID_ARG
    assert call(B=0) == S.SPA_OK
    assert L.spa_importance_permutation_workspace_size(1, 32, 65536) >= 32 * 65536 * 4


def test_int4_selector_rejections():
    q = L.spa_quantize_selector_keys
    assert q(_fake(), 10, 8, _fake(2), _fake(3), N) == S.SPA_ERR_UNSUPPORTED
    assert q(_fake(), -1, 16, _fake(2), _fake(3), N) == S.SPA_ERR_INVALID_ARG
    assert q(N, 10, 16, _fake(2), _fake(3), N) == S.SPA_ERR_INVALID_ARG
    assert q(N, 0, 16, N, N, N) == S.SPA_OK
    f = L.spa_index_score_q4
    base = [_fake(), _fake(2), _fake(3), _fake(4), 1, 8, 16, 1, 100, _fake(5), 64, 0, _fake(6), N]
    b = list(base); b[11] = 1                     # prefill modes are not supported
    assert f(*b) == S.SPA_ERR_INVALID_ARG
    b = list(base); b[5] = 64                     # H_idx above 32 could overflow
    assert f(*b) == S.SPA_ERR_UNSUPPORTED
    b = list(base); b[5] = 6
    assert f(*b) == S.SPA_ERR_UNSUPPORTED
    b = list(base); b[7] = 2                      # decode mode needs Mq == 1
    assert f(*b) == S.SPA_ERR_INVALID_ARG
    b = list(base); b[11] = 3; b[7] = 3           # groups must divide H_idx
    assert f(*b) == S.SPA_ERR_INVALID_ARG
    b = list(base); b[9] = N                      # seq_len is required
    assert f(*b) == S.SPA_ERR_INVALID_ARG
    b = list(base); b[4] = 0
    assert f(*b) == S.SPA_OK


def test_debug_check_switch_and_codes():
    # the switch is process-wide state; the codes match the header
    was = L.spa_debug_checks()
    try:
        S.spa_set_debug_checks(True)
        assert S.spa_debug_checks()
        S.spa_set_debug_checks(False)
        assert not S.spa_debug_checks()
    finally:
        L.spa_set_debug_checks(was)
    assert L.spa_debug_error() == S.SPA_DBG_NONE
    import re
    with open(S.declared_symbols.__globals__["HEADER"]) as f:
        text = f.read()
    for name, val in re.findall(r"#define (SPA_DBG_\w+) (\d+)", text):
        assert getattr(S, name) == int(val), name


def test_probe_rejections():
    bad = ctypes.c_void_p(0x1001)  # misaligned
    # spa_probe_read(buf, bytes, workgroups, sink, stream)
    r = L.spa_probe_read
    assert r(N, 16, 1, _fake(2), N) == S.SPA_ERR_INVALID_ARG
    assert r(_fake(), 16, 1, N, N) == S.SPA_ERR_INVALID_ARG
    assert r(bad, 16, 1, _fake(2), N) == S.SPA_ERR_INVALID_ARG
    assert r(_fake(), 0, 1, _fake(2), N) == S.SPA_ERR_INVALID_ARG
    assert r(_fake(), 24, 1, _fake(2), N) == S.SPA_ERR_INVALID_ARG
    assert r(_fake(), 16, 0, _fake(2), N) == S.SPA_ERR_INVALID_ARG
    assert r(_fake(), 16, (1 << 20) + 1, _fake(2), N) == S.SPA_ERR_INVALID_ARG
    assert b"workgroups" in L.spa_last_error()
    # spa_probe_mfma_bf16(workgroups, iters, sink, stream)
    m = L.spa_probe_mfma_bf16
    assert m(1, 1, N, N) == S.SPA_ERR_INVALID_ARG
    assert m(0, 1, _fake(), N) == S.SPA_ERR_INVALID_ARG
    assert m(1, 0, _fake(), N) == S.SPA_ERR_INVALID_ARG
    assert m(1, (1 << 24) + 1, _fake(), N) == S.SPA_ERR_INVALID_ARG
    assert b"iters" in L.spa_last_error()


def test_host_rejections_precede_device_checks():
    # with the device-side checks on, every host-side rejection still returns first, before any
    # device work (these calls pass fake host addresses and no GPU is needed)
    was = L.spa_debug_checks()
    L.spa_set_debug_checks(1)
    try:
        test_index_score_rejections()
        for suffix in ("", "_hist"):
            test_select_rejections(suffix)
        for name in ("spa_sparse_decode_attn", "spa_sparse_decode_attn_grouped"):
            test_decode_attn_rejections(name)
        test_prefill_and_permute_rejections()
        test_score_select_rejections()
        test_importance_permutation_rejections()
        test_int4_selector_rejections()
    finally:
        L.spa_set_debug_checks(was)
    assert L.spa_debug_error() == S.SPA_DBG_NONE
