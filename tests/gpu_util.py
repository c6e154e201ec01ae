"""Helpers for the GPU parity tests: device transfer and comparison rules."""
import numpy as np
import torch


def dev(x: np.ndarray, dtype: str = None) -> torch.Tensor:
    """Host array -> device tensor; ``dtype='bf16'`` reinterprets uint16 bits as bfloat16."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def check_list_rows(idx: np.ndarray, count: np.ndarray):
    """Every selection row as the library writes it: count in [0, cap], the first count entries
    strictly ascending (so free of duplicates) and non-negative, the rest of the row -1."""
    cap = idx.shape[-1]
    rows = idx.reshape(-1, cap)
    cnt = count.reshape(-1)
    assert rows.shape[0] == cnt.shape[0], "idx and count rows differ"
    for r in range(rows.shape[0]):
        c = int(cnt[r])
        assert 0 <= c <= cap, f"row {r}: count {c} outside [0, {cap}]"
        live = rows[r, :c]
        assert (live >= 0).all(), f"row {r}: negative block index in the list"
        assert (np.diff(live) > 0).all(), f"row {r}: list not strictly ascending"
        assert (rows[r, c:] == -1).all(), f"row {r}: entries past count are not -1"


def sel_lists(idx: torch.Tensor, count: torch.Tensor):
    """Device idx/count -> nested python lists of selected block indices (rows checked
    ascending, duplicate-free and padded with -1 first)."""
    idx = idx.cpu().numpy()
    count = count.cpu().numpy()
    check_list_rows(idx, count)
    if idx.ndim == 2:
        return [idx[b, :count[b]].tolist() for b in range(idx.shape[0])]
    return [[idx[b, i, :count[b, i]].tolist() for i in range(idx.shape[1])] for b in range(idx.shape[0])]


def attn_close(o_gpu: np.ndarray, o_ref: np.ndarray, max_abs=1e-2, rel_l2=2e-3, mask=None):
    """Attention tolerance: max |diff| <= 1e-2 and ||diff||_2 / ||ref||_2 <= 2e-3."""
    g = np.asarray(o_gpu, dtype=np.float64)
    r = np.asarray(o_ref, dtype=np.float64)
    if mask is not None:
        g, r = g[mask], r[mask]
    diff = g - r
    ma = float(np.max(np.abs(diff))) if diff.size else 0.0
    rl = float(np.linalg.norm(diff) / max(np.linalg.norm(r), 1e-30))
    assert np.isfinite(g).all(), "non-finite output"
    assert ma <= max_abs, f"max abs error {ma:.3e} > {max_abs}"
    assert rl <= rel_l2, f"relative L2 error {rl:.3e} > {rel_l2}"
    return ma, rl


def check_topp_row(gpu_sel, info, k_min, k_max, p, tol=1e-5):
    """The GPU set is reserved + a prefix of the oracle's rank order whose length may
    differ from the oracle's only through ranks whose cumulative mass lies within
    ``tol`` of p."""
    res = set(info["reserved"])
    order = info["order"]
    cum = info["cum"]
    gpu_sel = list(gpu_sel)
    assert all(a < b for a, b in zip(gpu_sel, gpu_sel[1:])), "GPU list not strictly ascending"
    assert res <= set(gpu_sel), "reserved block missing"
    chosen = [j for j in gpu_sel if j not in res]
    kg = len(chosen)
    assert set(chosen) == set(order[:kg]), "GPU set is not a prefix of the rank order"
    ko = info["k"]
    if kg == ko:
        return
    lo, hi = sorted((kg, ko))
    # one side stopped after lo blocks, the other after hi: the cumulative
    # masses after lo .. hi-1 blocks (cum[lo-1] .. cum[hi-2]) were read on
    # opposite sides of p, so each must sit on the threshold
    assert k_min <= lo and hi <= k_max, (kg, ko)
    for t in range(max(0, lo - 1), hi - 1):
        assert abs(cum[t] - p) <= tol, f"rank {t}: cumulative mass {cum[t]!r} not within {tol} of p (gpu {kg}, oracle {ko})"


def imp_close(imp_gpu: np.ndarray, imp_ref: np.ndarray, rel=1e-4):
    """Importance tolerance: |diff| <= rel * |ref| + 1e-12 per key (fp32 softmax over bf16 products)."""
    g = np.asarray(imp_gpu, dtype=np.float64)
    r = np.asarray(imp_ref, dtype=np.float64)
    bad = np.abs(g - r) > rel * np.abs(r) + 1e-12
    assert not bad.any(), f"{int(bad.sum())} importances out of tolerance, worst at {np.argmax(np.abs(g - r))}"


def check_importance_perm(perm_gpu, imp_gpu, imp_ref, seq_len, seg, rel=1e-4):
    """The GPU permutation of one sequence: every segment maps onto itself; the
    valid keys are sorted by the GPU's own importances (descending, equal values
    by position) and the keys past seq_len follow in order; measured with the
    oracle's importances the order may invert only pairs whose importances agree
    within the tolerance.  Returns the number of positions that differ from a
    sort by the oracle's importances."""
    perm = np.asarray(perm_gpu, dtype=np.int64)
    T = perm.shape[0]
    L = int(seq_len)
    assert np.array_equal(np.sort(perm), np.arange(T)), "not a permutation"
    assert np.all(perm // seg == np.arange(T) // seg), "permutation leaves its segment"
    differ = 0
    for s0 in range(0, T, seg):
        idx = perm[s0:min(s0 + seg, T)]
        valid = idx[idx < L]
        assert np.array_equal(idx[len(valid):], np.arange(max(L, s0), min(s0 + seg, T))), "tail out of order"
        assert np.all(idx[:len(valid)] < L), "a key past seq_len precedes a valid key"
        vg = np.asarray(imp_gpu, dtype=np.float64)[valid]
        assert np.all((vg[:-1] > vg[1:]) | ((vg[:-1] == vg[1:]) & (valid[:-1] < valid[1:]))), "not sorted by imp"
        vr = np.asarray(imp_ref, dtype=np.float64)[valid]
        # oracle importances along the GPU order never rise by more than the tolerance
        run_min = np.minimum.accumulate(vr)
        assert np.all(vr <= run_min + 2 * rel * np.abs(vr) + 1e-12), "order inverted beyond the tolerance"
        ref_order = np.array(sorted(valid.tolist(), key=lambda t: (-imp_ref[t], t)))
        differ += int((ref_order != valid).sum())
    return differ
