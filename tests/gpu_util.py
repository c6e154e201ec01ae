"""Helpers for the GPU parity tests: device transfer and comparison rules."""
import numpy as np
import torch


def dev(x: np.ndarray, dtype: str = None) -> torch.Tensor:
    """Host array -> device tensor; ``dtype='bf16'`` reinterprets uint16 bits as bfloat16."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def sel_lists(idx: torch.Tensor, count: torch.Tensor):
    """Device idx/count -> nested python lists of selected block indices."""
    idx = idx.cpu().numpy()
    count = count.cpu().numpy()
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
