"""Plant plausible mistakes into a copy of the oracle (on the CPU) and check
that the pins in test_oracle_pins.py and test_oracle_driver_pins.py reject
every one of them.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "spa_oracle.py")

# (name, original text, mistaken text)
MUTATIONS = [
    ("relu_dropped", "s = (np.maximum(dots, 0) * w[b]", "s = (dots * w[b]"),
    ("head_weight_dropped", "s = (np.maximum(dots, 0) * w[b].astype(np.int64)[None, :]).sum(axis=1)",
     "s = (np.maximum(dots, 0)).sum(axis=1)"),
    ("prefill_relu_dropped", "(np.maximum(dots, 0) * w[b, i]", "(dots * w[b, i]"),
    ("pool_no_half", "np.floor_divide(2 * s + n, 2 * n)", "np.floor_divide(s, n)"),
    ("pool_trunc", "np.floor_divide(2 * s + n, 2 * n)", "np.trunc((2 * s + n) / (2 * n))"),
    ("rank_ascending", "key=lambda j: (-int(s[j]), j)", "key=lambda j: (int(s[j]), j)"),
    ("ties_highest_index", "key=lambda j: (-int(s[j]), j)", "key=lambda j: (-int(s[j]), -j)"),
    ("topp_strict", "hit = np.nonzero(M >= p)[0]", "hit = np.nonzero(M > p)[0]"),
    ("topp_off_by_one", "kp = int(hit[0]) + 1 if len(hit)", "kp = int(hit[0]) if len(hit)"),
    ("kmin_ignored", "k = min(len(order), max(k_min, min(kp, k_max)))", "k = min(len(order), min(kp, k_max))"),
    ("kmax_ignored", "k = min(len(order), max(k_min, min(kp, k_max)))", "k = min(len(order), max(k_min, kp))"),
    ("beta_ignored", "lg = beta * np.array(", "lg = np.array("),
    ("scale_dropped", "x = (K @ qv) * scale", "x = (K @ qv)"),
    ("no_normalise", "return (e @ V) / z, float(m + np.log(z))", "return (e @ V), float(m + np.log(z))"),
    ("lse_no_max", "return (e @ V) / z, float(m + np.log(z))", "return (e @ V) / z, float(np.log(z))"),
    ("gqa_modulo", "            g = h // G\n            blocks", "            g = h % Hkv\n            blocks"),
    ("prefill_gqa_modulo", "                g = h // G\n                K = to_f64(k[b, g, kslots]",
     "                g = h % Hkv\n                K = to_f64(k[b, g, kslots]"),
    ("causal_strict", "keep = k_pos[kslots] <= pos_u", "keep = k_pos[kslots] < pos_u"),
    ("window_off_by_one", "set(range(max(0, L - window_tok), L))", "set(range(max(0, L - window_tok), L - 1))"),
    ("sink_tokens_dropped", "toks = sorted(set(range(min(sink_tok, L))) | ", "toks = sorted("),
    ("block_tail_unmasked", "for t in range(j * blk, min((j + 1) * blk, L))]", "for t in range(j * blk, (j + 1) * blk)]"),
    ("local_blocks_dropped", " | set(range(max(0, nbv - n_local), nbv))\n    cand", "\n    cand"),
    ("prefill_sink_dropped", "reserved = set(range(min(n_sink, i + 1))) | ", "reserved = "),
    ("prefill_diag_dropped", "set(range(max(0, i - n_local), i)) | {i}", "set(range(max(0, i - n_local), i))"),
    ("score_mask_inclusive", "J = min(ia, nKb)", "J = min(ia + 1, nKb)"),
    ("inverse_is_forward", "    out = np.empty_like(x)\n    idx = [slice(None)] * x.ndim",
     "    return np.take(x, perm, axis=axis)\n    idx = [slice(None)] * x.ndim"),
    ("bf16_shift", "u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)",
     "u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)"),
    ("grouped_heads_strided", "out[b, g, :nbv] = terms[:, g * hpg:(g + 1) * hpg].sum(axis=1)",
     "out[b, g, :nbv] = terms[:, g::groups].sum(axis=1)"),
    ("grouped_heads_overlap", "out[b, g, :nbv] = terms[:, g * hpg:(g + 1) * hpg].sum(axis=1)",
     "out[b, g, :nbv] = terms[:, g * hpg:(g + 1) * hpg + 1].sum(axis=1)"),
    ("per_group_first_list", "blocks = sel[b][g] if per_group else sel[b]", "blocks = sel[b][0] if per_group else sel[b]"),
    ("importance_not_causal", "x = np.where(visible, x, -np.inf)\n            e = np.exp(", "x = x\n            e = np.exp("),
    ("importance_first_block", "        u0 = L - n\n        # causal mask of the proxy", "        u0 = 0\n        # causal mask of the proxy"),
    ("importance_norm_heads_only", "imp[b] /= Hq * n", "imp[b] /= Hq"),
    ("importance_gqa_modulo", "to_f64(k[b, h // G, :L], dtype)", "to_f64(k[b, h % Hkv, :L], dtype)"),
    ("importance_sort_ascending", "key=lambda t: (-imp[b, t], t)", "key=lambda t: (imp[b, t], t)"),
    ("importance_ties_highest", "key=lambda t: (-imp[b, t], t)", "key=lambda t: (-imp[b, t], -t)"),
    ("int4_round_down", "c = np.floor_divide(2 * x + 2 ** e, 2 ** (e + 1))", "c = np.floor_divide(x, 2 ** e)"),
    ("int4_exponent_from_one", "    for e in range(8):\n        c = np.floor_divide(", "    for e in range(1, 8):\n        c = np.floor_divide("),
    ("int4_nibbles_swapped", "(c[..., 0::2] | (c[..., 1::2] << 4))", "(c[..., 1::2] | (c[..., 0::2] << 4))"),
    ("segment_check_loose", "return bool(np.all(np.asarray(perm) // seg == np.arange(T) // seg))", "return True"),
    # wiring of the whole-path drivers
    ("front_identity_positions", "pos=perm.astype(np.int64))", "pos=np.arange(len(perm)))"),
    ("front_qI_unpermuted", "qIb = pool_blocks(qI_p, cfg.blk)", "qIb = pool_blocks(inp[\"qI_tok\"], cfg.blk)"),
    ("front_kI_unpermuted", "kIb = pool_blocks(kI_p, cfg.blk)", "kIb = pool_blocks(inp[\"kI_tok\"], cfg.blk)"),
    ("step_lse_not_inverted", "res[\"lse\"] = segment_permute(lse_slot, perm, axis=2, inverse=True)",
     "res[\"lse\"] = lse_slot"),
    ("step_o_not_inverted", "res[\"o\"] = segment_permute(o_slot, perm, axis=2, inverse=True)", "res[\"o\"] = o_slot"),
    ("step_q_unpermuted", "qp = segment_permute(inp[\"q\"], perm, axis=2)", "qp = inp[\"q\"]"),
    ("step_v_unpermuted", "vp = segment_permute(inp[\"v\"], perm, axis=2)", "vp = inp[\"v\"]"),
    ("decode_int4_branch_dropped", "if getattr(cfg, \"selector_q4\", False):", "if False:"),
    ("decode_int4_branch_always", "if getattr(cfg, \"selector_q4\", False):", "if True:"),
    ("decode_topp_beta_dropped", "\"topp\",\n                                  beta=cfg.beta, p=cfg.p",
     "\"topp\",\n                                  p=cfg.p"),
    ("decode_group_topp_beta_dropped", "\"topp\",\n                                              beta=cfg.beta, p=cfg.p",
     "\"topp\",\n                                              p=cfg.p"),
    ("decode_head_mode_dropped", "                              inp[\"head_mode\"], cfg.local_sink_tok, cfg.local_window_tok,\n"
     "                              batches=batches, heads=heads)",
     "                              None, cfg.local_sink_tok, cfg.local_window_tok,\n"
     "                              batches=batches, heads=heads)"),
    ("decode_sink_window_swapped", "                              inp[\"head_mode\"], cfg.local_sink_tok, cfg.local_window_tok,\n"
     "                              batches=batches, heads=heads)",
     "                              inp[\"head_mode\"], cfg.local_window_tok, cfg.local_sink_tok,\n"
     "                              batches=batches, heads=heads)"),
    ("dense_mass_scale_dropped", "x = (K @ to_f64(q[h], dtype)) * scale", "x = (K @ to_f64(q[h], dtype))"),
    ("dense_mass_gqa_modulo", "K = to_f64(k[h // G, :L], dtype)", "K = to_f64(k[h % Hkv, :L], dtype)"),
    ("dense_mass_ignores_seq_len", "K = to_f64(k[h // G, :L], dtype)", "K = to_f64(k[h // G], dtype)"),
]

PIN_FILES = ["test_oracle_pins.py", "test_oracle_driver_pins.py"]


def test_mutation_list_applies():
    src = open(SRC).read()
    for name, old, new in MUTATIONS:
        assert src.count(old) == 1, name


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_reject_planted_mistake(tmp_path, name, old, new):
    src = open(SRC).read()
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), pkg / "__init__.py")
    (pkg / "spa_oracle.py").write_text(src.replace(old, new))
    env = dict(os.environ, SPA_ORACLE_UNDER_TEST=str(tmp_path), PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"]
                       + [os.path.join(ROOT, "tests", f) for f in PIN_FILES],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutation {name} survived the pins:\n{r.stdout[-2000:]}"
