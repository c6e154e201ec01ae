"""Throughput of the block-sparse attention hot path on one MI355X.

Default workload: one sparse decode step at 128K context.  A step is the
whole decode hot path of one attention layer over one batch: int8 indexer
scores, dual top-p selection, then the split sparse flash-decode and its
log-sum-exp merge, replayed as HIP graphs.  B = 16 sequences of 131072 tokens,
64 query heads over 8 KV heads, d = 128, 64-token blocks, top-p 0.9 over
softmax(s/8) with K_min 16 / K_max 512 plus 1 sink and 4 local blocks
(seeded synthetic inputs, planted relevant blocks per sequence drawn from
1..200).  value = sequences decoded per second (tokens/s).

``--workload`` selects another of the named workloads: the other decode
shapes (tokens/s, same definition) or the 64K permuted block-sparse prefill
(prompt tokens/s; a step is pool + score of the per-token indexer vectors
gathered through the permutation, select, and the sparse attention reading
Q, K, V and writing O in the original token order; with the importance
permutation, computing it first; in chunks of query tokens with ``--chunk``;
replayed as one HIP graph per step).

All inputs are resident in HBM before the timed region.  Every per-step input
is replicated in ``--copies`` buffer sets that consecutive steps rotate
through, so that the union of the bytes one rotation touches is at least
1 GiB and a step cannot be served from the 256 MB Infinity Cache left warm by
the previous one (0 = choose that count automatically).

Prints one JSON line.  roofline: the dominant launch (decode: the sparse
attention entry point, main kernel + merge, against 8 TB/s of HBM; prefill:
the block-sparse attention kernel against the bf16 dense MFMA peak), timed
with HIP events on the stream it runs on.  cpu_baseline: the CPU oracle on a
bounded sample of the same inputs.  achievable: what the library's two rate
probes (include/spa_probe.h) reach on the same GPU, a plain streaming HBM read
and a loop of independent bf16 MFMAs; the roofline also states its fraction of
that achievable rate beside the fraction of the vendor peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
INT8_MFMA_PEAK_TOPS = 5000.0
PROBE_READ_BYTES = 2 << 30      # the read probe's buffer: well beyond the 256 MB Infinity Cache
PROBE_MFMA_ITERS = 4096         # rounds of the MFMA probe (about half a millisecond per call)
ROTATE_BYTES = 1 << 30          # bytes one rotation over the copies must touch
COPY_MEM_LIMIT = 64 << 30       # device bytes all copies together may take

DECODE_METRIC = "sparse-decode tokens/s at 128K ctx (1 GPU); achieved HBM GB/s vs peak"
WORKLOADS = ("decode_128k_topp", "decode_32k", "decode_64k_headsplit", "decode_128k_pergroup", "decode_128k_topp_q4",
             "tiny_decode", "prefill_64k", "prefill_64k_importance")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 50 decode, 20 prefill)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 10 decode, 3 prefill)")
    ap.add_argument("--workload", choices=WORKLOADS, default="decode_128k_topp")
    ap.add_argument("--copies", type=int, default=0, help="input buffer sets to rotate through (0 = auto)")
    ap.add_argument("--select-path", choices=("fused", "separate"), default="separate",
                    help="decode: one fused scoring+selection launch, or the scoring kernel then the selection kernel")
    ap.add_argument("--select-algo", choices=("sort", "hist"), default="sort",
                    help="selection kernel: bitonic sort of the candidates, or the sort-free radix threshold search")
    ap.add_argument("--launch", choices=("graph", "eager"), default="graph",
                    help="replay the timed steps as HIP graphs (decode: one per input set; prefill: one whole "
                         "step, every chunk) or launch them call by call")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true", help="skip the achievable-rate probes")
    ap.add_argument("--traffic-json", default=None,
                    help="counter-measured HBM traffic of the dominant launch (default profiles/<workload>_traffic.json)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this size before the timed steps (counter calibration)")
    ap.add_argument("--chunk", type=int, default=0,
                    help="prefill: query tokens per chunk (0 = one chunk covering the sequence)")
    a = ap.parse_args()
    prefill = a.workload.startswith("prefill")
    if a.steps is None:
        a.steps = 20 if prefill else 50
    if a.warmup is None:
        a.warmup = 3 if prefill else 10
    if a.traffic_json is None:
        a.traffic_json = os.path.join(ROOT, "profiles", f"{a.workload}_traffic.json")
    return a


def config_of(name):
    import gen
    return {"decode_128k_topp": gen.DECODE_128K_TOPP, "decode_32k": gen.DECODE_32K,
            "decode_64k_headsplit": gen.DECODE_64K_HEADSPLIT, "decode_128k_pergroup": gen.DECODE_128K_PERGROUP,
            "tiny_decode": gen.TINY_DECODE, "prefill_64k_importance": gen.PREFILL_64K_IMPORTANCE,
            "decode_128k_topp_q4": gen.DECODE_128K_TOPP_Q4,
            "prefill_64k": gen.PREFILL_64K}[name]


def source_sha(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "block_sparse_long_int8_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(path, sha):
    """Counter-measured HBM bytes per launch of the dominant kernel, as stored by profile_summary.py, if
    they were taken on the current kernel source (else None: the counters would describe another kernel)."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tj = json.load(f)
    return tj.get("traffic_bytes_per_launch") if tj.get("kernel_source_sha") == sha else None


TRAFFIC_NOTE = ("stored counter figure (rocprofv3 FETCH_SIZE and WRITE_SIZE passes scaled by a copy of known size, "
                "profiles/{w}_traffic.json), not measured in this run; null when the kernel source changed since")


def pct(v, q):
    import numpy as np
    return float(np.percentile(np.asarray(v), q))


def dev(x, dt=None):
    import numpy as np
    import torch
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def calibration_copy(mib):
    """One plain copy of ``mib`` MiB through the library's permute_kernel (identity permutation:
    exactly mib MiB read and mib MiB written), the reference the HBM byte counters are scaled by."""
    import torch

    import block_sparse_long_int8_amd as S
    rows = (mib << 20) // 4096
    src = torch.ones((1, rows, 4096), dtype=torch.uint8, device="cuda")
    perm = torch.arange(rows, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    S.spa_segment_permute(src, perm, rows, dim=1)
    torch.cuda.synchronize()
    del src, perm
    log(f"[bench] calibration copy of {mib} MiB done")


MAX_GRAPH_STEPS = 64


def n_copies(args, touched, per_copy):
    if args.copies > 0:
        return args.copies
    want = max(3, -(-ROTATE_BYTES // max(1, touched)))
    return int(max(1, min(want, 4096, COPY_MEM_LIMIT // max(1, per_copy))))


# ---------------------------------------------------------------- decode ----

def decode_attn_bytes(cfg, idx, counts, seq_len, head_mode) -> int:
    """Algorithmic HBM bytes of one sparse attention launch.

    K and V rows of the tokens each KV group attends (selected blocks clipped
    to the sequence for retrieval groups, sink tokens + window for local
    groups), plus Q, O (fp32), lse (fp32), the block lists and counts.
    idx/counts hold one list per sequence ([B, cap] / [B]) or, with per-group
    selection, one per (sequence, KV head) ([B, Hkv, cap] / [B, Hkv]).
    """
    el = 4 if cfg.dtype == "f32" else 2
    row = cfg.d * el
    kv = 0
    per_group = idx.ndim == 3
    for b in range(cfg.B):
        L = int(seq_len[b])
        loc_tok = min(L, cfg.local_sink_tok + cfg.local_window_tok) if cfg.local_window_tok else 0
        for g in range(cfg.Hkv):
            lst = idx[b, g, :counts[b, g]] if per_group else idx[b, :counts[b]]
            sel_tok = sum(min(cfg.blk, L - int(j) * cfg.blk) for j in lst)
            kv += 2 * row * (loc_tok if head_mode[g] else sel_tok)
    q = cfg.B * cfg.Hq * cfg.d * el
    o = cfg.B * cfg.Hq * cfg.d * 4
    lse = cfg.B * cfg.Hq * 4
    lists = int(counts.sum()) * 4 + counts.size * 4 + cfg.B * 4
    return kv + q + o + lse + lists


def decode_index_bytes(cfg, seq_len) -> int:
    """Algorithmic bytes of scoring + selection: the selector keys of the valid blocks
    (int8: r bytes per head; int4 cache: r/2 bytes of codes + 1 exponent byte), qI, w,
    block lists."""
    nbv = sum(-(-int(L) // cfg.blk) for L in seq_len)
    per_head = cfg.r // 2 + 1 if cfg.selector_q4 else cfg.r
    return nbv * cfg.H_idx * per_head + cfg.B * cfg.H_idx * (cfg.r + 1) + cfg.B * 4


def best_cpu(threaded, single):
    """The faster of the threaded and the one-thread oracle run is the baseline; the other is kept beside it
    (the oracle's many small numpy calls do not always gain from threads)."""
    best, other = (threaded, single) if threaded["value"] >= single["value"] else (single, threaded)
    return dict(best, other_thread_count={k: other[k] for k in ("value", "cores", "sample")})


def decode_cpu_baseline(inp, cfg):
    """The CPU oracle on one full decode step (all sequences), repeated to about 10 s."""
    from threadpoolctl import threadpool_info

    import oracle as O
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    t0 = time.perf_counter()
    O.decode_step(inp)
    reps = 1
    while time.perf_counter() - t0 < 10.0 and reps < 20:
        O.decode_step(inp)
        reps += 1
    dt = (time.perf_counter() - t0) / reps
    # the same step on one thread (BLAS pools limited to 1)
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        t1 = time.perf_counter()
        O.decode_step(inp)
        dt1 = time.perf_counter() - t1
    return best_cpu({"value": cfg.B / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
                     "sample": f"full decode step of all {cfg.B} sequences (integer scores, selection, fp64 "
                               f"attention), mean of {reps} runs, {dt:.3f} s each"},
                    {"value": cfg.B / dt1, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                     "sample": f"one run of the same step on one thread, {dt1:.3f} s"})


def bench_decode(args, cfg):
    import numpy as np
    import torch

    import block_sparse_long_int8_amd as S
    import gen

    t0 = time.time()
    inp = gen.make(cfg, seed=args.seed)
    log(f"[bench] generated {cfg.name} in {time.time() - t0:.1f} s")
    torch.cuda.set_device(0)
    dt = cfg.dtype
    base = {"q": dev(inp["q"], dt), "k": dev(inp["k"], dt), "v": dev(inp["v"], dt), "qI": dev(inp["qI"]),
            "kI": dev(inp["kI"]), "w": dev(inp["w"])}
    if cfg.selector_q4:
        # the selector cache is written as int4 when keys enter it (outside the step)
        base["kq"], base["ke"] = S.spa_quantize_selector_keys(base.pop("kI"))

    def sel_keys(x):
        return (x["kq"], x["ke"]) if cfg.selector_q4 else x["kI"]
    seq_len, head_mode = dev(inp["seq_len"]), dev(inp["head_mode"])
    spec = S.DecodeSpec(B=cfg.B, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d, Tcap=cfg.T, blk=cfg.blk, H_idx=cfg.H_idx,
                        r=cfg.r, n_sink=cfg.n_sink, n_local=cfg.n_local, select=cfg.select, k=cfg.k, beta=cfg.beta,
                        p=cfg.p, k_min=cfg.k_min, k_max=cfg.k_max, local_sink_tok=cfg.local_sink_tok,
                        local_window_tok=cfg.local_window_tok, select_algo=args.select_algo,
                        per_group=cfg.per_group, selector_q4=cfg.selector_q4)
    if (cfg.per_group or cfg.selector_q4) and args.select_path == "fused":
        raise SystemExit("per-group and int4 selection have no fused score+select launch; use --select-path separate")
    step = S.DecodeStep(spec, fused=args.select_path == "fused")
    step(base["q"], base["k"], base["v"], base["qI"], sel_keys(base), base["w"], seq_len, head_mode)
    torch.cuda.synchronize()
    idx, counts = step.idx.cpu().numpy(), step.count.cpu().numpy()
    ab = decode_attn_bytes(cfg, idx, counts, inp["seq_len"], inp["head_mode"])
    ib = decode_index_bytes(cfg, inp["seq_len"])
    per_copy = sum(t.numel() * t.element_size() for t in base.values())
    copies = n_copies(args, ab + ib, per_copy)
    if args.launch == "graph":
        # a graph holds at most 64 steps; only a step of well under 16 MB (the
        # tiny workload) wants more copies, and it is latency-bound anyway
        copies = min(copies, MAX_GRAPH_STEPS)
    sets = [base] + [{n: t.clone() for n, t in base.items()} for _ in range(copies - 1)]
    torch.cuda.synchronize()
    log(f"[bench] inputs resident: {copies} copies of {per_copy / 2**30:.3f} GiB; "
        f"{(ab + ib) / 1e6:.1f} MB touched per step")

    # HIP graphs: one graph of C = min(copies, steps) consecutive steps on input
    # sets 0 .. C-1 (steps inside a graph follow each other without a launch
    # boundary) and one of the remaining K mod C steps; the timed steps use input
    # set j % copies for step j.
    use_graph = args.launch == "graph"
    step_args = [(x["q"], x["k"], x["v"], x["qI"], sel_keys(x), x["w"], seq_len, head_mode) for x in sets]
    chunk_len = min(copies, args.steps)
    tail_len = args.steps % chunk_len
    chunk = step.capture_steps(step_args[:chunk_len]) if use_graph else None
    tail = step.capture_steps(step_args[:tail_len]) if use_graph and tail_len else None
    if use_graph:
        log(f"[bench] captured a {chunk_len}-step graph" + (f" and a {tail_len}-step graph" if tail else ""))

    def launches(n):
        """The launches of n steps on input sets 0, 1, ... (mod copies): (graph or None, steps)."""
        out, j = [], 0
        while j < n:
            m = chunk_len if n - j >= chunk_len else n - j
            out.append((chunk if m == chunk_len else tail, m) if use_graph else (None, 1))
            j += m if use_graph else 1
        return out

    def run(i, ev=None):
        x = sets[i % copies]
        if ev is not None:
            ev[0].record()
        if step.fused:
            step.score_select(x["qI"], x["kI"], x["w"], seq_len)
        else:
            step.score(x["qI"], sel_keys(x), x["w"], seq_len)
            step.select(seq_len)
        if ev is not None:
            ev[1].record()
        step.attend(x["q"], x["k"], x["v"], seq_len, head_mode)
        if ev is not None:
            ev[2].record()

    def run_steps(n):
        """Untimed steps: whole graphs of chunk_len steps (n rounded up), or eager steps."""
        for j in range(-(-n // chunk_len) if use_graph else n):
            chunk.replay() if use_graph else run(j)

    run_steps(args.warmup)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")
    if args.copy_calibration_mib:
        calibration_copy(args.copy_calibration_mib)

    # the timed steps, an event after each launch (a graph of chunk_len steps, or one eager step);
    # value comes from the first and last event, the per-step spread from the launches between them
    plan = launches(args.steps)
    evt = [torch.cuda.Event(enable_timing=True) for _ in range(len(plan) + 1)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    evt[0].record()
    j = 0
    for n, (g, m) in enumerate(plan):
        if g is not None:
            g.replay()
        else:
            run(j)
        j += m
        evt[n + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = evt[0].elapsed_time(evt[-1])
    per_step = [evt[n].elapsed_time(evt[n + 1]) / m for n, (_, m) in enumerate(plan)]
    ms_step = total_ms / args.steps
    log(f"[bench] timed {args.steps} steps in {len(plan)} launches: {total_ms:.3f} ms on events, "
        f"{wall * 1e3:.3f} ms wall")
    # a second pass of the same steps with events between the stages, for the per-stage breakdown
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        run(args.warmup + args.steps + i, evs[i])
    torch.cuda.synchronize()
    sel_ms = [e[0].elapsed_time(e[1]) for e in evs]
    attn_ms = [e[1].elapsed_time(e[2]) for e in evs]
    step_ms = [e[0].elapsed_time(e[2]) for e in evs]

    # Each stage on its own, without host launch gaps: a graph of chunk_len
    # consecutive calls of the stage on the rotating input sets (the attention
    # calls all use the last step's block lists), replayed with one event pair
    # around all the replays.  The roofline's launch duration is the attention
    # operation's time from this pass (both of its kernels and the gap between).
    op_ms = None
    if use_graph:
        def stage_graph(fns):
            for f in fns:
                f()  # settle lazy state outside the capture
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for f in fns:
                    f()
            return g

        def sel_call(x):
            if step.fused:
                step.score_select(x["qI"], x["kI"], x["w"], seq_len)
            else:
                step.score(x["qI"], sel_keys(x), x["w"], seq_len)
                step.select(seq_len)

        g_sel = stage_graph([lambda x=sets[j]: sel_call(x) for j in range(chunk_len)])
        g_att = stage_graph([lambda x=sets[j]: step.attend(x["q"], x["k"], x["v"], seq_len, head_mode)
                             for j in range(chunk_len)])
        reps = max(1, -(-args.steps // chunk_len))
        op_ms = {}
        for name, g in (("select", g_sel), ("attention", g_att)):
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            op_ms[name] = e0.elapsed_time(e1) / (reps * chunk_len)
        log(f"[bench] stages alone (graph replays of {chunk_len} calls): select {op_ms['select'] * 1e3:.2f} us, "
            f"attention {op_ms['attention'] * 1e3:.2f} us")

    attn_s = (op_ms["attention"] if op_ms else float(np.mean(attn_ms))) * 1e-3
    achieved = ab / attn_s / 1e9
    traffic = load_traffic(args.traffic_json, source_sha("decode_attn.hip"))
    select_name = ("score_select_topp" if cfg.select == "topp" else "score_select_topk") + \
        ("" if step.fused else " (score, then select)")
    res = {
        "metric": DECODE_METRIC if cfg is config_of("decode_128k_topp")
        else f"sparse-decode tokens/s ({cfg.name}, 1 GPU); achieved HBM GB/s vs peak",
        "value": cfg.B / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "T": cfg.T, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "d": cfg.d,
                   "blk": cfg.blk, "H_idx": cfg.H_idx, "r": cfg.r, "select": cfg.select, "k": cfg.k, "p": cfg.p,
                   "beta": cfg.beta, "k_min": cfg.k_min, "k_max": cfg.k_max, "n_sink": cfg.n_sink,
                   "n_local": cfg.n_local, "retrieval_groups": int(sum(1 for m in inp["head_mode"] if m == 0)),
                   "per_group_selection": cfg.per_group,
                   "selector_cache": "int4, one power-of-two scale per 16 keys" if cfg.selector_q4 else "int8",
                   "local_sink_tok": cfg.local_sink_tok, "local_window_tok": cfg.local_window_tok,
                   "input_copies_rotated": copies, "seed": args.seed,
                   "launch": f"hip_graph, {chunk_len} steps per graph" if use_graph else "eager",
                   "select_path": args.select_path, "select_algo": args.select_algo},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "traffic_source": TRAFFIC_NOTE.format(w=args.workload),
                     "kernel": "spa_sparse_decode_attn (decode main kernel + decode_merge_kernel)",
                     "algorithmic_bytes_per_launch": ab, "avg_launch_ms": attn_s * 1e3,
                     "launch_timing": ("graph replays of the attention calls alone, one event pair around them"
                                       if op_ms else "events around each eager attention call")},
        "step_ms_p10_p50_p90": [pct(per_step, 10), pct(per_step, 50), pct(per_step, 90)],
        "step_timing": (f"events around each timed graph launch ({chunk_len} steps each), per step"
                        if use_graph else "events around each timed step"),
        "stages_ms": {select_name: float(np.mean(sel_ms)), "attention": float(np.mean(attn_ms))},
        "stages_alone_ms": ({select_name: op_ms["select"], "attention": op_ms["attention"]} if op_ms else None),
        "staged_step_ms_p10_p50_p90": [pct(step_ms, 10), pct(step_ms, 50), pct(step_ms, 90)],
        "stage_timing": "stages_ms: a second pass of the same steps, launched call by call with events between "
                        "stages (host launch gaps included); stages_alone_ms: graph replays of each stage alone",
        "selected_blocks": {"mean": float(counts.mean()), "min": int(counts.min()), "max": int(counts.max())},
        "step_algorithmic_bytes": ab + ib,
        "selector_cache_bytes": {"int8": cfg.B * cfg.nb * cfg.H_idx * cfg.r,
                                 "int4": cfg.B * cfg.nb * cfg.H_idx * (cfg.r // 2 + 1),
                                 "held": "int4" if cfg.selector_q4 else "int8"},
        "step_hbm_gbs": (ab + ib) / (ms_step * 1e-3) / 1e9,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        res["cpu_baseline"] = decode_cpu_baseline(inp, cfg)
    return res


# --------------------------------------------------------------- prefill ----

def prefill_pairs(perm, idx, counts, blk) -> int:
    """Attended (query, key) pairs of one head: selected slots with an original position <= the query's."""
    import numpy as np
    pos = np.asarray(perm, dtype=np.int64)
    total = 0
    for i in range(len(counts)):
        sel = idx[i, :counts[i]]
        kp = np.sort(np.concatenate([pos[j * blk:(j + 1) * blk] for j in sel]))
        total += int(np.searchsorted(kp, pos[i * blk:(i + 1) * blk], side="right").sum())
    return total


def prefill_cpu_baseline(inp, cfg):
    """The CPU oracle on the full front end plus the attention of sampled query blocks, scaled to T."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle as O
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    nq = cfg.nb
    sample = list(range(nq // 32, nq, nq // 16))  # 16 evenly spaced query blocks
    t0 = time.perf_counter()
    if cfg.perm_kind == "importance":
        imp = O.key_importance(inp["q"], inp["k"], cfg.dtype, inp["seq_len"], cfg.proxy)
        inp = dict(inp, perm=O.importance_permutation(imp, inp["seq_len"], cfg.seg)[0].astype(np.int32))
    front = O.prefill_front(inp)
    t_front = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.prefill_step(inp, front=front, blocks=[])
    t_fixed = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.prefill_step(inp, front=front, blocks=sample)
    t_sample = time.perf_counter() - t0
    t_full = t_front + t_fixed + (t_sample - t_fixed) * nq / len(sample)
    # one thread: the attention of 4 of the sampled blocks, scaled the same way
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        t1 = time.perf_counter()
        O.prefill_step(inp, front=front, blocks=sample[:4])
        t_sample1 = time.perf_counter() - t1
        t1 = time.perf_counter()
        front1 = O.prefill_front(inp)
        t_front1 = time.perf_counter() - t1
    del front1
    t_full1 = t_front1 + t_fixed + (t_sample1 - t_fixed) * nq / 4
    single = {"value": cfg.B * cfg.T / t_full1, "unit": "tokens/s", "cores": 1, "kind": "oracle",
              "sample": f"front end ({t_front1:.2f} s) and 4 sampled query blocks ({t_sample1 - t_fixed:.2f} s) on one "
                        f"thread, the permutation time of the threaded run, scaled to all {nq}"}
    return best_cpu({"value": cfg.B * cfg.T / t_full, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"oracle front end ({'importance permutation, ' if cfg.perm_kind == 'importance' else ''}"
                      f"permute, pool, score, select) on all {nq} query blocks ({t_front:.2f} s), "
                      f"Q/K/V permutation ({t_fixed:.2f} s), and fp64 attention of {len(sample)} evenly spaced "
                      f"query blocks ({t_sample - t_fixed:.2f} s) scaled to all {nq}"}, single)


def bench_prefill(args, cfg):
    import numpy as np
    import torch

    import block_sparse_long_int8_amd as S
    import gen

    t0 = time.time()
    inp = gen.make(cfg, seed=args.seed)
    log(f"[bench] generated {cfg.name} in {time.time() - t0:.1f} s")
    torch.cuda.set_device(0)
    x = {"q": dev(inp["q"], "bf16"), "k": dev(inp["k"], "bf16"), "v": dev(inp["v"], "bf16"),
         "qI": dev(inp["qI_tok"]), "kI": dev(inp["kI_tok"]), "w": dev(inp["w"]), "perm": dev(inp["perm"])}
    importance = cfg.perm_kind == "importance"
    spec = S.PrefillSpec(B=cfg.B, T=cfg.T, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d, blk=cfg.blk, H_idx=cfg.H_idx, r=cfg.r,
                         k=cfg.k, n_sink=cfg.n_sink, n_local=cfg.n_local, seg=cfg.seg, select_algo=args.select_algo,
                         perm_kind="importance" if importance else "given", proxy=cfg.proxy, chunk=args.chunk)
    step = S.PrefillStep(spec)
    step(x["q"], x["k"], x["v"], x["qI"], x["kI"], x["w"], None if importance else x["perm"])
    torch.cuda.synchronize()
    log(f"[bench] inputs resident: {sum(t.numel() * t.element_size() for t in x.values()) / 2**30:.2f} GiB")

    stages = (("importance_perm",) if importance else ()) + \
        ("pool_score", "select", "attention")

    def run(ev=None):
        marks = iter(range(len(stages) + 1))

        def mark():
            j = next(marks)
            if ev is not None:
                ev[j].record()
        mark()
        if importance:
            perm = step.importance(x["q"], x["k"])
            mark()
        else:
            perm = x["perm"]
        step.set_perm(perm)
        step.score(x["qI"], x["kI"], x["w"])
        mark()
        step.select()
        mark()
        step.attend(x["q"], x["k"], x["v"])
        mark()

    # the timed steps: replays of one HIP graph holding a whole step (every chunk), or eager calls
    use_graph = args.launch == "graph"
    launch = run
    if use_graph:
        run()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        launch = graph.replay
    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")
    if args.copy_calibration_mib:
        calibration_copy(args.copy_calibration_mib)
    evt = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evt[0].record()
    for i in range(args.steps):
        launch()
        evt[i + 1].record()
    torch.cuda.synchronize()
    total_ms = evt[0].elapsed_time(evt[-1])
    per_step = [evt[j].elapsed_time(evt[j + 1]) for j in range(args.steps)]
    ms_step = total_ms / args.steps
    log(f"[bench] timed {args.steps} steps: {total_ms:.3f} ms on events")
    # a second pass with events between the stages, for the per-stage breakdown
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    for i in range(args.steps):
        run(evs[i])
    torch.cuda.synchronize()
    st_ms = {n: float(np.median([e[j].elapsed_time(e[j + 1]) for e in evs])) for j, n in enumerate(stages)}
    # with graphs, each stage alone: one graph holding the stage's calls (every chunk) for all the
    # timed steps back to back, replayed once between one event pair, so the time per call carries no
    # host or graph launch gap; the roofline uses the attention's
    st_alone = None
    if use_graph:
        fns = {}
        if importance:
            fns["importance_perm"] = lambda: step.importance(x["q"], x["k"])
        fns["pool_score"] = lambda: step.score(x["qI"], x["kI"], x["w"])
        fns["select"] = step.select
        fns["attention"] = lambda: step.attend(x["q"], x["k"], x["v"])
        st_alone = {}
        for name, fn in fns.items():
            fn()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(args.steps):
                    fn()
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            st_alone[name] = e0.elapsed_time(e1) / args.steps
    st_op = st_alone or st_ms

    idx, counts = step.idx[0].cpu().numpy(), step.count[0].cpu().numpy()
    chunks = len(step.chunks)
    used_perm = step.perm[0].cpu().numpy() if importance else inp["perm"]
    pairs = prefill_pairs(used_perm, idx, counts, cfg.blk)
    flop = 4.0 * cfg.d * cfg.Hq * pairs * cfg.B
    attn_s = st_op["attention"] * 1e-3
    achieved = flop / attn_s / 1e12
    nq = cfg.nb
    score_ops = 2.0 * cfg.r * cfg.H_idx * (nq * (nq - 1) // 2) * cfg.B
    score_s = st_op["pool_score"] * 1e-3
    pool_bytes = cfg.B * cfg.T * (2 * cfg.H_idx * cfg.r)
    traffic = load_traffic(args.traffic_json, source_sha("prefill_attn.hip"))
    res = {
        "metric": f"block-sparse prefill tokens/s ({cfg.name}, 1 GPU); attention TFLOP/s vs bf16 MFMA peak",
        "value": cfg.B * cfg.T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "T": cfg.T, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "d": cfg.d,
                   "blk": cfg.blk, "H_idx": cfg.H_idx, "r": cfg.r, "k": cfg.k, "n_sink": cfg.n_sink,
                   "seg": cfg.seg, "causal": True, "seed": args.seed, "select_algo": args.select_algo,
                   "permutation": "importance-sorted (last query block as proxy)" if importance
                   else "uniform random per segment", "heavy_hitter_frac": cfg.hh_frac,
                   "chunks": chunks, "chunk_tokens": args.chunk or cfg.T,
                   "launch": "hip_graph, one step per graph" if use_graph else "eager"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / BF16_MFMA_PEAK_TFLOPS, "traffic": traffic if chunks == 1 else None,
                     "traffic_source": TRAFFIC_NOTE.format(w=args.workload) + " (one-chunk runs only)",
                     "kernel": "spa_block_sparse_prefill (prefill attention kernel"
                               + (f", {chunks} launches per step" if chunks > 1 else "") + ")",
                     "algorithmic_flop_per_launch": flop / chunks, "attended_pairs_per_head": pairs,
                     "avg_launch_ms": attn_s * 1e3 / chunks,
                     "launch_timing": ("one graph of the attention calls of every timed step back to back, one "
                                       "event pair around its replay" if st_alone
                                       else "events around the eager attention calls")},
        "step_ms_p10_p50_p90": [pct(per_step, 10), pct(per_step, 50), pct(per_step, 90)],
        "step_timing": "events between the timed steps themselves" + (" (graph replays)" if use_graph else ""),
        "stages_ms": st_ms,
        "stages_alone_ms": st_alone,
        "stage_timing": "stages_ms: median over a second pass of the same steps, launched call by call with "
                        "events between stages; stages_alone_ms: each stage alone, its calls for every timed step in one graph",
        "scoring": {"int8_ops": score_ops, "tops": score_ops / score_s / 1e12,
                    "frac_of_int8_mfma_peak": score_ops / score_s / 1e12 / INT8_MFMA_PEAK_TOPS,
                    "pool_read_bytes": pool_bytes,
                    "note": "one pooling launch over both per-token tensors (gathered through the permutation) "
                            "and the block-pair scoring launch"},
        "selected_blocks": {"mean": float(counts.mean()), "max": int(counts.max())},
    }
    if importance:
        # two passes of S = Q_proxy K^T over every key (4 query heads per wave group), K read twice
        n_proxy = min(cfg.proxy, cfg.T)
        imp_flop = 2 * 2.0 * cfg.B * cfg.Hq * n_proxy * cfg.T * cfg.d
        imp_bytes = 2 * cfg.B * cfg.Hkv * cfg.T * cfg.d * 2
        t_imp = st_op["importance_perm"] * 1e-3
        res["importance"] = {"ms": st_op["importance_perm"], "flop": imp_flop, "tflops": imp_flop / t_imp / 1e12,
                             "k_bytes": imp_bytes, "k_gbs": imp_bytes / t_imp / 1e9,
                             "share_of_step": st_op["importance_perm"] / sum(st_op.values())}
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        res["cpu_baseline"] = prefill_cpu_baseline(inp, cfg)
    return res


def achievable_rates():
    """The achievable HBM read rate and bf16 MFMA rate of this GPU: the best of five event-timed calls of
    each rate probe, after one warm-up, on the stream they run on."""
    import torch

    import block_sparse_long_int8_amd as S
    n_cu = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    buf = torch.empty(PROBE_READ_BYTES, dtype=torch.uint8, device="cuda")
    sink_i = torch.zeros(1, dtype=torch.int32, device="cuda")
    sink_f = torch.zeros(1, dtype=torch.float32, device="cuda")

    def best(fn, n=5):
        fn()
        ts = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return min(ts)

    read_wg, mfma_wg = 8 * n_cu, 2 * n_cu
    t_read = best(lambda: S.spa_probe_read(buf, read_wg, sink_i))
    flops = mfma_wg * 4 * PROBE_MFMA_ITERS * S.PROBE_MFMA_FLOPS_PER_WAVE_ROUND
    t_mfma = best(lambda: S.spa_probe_mfma_bf16(mfma_wg, PROBE_MFMA_ITERS, sink_f))
    del buf
    torch.cuda.synchronize()
    log("[bench] rate probes done")
    return {"hbm_read_gbs": PROBE_READ_BYTES / t_read / 1e9, "mfma_bf16_tflops": flops / t_mfma / 1e12,
            "read_probe": f"spa_probe_read: {PROBE_READ_BYTES} bytes, 16-byte non-temporal loads, {read_wg} "
                          f"workgroups of 256 threads",
            "mfma_probe": f"spa_probe_mfma_bf16: {mfma_wg} workgroups of four waves, {PROBE_MFMA_ITERS} rounds of "
                          f"four independent 32x32x16 bf16 products",
            "timing": "best of five event-timed calls after one warm-up"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    cfg = config_of(args.workload)
    res = bench_prefill(args, cfg) if args.workload.startswith("prefill") else bench_decode(args, cfg)
    if not args.no_probes:
        rates = achievable_rates()
        res["achievable"] = rates
        r = res["roofline"]
        r["achievable_peak"] = rates["hbm_read_gbs"] if r["bound"] == "hbm" else rates["mfma_bf16_tflops"]
        r["frac_of_achievable"] = r["achieved"] / r["achievable_peak"]
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
