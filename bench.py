"""Throughput of one sparse decode step at 128K context on one MI355X.

A step is the whole decode hot path for one attention layer over one batch:
int8 indexer scores and dual top-p selection (one fused launch) -> split
sparse flash-decode and its log-sum-exp merge.  Workload: B = 16 sequences of 131072 tokens, 64 query
heads over 8 KV heads, d = 128, 64-token blocks, top-p 0.9 over softmax(s/8)
with K_min 16 / K_max 512 plus 1 sink and 4 local blocks (seeded synthetic
inputs, planted relevant blocks per sequence drawn from 1..200).

Prints one JSON line.  value = sequences decoded per second (tokens/s) with
all inputs resident in HBM.  The K/V cache is replicated in `--copies`
buffers that consecutive steps rotate through, so a step cannot be served
from the 256 MB Infinity Cache left warm by the previous one.

roofline: the dominant op is the sparse attention (main kernel + merge);
its algorithmic bytes (selected K/V rows, Q, O, lse, the block list) over
its event-timed duration, against 8 TB/s.
cpu_baseline: the CPU oracle (numpy fp64) on the same inputs, one full step.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-decode tokens/s at 128K ctx (1 GPU); achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "decode_128k_traffic.json"))
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this size before the timed steps (counter calibration)")
    return ap.parse_args()


def attn_bytes(cfg, counts, seq_len) -> int:
    """Algorithmic HBM bytes of one sparse attention launch.

    Selected K and V rows (bf16) of every KV head, clipped to the sequence,
    plus Q (bf16), O (fp32), lse (fp32), the block lists and counts (int32).
    """
    tok = 0
    for b, c in enumerate(counts):
        tok += int(c) * cfg.blk  # every selected block is a whole block in this workload
    kv = tok * cfg.Hkv * cfg.d * 2 * 2
    q = cfg.B * cfg.Hq * cfg.d * 2
    o = cfg.B * cfg.Hq * cfg.d * 4
    lse = cfg.B * cfg.Hq * 4
    idx = int(sum(int(c) for c in counts)) * 4 + cfg.B * 4 * 2
    return kv + q + o + lse + idx


def index_bytes(cfg) -> int:
    """Algorithmic bytes of scoring + selection: kI, qI, w, scores written and read."""
    return cfg.B * (cfg.nb * cfg.H_idx * cfg.r + cfg.H_idx * (cfg.r + 1) + cfg.nb * 4 * 2)


def cpu_baseline(inp, cfg):
    """Time the CPU oracle on one full decode step (all sequences)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle as O
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    t0 = time.perf_counter()
    O.decode_step(inp)
    dt = time.perf_counter() - t0
    reps = 1
    # repeat to roughly 10 s of CPU work, bounded
    while time.perf_counter() - t0 < 10.0 and reps < 20:
        O.decode_step(inp)
        reps += 1
    dt = (time.perf_counter() - t0) / reps
    return {"value": cfg.B / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"full decode step of all {cfg.B} sequences (score, top-p, fp64 attention), "
                      f"mean of {reps} runs, {dt:.3f} s each"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import block_sparse_long_int8_amd as S
    import gen

    cfg = gen.DECODE_128K_TOPP
    t0 = time.time()
    inp = gen.make(cfg, seed=args.seed)
    log(f"[bench] generated {cfg.name} in {time.time() - t0:.1f} s")

    torch.cuda.set_device(0)

    def dev(x, dt=None):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    q = dev(inp["q"], "bf16")
    k0 = dev(inp["k"], "bf16")
    v0 = dev(inp["v"], "bf16")
    ks = [k0] + [k0.clone() for _ in range(args.copies - 1)]
    vs = [v0] + [v0.clone() for _ in range(args.copies - 1)]
    qI, kI, w, seq_len = dev(inp["qI"]), dev(inp["kI"]), dev(inp["w"]), dev(inp["seq_len"])
    torch.cuda.synchronize()
    log(f"[bench] inputs resident: {args.copies} copies of the {2 * k0.numel() * 2 / 2**30:.1f} GiB K/V cache")

    spec = S.DecodeSpec(B=cfg.B, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d, Tcap=cfg.T, blk=cfg.blk, H_idx=cfg.H_idx,
                        r=cfg.r, n_sink=cfg.n_sink, n_local=cfg.n_local, select="topp", beta=cfg.beta, p=cfg.p,
                        k_min=cfg.k_min, k_max=cfg.k_max)
    step = S.DecodeStep(spec)

    def run(i, ev=None):
        c = i % args.copies
        if ev is not None:
            ev[0].record()
        step.score_select(qI, kI, w, seq_len)
        if ev is not None:
            ev[1].record()
        step.attend(q, ks[c], vs[c], seq_len)
        if ev is not None:
            ev[2].record()

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] calibration copy of {args.copy_calibration_mib} MiB done")

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for i in range(args.steps):
        run(args.warmup + i, evs[i])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / args.steps
    select_ms = [e[0].elapsed_time(e[1]) for e in evs]
    attn_ms = [e[1].elapsed_time(e[2]) for e in evs]
    log(f"[bench] timed {args.steps} steps: {total_ms:.3f} ms on events, {wall * 1e3:.3f} ms wall")

    counts = step.count.cpu().numpy()
    ab = attn_bytes(cfg, counts, inp["seq_len"])
    attn_avg_s = float(np.mean(attn_ms)) * 1e-3
    achieved = ab / attn_avg_s / 1e9
    traffic = None
    if os.path.exists(args.traffic_json):
        with open(args.traffic_json) as f:
            tj = json.load(f)
        if tj.get("kernel_source_sha") == _kernel_sha():
            traffic = tj.get("traffic_bytes_per_launch")

    res = {
        "metric": METRIC,
        "value": cfg.B / (ms_step * 1e-3),
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
                   "blk": cfg.blk, "H_idx": cfg.H_idx, "r": cfg.r, "select": "top-p", "p": cfg.p, "beta": cfg.beta,
                   "k_min": cfg.k_min, "k_max": cfg.k_max, "n_sink": cfg.n_sink, "n_local": cfg.n_local,
                   "kv_copies_rotated": args.copies, "seed": args.seed},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "spa_sparse_decode_attn (decode_bf16_kernel + decode_merge_kernel)",
                     "algorithmic_bytes_per_launch": ab, "avg_launch_ms": attn_avg_s * 1e3},
        "stages_ms": {"score_select_topp": float(np.mean(select_ms)), "attention": float(np.mean(attn_ms))},
        "selected_blocks": {"mean": float(counts.mean()), "min": int(counts.min()), "max": int(counts.max())},
        "step_algorithmic_bytes": ab + index_bytes(cfg),
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        res["cpu_baseline"] = cpu_baseline(inp, cfg)
    print(json.dumps(res), flush=True)


def _kernel_sha() -> str:
    import hashlib
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "block_sparse_long_int8_amd", "csrc", "decode_attn.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
