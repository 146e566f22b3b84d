"""Benchmark of the real-time expert load-balancing path on one MI355X.

One step = one pass of the whole per-layer path over one batch of a Qwen3-235B-shaped
MoE layer simulated as R = 32 virtual EP ranks on one GPU (128 experts, 8192 tokens
per rank, top-8, hidden 4096 bf16, 1 redundant slot per rank, minimum quota 1024):

    load matrix -> quota solve -> reroute + token assignment (all ranks)
    -> forward staging of every used redundant slot (3 x 4096 x 1536 bf16 each)
    -> permute of every rank's activations into the dispatch buffer

value = tokens of the whole EP group per second (R * T / step time), inputs resident
in HBM.  The JSON line also carries the permute kernel's roofline (algorithmic bytes
per launch / its event-timed average duration), the per-rank share of a layer in us
(plan + one rank's permute + its slot staging), and the CPU oracle's throughput on a
bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "balance-plan+permute µs/layer and tokens/s; permute/stage HBM GB/s (% peak)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Layer:
    """Preallocated device buffers of one layer (the library never allocates)."""

    def __init__(self, U, W, torch, w, ids):
        dev = "cuda:0"
        self.U, self.w = U, w
        R, T, K, E, S, H = w.R, w.T, w.K, w.E, w.S, w.H
        i32 = dict(dtype=torch.int32, device=dev)
        self.ids = torch.from_numpy(ids).to(dev)
        self.counts = torch.empty(R, E, **i32)
        self.bp = torch.empty(R, T, K, **i32)
        self.lm_ws = torch.empty(max(U.load_matrix_workspace_size(R, T, K, E), 4), dtype=torch.uint8,
                                 device=dev)
        ipr = E // R + S
        self.ipr = ipr
        self.plan = {"slot_expert": torch.empty(R, S, **i32), "inst_expert": torch.empty(R * ipr, **i32),
                     "inst_quota": torch.empty(R * ipr, **i32), "rank_load": torch.empty(R, **i32),
                     "stats": torch.empty(4, **i32)}
        self.xfer = torch.empty(R, R * ipr, **i32)
        self.ioff = torch.empty(R * ipr + 1, **i32)
        self.dinst = torch.empty(R, T, K, **i32)
        self.drow = torch.empty(R, T, K, **i32)
        self.rr_ws = torch.empty(max(U.reroute_workspace_size(R, E, ipr), 4), dtype=torch.uint8,
                                 device=dev)
        self.err = torch.zeros(1, **i32)
        gen = torch.Generator(device=dev).manual_seed(W.tensor_seed(w, 0, 0))
        self.x = torch.randn(R, T, H, generator=gen, device=dev).to(torch.bfloat16)
        self.out = torch.empty(w.P, H, dtype=torch.bfloat16, device=dev)
        self.row_src = torch.empty(w.P, **i32)
        gen = torch.Generator(device=dev).manual_seed(W.tensor_seed(w, 0, 1))
        self.main_w = (torch.randn(E, w.expert_elems, generator=gen, device=dev) * 0.02).to(torch.bfloat16)
        self.slot_w = torch.empty(R, S, w.expert_elems, dtype=torch.bfloat16, device=dev)

    def plan_step(self, stream):
        U, w = self.U, self.w
        U.load_matrix(self.ids, w.E, self.counts, self.bp, None, self.lm_ws, stream)
        U.solve_quota(self.counts, w.S, w.q_min, out=self.plan, stream=stream)
        U.reroute_assign(self.counts, self.ids, self.bp, self.ipr, self.plan["inst_expert"],
                         self.plan["inst_quota"], 0, w.R, self.xfer, self.ioff, self.dinst, self.drow,
                         None, self.rr_ws, stream)

    def plan_step_rank(self, stream, r):
        U, w = self.U, self.w
        U.load_matrix(self.ids, w.E, self.counts, self.bp, None, self.lm_ws, stream)
        U.solve_quota(self.counts, w.S, w.q_min, out=self.plan, stream=stream)
        U.reroute_assign(self.counts, self.ids, self.bp, self.ipr, self.plan["inst_expert"],
                         self.plan["inst_quota"], r, r + 1, self.xfer, self.ioff, self.dinst,
                         self.drow, None, self.rr_ws, stream)

    def stage(self, stream, r_begin=0, r_end=None):
        w = self.w
        self.U.stage_replica_weights(self.U.STAGE_WEIGHTS, w.R, w.E, w.S, self.plan["slot_expert"],
                                     w.expert_elems, main_w=self.main_w, slot_w=self.slot_w,
                                     r_begin=r_begin, r_end=r_end, stream=stream)

    def permute(self, stream, r_begin=0, r_end=None):
        self.U.permute(self.x, self.drow, self.out, self.row_src, r_begin, r_end, stream)


def cpu_baseline(w, ids, x_host, slot_expert, n_rank_sample=2):
    """The oracle as it stands, single process, on a bounded sample of the same layer:
    the whole plan (load matrix, quota solve, reroute, assignment) plus the permute of
    n_rank_sample ranks and the staging of one used slot, scaled to the whole layer."""
    import oracle as O
    t0 = time.perf_counter()
    counts, bp = O.load_matrix(ids, w.E)
    plan = O.solve_quota(counts, w.S, w.q_min)
    X, io, so = O.reroute(counts, plan["inst_expert"], plan["inst_quota"], plan["inst_per_rank"])
    _, dr = O.assign(ids, bp, X, plan["inst_expert"], plan["inst_per_rank"], io, so)
    t_plan = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.permute(x_host, dr, 0, n_rank_sample, w.P)
    t_perm = (time.perf_counter() - t0) * w.R / n_rank_sample
    used = [(r, s) for r in range(w.R) for s in range(w.S) if plan["slot_expert"][r, s] >= 0]
    n = w.expert_elems
    mw = np.zeros((w.E, n), dtype=np.uint16)
    sw = np.zeros((w.R, w.S, n), dtype=np.uint16)
    one = np.full((w.R, w.S), -1, dtype=np.int64)
    if used:
        one[used[0]] = plan["slot_expert"][used[0]]
    t0 = time.perf_counter()
    O.stage_forward(one, mw, sw)
    t_stage = (time.perf_counter() - t0) * len(used)
    total = t_plan + t_perm + t_stage
    return {
        "value": w.N / total, "unit": "tokens/s", "cores": 1, "kind": "oracle",
        "sample": (f"whole-layer plan ({t_plan:.2f} s) + permute of {n_rank_sample} of {w.R} ranks "
                   f"scaled x{w.R // n_rank_sample} ({t_perm:.2f} s) + staging of 1 of {len(used)} "
                   f"used slots scaled ({t_stage:.2f} s); Python+numpy, one thread"),
        "seconds_per_layer": total,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the EP group is simulated as virtual ranks on a "
              "single device, so --gpus above 1 is not supported.", file=sys.stderr)
        sys.exit(2)
    os.environ.setdefault("OMP_NUM_THREADS", "1")

    import torch
    from moe_expert_load_amd import uep as U
    from moe_expert_load_amd import workload as W

    w = W.QWEN_LAYER
    log(f"workload {w.name}: R={w.R} E={w.E} S={w.S} T={w.T} K={w.K} H={w.H}")
    ids = W.routing(w)
    L = Layer(U, W, torch, w, ids)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    # warmup
    for _ in range(args.warmup):
        L.plan_step(stream)
        L.stage(stream)
        L.permute(stream)
    torch.cuda.synchronize()

    # timed region: K whole steps; per-kernel events around permute and staging
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    p_ev = [(ev(), ev()) for _ in range(args.steps)]
    s_ev = [(ev(), ev()) for _ in range(args.steps)]
    q_ev = [(ev(), ev()) for _ in range(args.steps)]
    t_start, t_end = ev(), ev()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for k in range(args.steps):
        q_ev[k][0].record(stream)
        L.plan_step(stream)
        q_ev[k][1].record(stream)
        s_ev[k][0].record(stream)
        L.stage(stream)
        s_ev[k][1].record(stream)
        p_ev[k][0].record(stream)
        L.permute(stream)
        p_ev[k][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    perm_ms = float(np.mean([a.elapsed_time(b) for a, b in p_ev]))
    stage_ms = float(np.mean([a.elapsed_time(b) for a, b in s_ev]))
    plan_ms = float(np.mean([a.elapsed_time(b) for a, b in q_ev]))
    stats = L.plan["stats"].cpu().numpy()
    n_used = int(stats[0])
    perm_bytes = w.N * w.H * 2 + w.P * w.H * 2 + w.P * 4
    stage_bytes = 2 * n_used * w.expert_elems * 2
    perm_gbs = perm_bytes / (perm_ms * 1e-3) / 1e9
    stage_gbs = stage_bytes / (stage_ms * 1e-3) / 1e9 if n_used else 0.0

    # per-rank share: plan of the whole group + one rank's assignment, permute and slot
    r = 0
    n_rep = 50
    a, b = ev(), ev()
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(n_rep):
        L.plan_step_rank(stream, r)
        L.stage(stream, r, r + 1)
        L.permute(stream, r, r + 1)
    b.record(stream)
    torch.cuda.synchronize()
    rank_us = a.elapsed_time(b) / n_rep * 1e3
    a2, b2 = ev(), ev()
    a2.record(stream)
    for _ in range(n_rep):
        L.plan_step(stream)
    b2.record(stream)
    torch.cuda.synchronize()
    plan_us = a2.elapsed_time(b2) / n_rep * 1e3
    rl = L.plan["rank_load"].cpu().numpy()
    c = L.counts.cpu().numpy().sum(0)
    before = c.reshape(w.R, w.E_loc).sum(1)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        x_host = L.x.view(torch.int16).cpu().numpy().view(np.uint16)
        cpu = cpu_baseline(w, ids, x_host, L.plan["slot_expert"].cpu().numpy())
        cpu.pop("seconds_per_layer")

    out = {
        "metric": METRIC,
        "value": w.N / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic",
        "config": {"workload": w.name, "R": w.R, "E": w.E, "S": w.S, "tokens_per_rank": w.T,
                   "top_k": w.K, "hidden": w.H, "q_min": w.q_min, "ffn": list(w.ffn_shape),
                   "zipf_s": round(W.zipf_exponent(w, 0), 4), "parallelism": "ep32 virtual ranks on 1 GPU"},
        "roofline": {"bound": "hbm", "kernel": "permute_kernel", "achieved": perm_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": perm_gbs / HBM_PEAK_GBS,
                     "traffic": None, "algorithmic_bytes_per_launch": perm_bytes,
                     "avg_launch_ms": perm_ms},
        "cpu_baseline": cpu,
        "extra": {
            "us_per_layer_rank_share": rank_us,
            "plan_us": plan_us,
            "plan_ms_in_step": plan_ms,
            "stage_ms": stage_ms,
            "stage_gbs": stage_gbs,
            "stage_frac": stage_gbs / HBM_PEAK_GBS,
            "replicas": n_used,
            "solver_steps": int(stats[1]),
            "imbalance_before": float(before.max() / before.mean()),
            "imbalance_after": float(rl.max() / rl.mean()),
            "wall_s_timed": wall,
        },
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
