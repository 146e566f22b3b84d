"""Benchmark of the real-time expert load-balancing path on one MI355X.

Default (the contract line): one step = one pass of the whole per-layer path over one
batch of a Qwen3-235B-shaped MoE layer simulated as R = 32 virtual EP ranks on one GPU
(128 experts, 8192 tokens per rank, top-8, hidden 4096 bf16, 1 redundant slot per
rank, minimum quota 1024):

    load matrix -> quota solve -> reroute + token assignment (all ranks)
    -> forward staging of every used redundant slot (3 x 4096 x 1536 bf16 each)
    -> permute of every rank's activations into the dispatch buffer

value = tokens of the whole EP group per second (R * T / step time), inputs resident
in HBM.  The line also carries the permute kernel's roofline (algorithmic bytes per
launch / its event-timed average duration inside the timed region), the per-rank share
of a layer in us (whole-group plan + one rank's assignment, permute and slot staging,
replayed from a HIP graph so host launch overhead is not counted), and the CPU
oracle's throughput on a bounded sample of the same workload.

Other workloads (one JSON line each, not the contract line):
  --workload tiny | dsv3_waterfill | lplb_layer | qwen3_235b_94layer_sweep
--kernels prints a per-kernel timing table (graph-replayed) of every workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--workload NAME] [--kernels]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# The CPU leg times the oracle on one thread: pin every BLAS / OpenMP pool before numpy
# (or torch) loads one.  The GPU legs do no host compute that these pools would serve.
for _var in ("OMP_NUM_THREADS", "MKL_NUM_THREADS", "OPENBLAS_NUM_THREADS", "BLIS_NUM_THREADS",
             "NUMEXPR_NUM_THREADS"):
    os.environ.setdefault(_var, "1")

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "balance-plan+permute µs/layer and tokens/s; permute/stage HBM GB/s (% peak)"
DEV = "cuda:0"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- helpers
class Timer:
    """Event pairs on one stream; mean duration in ms."""

    def __init__(self, torch, n):
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(n)]
        self.k = 0

    def start(self, stream):
        self.ev[self.k][0].record(stream)

    def stop(self, stream):
        self.ev[self.k][1].record(stream)
        self.k += 1

    def mean_ms(self):
        return float(np.mean([a.elapsed_time(b) for a, b in self.ev[:self.k]]))

    def all_ms(self):
        return [a.elapsed_time(b) for a, b in self.ev[:self.k]]


def graph_us(torch, fn, reps=20, replays=5, indexed=False):
    """Mean GPU time of fn() in us: fn is captured `reps` times into one HIP graph and
    the graph is replayed; host launch overhead is not counted.  With indexed=True,
    fn(stream, i) gets the repetition index, so per-rank work can rotate over ranks and
    no repetition re-reads the previous one's inputs from the 256 MB last-level cache."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(s, 0) if indexed else fn(s)           # warm (first-call setup outside the graph)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(reps):
            fn(s, i) if indexed else fn(s)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream()
    a.record(cur)
    for _ in range(replays):
        g.replay()
    b.record(cur)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (reps * replays)


class Layer:
    """Preallocated device buffers of one layer (the library never allocates)."""

    def __init__(self, U, W, torch, w, ids, E=None, K=None, ipr=None, weights=True):
        self.U, self.w, self.torch = U, w, torch
        R, T, H = w.R, w.T, w.H
        E = w.E if E is None else E
        K = w.K if K is None else K
        self.E, self.K = E, K
        i32 = dict(dtype=torch.int32, device=DEV)
        self.ids = torch.from_numpy(np.ascontiguousarray(ids)).to(DEV) if ids is not None else \
            torch.empty(R, T, K, **i32)
        self.counts = torch.empty(R, E, **i32)
        self.bp = torch.empty(R, T, K, **i32)
        self.lm_ws = torch.empty(max(U.load_matrix_workspace_size(R, T, K, E), 4),
                                 dtype=torch.uint8, device=DEV)
        self.ipr = (E // R + w.S) if ipr is None else ipr
        I = R * self.ipr
        self.plan = {"slot_expert": torch.full((R, max(w.S, 1)), -1, **i32),
                     "inst_expert": torch.empty(I, **i32), "inst_quota": torch.empty(I, **i32),
                     "rank_load": torch.empty(R, **i32), "stats": torch.zeros(4, **i32)}
        self.xfer = torch.empty(R, I, **i32)
        self.ioff = torch.empty(I + 1, **i32)
        self.dinst = torch.empty(R, T, K, **i32)
        self.drow = torch.empty(R, T, K, **i32)
        self.rr_ws = torch.empty(max(U.reroute_workspace_size(R, E, self.ipr), 4),
                                 dtype=torch.uint8, device=DEV)
        self.plan_ws = torch.empty(max(U.plan_workspace_size(R, T, K, E, max(w.S, 0)), 4),
                                   dtype=torch.uint8, device=DEV)
        gen = torch.Generator(device=DEV).manual_seed(W.tensor_seed(w, 0, 0))
        self.x = torch.randn(R, T, H, generator=gen, device=DEV, dtype=torch.bfloat16)
        self.P = R * T * K
        self.out = torch.empty(self.P, H, dtype=torch.bfloat16, device=DEV)
        self.row_src = torch.empty(self.P, **i32)
        if weights and w.S > 0:
            gen = torch.Generator(device=DEV).manual_seed(W.tensor_seed(w, 0, 1))
            self.main_w = (torch.randn(w.E, w.expert_elems, generator=gen, device=DEV,
                                       dtype=torch.bfloat16) * 0.02)
            self.slot_w = torch.empty(R, w.S, w.expert_elems, dtype=torch.bfloat16, device=DEV)

    # the steps of the path
    def load(self, s):
        self.U.load_matrix(self.ids, self.E, self.counts, self.bp, None, self.lm_ws, s)

    def solve(self, s):
        self.U.solve_quota(self.counts, self.w.S, self.w.q_min, out=self.plan, stream=s)

    def reroute(self, s, r_begin=0, r_end=None):
        self.U.reroute_assign(self.counts, self.ids, self.bp, self.ipr, self.plan["inst_expert"],
                              self.plan["inst_quota"], r_begin, r_end, self.xfer, self.ioff,
                              self.dinst, self.drow, None, self.rr_ws, s)

    def stage(self, s, r_begin=0, r_end=None):
        w = self.w
        self.U.stage_replica_weights(self.U.STAGE_WEIGHTS, w.R, w.E, w.S, self.plan["slot_expert"],
                                     w.expert_elems, main_w=self.main_w, slot_w=self.slot_w,
                                     r_begin=r_begin, r_end=r_end, stream=s)

    def permute(self, s, r_begin=0, r_end=None, row_src=True):
        self.U.permute(self.x, self.drow, self.out, self.row_src if row_src else None,
                       r_begin, r_end, s)

    def plan_step(self, s, r_begin=0, r_end=None):
        """The layer's plan in one uep_plan call (the solve overlapped with the ranking)."""
        out = {"counts": self.counts, "bucket_pos": self.bp, "xfer": self.xfer,
               "inst_offset": self.ioff, "dest_inst": self.dinst, "dest_row": self.drow,
               **{k: self.plan[k] for k in ("slot_expert", "inst_expert", "inst_quota",
                                            "rank_load", "stats")}}
        self.U.plan(self.ids, self.E, self.w.S, self.w.q_min, r_begin, r_end, out, None,
                    self.plan_ws, s)

    def plan_separate(self, s, r_begin=0, r_end=None):
        """The same plan as three calls: load matrix, quota solve, reroute/assignment."""
        self.load(s)
        self.solve(s)
        self.reroute(s, r_begin, r_end)


def permute_bytes(N, P, H):
    """Algorithmic bytes of one whole-group permute: every source row read once, every
    dispatch row written once, plus the 4-byte row_src entry of every row."""
    return N * H * 2 + P * H * 2 + P * 4


PERMUTE_CALL = ("prefetch_kernel + permute_kernel per chunk of at most 224 MiB of source rows, "
                "then row_src_kernel (one uep_permute call)")
PERMUTE_SOURCES = ("moe_expert_load_amd/csrc/permute.hip", "moe_expert_load_amd/csrc/common.h")


def source_digest(paths=PERMUTE_SOURCES):
    """sha256 over the kernel's source files: ties stored counter figures to the code."""
    import hashlib
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the permute call from the committed counter summary
    profiles/permute_<workload>_pmc.md, or None when there is none or the permute
    sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"permute_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if line.startswith("- ") and " = " in line:
            k, v = line[2:].split(" = ", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha256") != source_digest():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def combine_bytes(N, P, H):
    """Algorithmic bytes of one whole-group combine: every dispatch row read once,
    every token row written once, plus each pair's row index and weight."""
    return N * H * 2 + P * H * 2 + P * 8


def roofline(bytes_, ms, kernel, traffic=None):
    gbs = bytes_ / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": gbs, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": traffic,
            "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_bytes_per_launch": bytes_, "avg_launch_ms": ms}


def grad_reduce_figures(torch, U, L, reps=3):
    """Backward replica-gradient reduction (fp32) on the step's plan, event-timed.
    Algorithmic bytes: per replicated expert its main gradient read and written once,
    per replica its gradient read once and zeroed once."""
    w = L.w
    se = L.plan["slot_expert"][:, :w.S].contiguous()
    gen = torch.Generator(device=DEV).manual_seed(17)
    main_grad = torch.zeros(w.E, w.expert_elems, dtype=torch.float32, device=DEV)
    slot_grad = torch.randn(w.R, w.S, w.expert_elems, generator=gen, dtype=torch.float32,
                            device=DEV)
    sh = se.cpu().numpy()
    reps_of = {}
    for e in sh[sh >= 0]:
        reps_of[int(e)] = reps_of.get(int(e), 0) + 1
    nbytes = sum((2 + 2 * n) * w.expert_elems * 4 for n in reps_of.values())
    s = torch.cuda.current_stream()
    t = Timer(torch, reps)
    for _ in range(reps):
        t.start(s)
        U.stage_replica_weights(U.STAGE_GRAD_REDUCE, w.R, w.E, w.S, se, w.expert_elems,
                                main_grad=main_grad, slot_grad=slot_grad, stream=s)
        t.stop(s)
    torch.cuda.synchronize()
    ms = t.mean_ms()
    del main_grad, slot_grad
    torch.cuda.empty_cache()
    gbs = nbytes / (ms * 1e-3) / 1e9 if nbytes else 0.0
    return {"grad_reduce_ms": ms, "grad_reduce_gbs": gbs, "grad_reduce_frac": gbs / HBM_PEAK_GBS,
            "replicated_experts": len(reps_of)}


def launch_floor(torch, U, n=1000):
    """The launch floor the latency-bound kernels are read against: the library's
    smallest launch (a 16-byte uep_device_copy, one workgroup) on the bench stream,
    as the mean of graph-replayed back-to-back launches and as the median of n
    event-timed single launches."""
    a = torch.zeros(4, dtype=torch.int32, device=DEV)
    b = torch.empty_like(a)
    graph = graph_us(torch, lambda st: U.device_copy(a, b, st), reps=100, replays=10)
    s = torch.cuda.current_stream()
    t = Timer(torch, n)
    for _ in range(n):
        t.start(s)
        U.device_copy(a, b, s)
        t.stop(s)
    torch.cuda.synchronize()
    return {"launch_floor_us_graph": graph,
            "launch_floor_us_event_median": float(np.median(t.all_ms()) * 1e3)}


def copy_reference(torch, U, nbytes=1 << 30, reps=5):
    """Event-timed plain device copy (uep_device_copy) of nbytes: the achievable
    bandwidth line, and the known-size kernel that calibrates byte counters."""
    a = torch.empty(nbytes // 2, dtype=torch.int16, device=DEV)
    b = torch.empty_like(a)
    s = torch.cuda.current_stream()
    U.device_copy(a, b, s)
    torch.cuda.synchronize()
    t = Timer(torch, reps)
    for _ in range(reps):
        t.start(s)
        U.device_copy(a, b, s)
        t.stop(s)
    torch.cuda.synchronize()
    ms = t.mean_ms()
    del a, b
    torch.cuda.empty_cache()
    return {"bytes_per_launch": 2 * nbytes, "avg_launch_ms": ms,
            "gbs": 2 * nbytes / (ms * 1e-3) / 1e9}


def fill_reference(torch, U, nbytes=1 << 30, reps=5):
    """Event-timed uep_device_fill of nbytes: the write-only bandwidth line (the permute
    and staging streams are mostly writes)."""
    a = torch.empty(nbytes // 4, dtype=torch.int32, device=DEV)
    s = torch.cuda.current_stream()
    U.device_fill(a, 0, s)
    torch.cuda.synchronize()
    t = Timer(torch, reps)
    for _ in range(reps):
        t.start(s)
        U.device_fill(a, 0x01010101, s)
        t.stop(s)
    torch.cuda.synchronize()
    ms = t.mean_ms()
    del a
    torch.cuda.empty_cache()
    return {"bytes_per_launch": nbytes, "avg_launch_ms": ms, "gbs": nbytes / (ms * 1e-3) / 1e9}


def sequential_permute_line(torch, U, L, perm_ms, reps=5):
    """The same uep_permute call on the layer's own x and dispatch buffers, with
    destination rows t*K + k: the same bytes as the real permute, written as one fully
    sequential stream.  How fast HBM takes the permute's traffic depends on where the
    driver placed these buffers (the same kernel varies by up to a third between fresh
    allocations), so the permute is judged against this line from the same process and
    the same memory.  Returns its rate and the permute's fraction of it."""
    R, T, K = L.dinst.shape
    H = L.x.shape[2]
    dseq = torch.arange(R * T * K, dtype=torch.int32, device=DEV).view(R, T, K)
    rs = torch.empty(R * T * K, dtype=torch.int32, device=DEV)
    s = torch.cuda.current_stream()
    U.permute(L.x, dseq, L.out, rs, 0, None, s)
    torch.cuda.synchronize()
    t = Timer(torch, reps)
    for _ in range(reps):
        t.start(s)
        U.permute(L.x, dseq, L.out, rs, 0, None, s)
        t.stop(s)
    torch.cuda.synchronize()
    ms = t.mean_ms()
    del dseq, rs
    torch.cuda.empty_cache()
    return {"sequential_permute_gbs": permute_bytes(R * T, R * T * K, H) / (ms * 1e-3) / 1e9,
            "permute_over_sequential": ms / perm_ms}


def base_line(w, W, value, ms, args, dtype, extra_cfg=None):
    cfg = {"workload": w.name, "R": w.R, "E": w.E, "S": w.S, "tokens_per_rank": w.T,
           "top_k": w.K, "hidden": w.H, "q_min": w.q_min,
           "zipf_s": round(W.zipf_exponent(w, 0), 4), "parallelism": f"ep{w.R} virtual ranks on 1 GPU"}
    if extra_cfg:
        cfg.update(extra_cfg)
    return {"metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "data": "synthetic", "config": cfg}


def timed_steps(torch, args, step, stream, timers=()):
    for _ in range(args.warmup):
        step(stream, None)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(args.steps):
        step(stream, timers)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / args.steps


def combine_figures(torch, U, W, L, reps=5):
    """Combine (the step after the experts: dispatch rows back to token order with the
    router weights), timed outside the step: whole group event-timed, one rank's share
    graph-replayed.  Its input here is the permuted buffer of the step."""
    w = L.w
    gen = torch.Generator(device=DEV).manual_seed(W.tensor_seed(w, 0, 5))
    gate = torch.rand(w.R, w.T, L.K, generator=gen, device=DEV)
    y = torch.empty(w.R, w.T, w.H, dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.current_stream()
    U.combine(L.out, L.drow, gate, y, stream=s)
    torch.cuda.synchronize()
    t = Timer(torch, reps)
    for _ in range(reps):
        t.start(s)
        U.combine(L.out, L.drow, gate, y, stream=s)
        t.stop(s)
    torch.cuda.synchronize()
    ms = t.mean_ms()
    rank_us = graph_us(torch, lambda st, i: U.combine(L.out, L.drow, gate, y, i % w.R,
                                                      i % w.R + 1, stream=st), indexed=True)
    cb = combine_bytes(w.N, L.P, w.H)
    del y, gate
    torch.cuda.empty_cache()
    return {"combine_ms": ms, "combine_gbs": cb / (ms * 1e-3) / 1e9,
            "combine_frac": cb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "combine_rank_us": rank_us}


# ----------------------------------------------------------------------------- CPU leg
def host_cpu():
    """CPU model name (lscpu's, else /proc/cpuinfo's), logical CPUs, and the threads the
    numpy / BLAS / OpenMP pools of this process actually hold."""
    import subprocess
    model = "unknown"
    try:
        r = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10)
        for line in r.stdout.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    if model == "unknown":
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
    threads = 1
    try:
        from threadpoolctl import threadpool_info
        pools = threadpool_info()
        threads = max([p.get("num_threads", 1) for p in pools] + [1])
    except ImportError:
        pools = []
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "pool_threads": threads,
            "pools": sorted({p.get("internal_api", "?") for p in pools})}


def _one_thread(fn):
    """Run a CPU leg with every BLAS / OpenMP pool limited to one thread (threadpoolctl),
    on top of the environment pins set before numpy loaded."""
    def run(*a, **k):
        try:
            from threadpoolctl import threadpool_limits
        except ImportError:
            return fn(*a, **k)
        with threadpool_limits(limits=1):
            return fn(*a, **k)
    run.__doc__ = fn.__doc__
    return run


def _median_s(fn, runs=3):
    """Median wall-clock seconds of `runs` calls of fn (its last result kept in fn.last)."""
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn.last = fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def _cpu_line(value, per_step_s, sample, host):
    return {"value": value, "unit": "tokens/s", "cores": host["pool_threads"], "kind": "oracle",
            "sample": sample, "per_step_ms_median": {k: v * 1e3 for k, v in per_step_s.items()},
            "host": host}


@_one_thread
def cpu_baseline_layer(w, ids, x_host, runs=3):
    """The oracle as it stands, one thread, on the Qwen layer: each step of the path
    (load matrix, quota solve, reroute + assignment, whole-group permute, staging of every
    used slot, backward gradient reduction of the plan) timed `runs` times, median.  value
    = tokens per second of the forward step (load matrix + solve + reroute/assign +
    permute + staging), the GPU step's content."""
    import oracle as O
    n = w.expert_elems
    host = host_cpu()
    t = {}
    f = lambda: O.load_matrix(ids, w.E)                              # noqa: E731
    t["load_matrix"] = _median_s(f, runs)
    counts, bp = f.last
    f = lambda: O.solve_quota(counts, w.S, w.q_min)                  # noqa: E731
    t["solve_quota"] = _median_s(f, runs)
    plan = f.last
    ie, ipr = plan["inst_expert"], plan["inst_per_rank"]

    def rr():
        X, io, so = O.reroute(counts, ie, plan["inst_quota"], ipr)
        return O.assign(ids, bp, X, ie, ipr, io, so)[1]
    t["reroute_assign"] = _median_s(rr, runs)
    dr = rr.last
    f = lambda: O.permute(x_host, dr, 0, w.R, w.P)[1]                 # noqa: E731
    t["permute"] = _median_s(f, runs)
    se = plan["slot_expert"]
    rep = sorted(set(int(e) for e in se.reshape(-1) if e >= 0))
    # staging and the reduction on the touched expert rows only (the others are never read)
    remap = {e: i for i, e in enumerate(rep)}
    se_c = np.vectorize(lambda e: remap.get(int(e), -1))(se).astype(np.int64)
    rng = np.random.default_rng(5)
    main_w = rng.integers(0, 1 << 16, (len(rep), n), dtype=np.uint16)
    slot_w = np.zeros((w.R, w.S, n), dtype=np.uint16)
    t["stage_forward"] = _median_s(lambda: O.stage_forward(se_c, main_w, slot_w), runs)
    del main_w, slot_w
    main_g = rng.standard_normal((len(rep), n), dtype=np.float32)
    slot_g = rng.standard_normal((w.R, w.S, n), dtype=np.float32)
    t["grad_reduce"] = _median_s(lambda: O.grad_reduce(se_c, main_g, slot_g, w.E_loc), runs)
    del main_g, slot_g
    fwd = sum(t[k] for k in ("load_matrix", "solve_quota", "reroute_assign", "permute",
                             "stage_forward"))
    sample = (f"each step of the whole layer {runs} times, median: the forward step (plan, "
              f"permute of all {w.R} ranks, staging of all {int((se >= 0).sum())} used slots) "
              f"{fwd:.2f} s, the backward reduction {t['grad_reduce']:.2f} s; Python+numpy, "
              f"BLAS/OpenMP pinned to one thread")
    return _cpu_line(w.N / fwd, t, sample, host)


@_one_thread
def cpu_baseline_waterfill(w, ids, x_host, inst, ipr, seed, runs=3):
    """The oracle, one thread, on the DeepSeek-V3 Waterfill layer: routed loads, Waterfill,
    the fused (K+1)-column layout's load matrix, identity quotas, reroute + assignment, and
    the whole group's permute (31.5 GiB of dispatch rows, produced in blocks of 131072
    rows from the oracle's row map, each block's time summed), median of `runs`."""
    import oracle as O
    host = host_cpu()
    t = {}
    B = np.full(w.R, w.T, dtype=np.int32)
    f = lambda: O.load_matrix(ids, w.E)[0]                           # noqa: E731
    t["load_matrix_routed"] = _median_s(f, runs)
    counts = f.last
    f = lambda: O.waterfill(counts, ids, B, seed, 0)                  # noqa: E731
    t["waterfill"] = _median_s(f, runs)
    ext = O.extend_topk(ids, f.last[0], w.E)
    E2 = w.E + w.R
    f = lambda: O.load_matrix(ext, E2)                                # noqa: E731
    t["load_matrix_fused"] = _median_s(f, runs)
    c2, bp2 = f.last
    f = lambda: O.identity_quota(c2, inst)                            # noqa: E731
    t["identity_quota"] = _median_s(f, runs)
    q = f.last

    def rr():
        X, io, so = O.reroute(c2, inst, q, ipr)
        return O.assign(ext, bp2, X, inst, ipr, io, so)[1]
    t["reroute_assign"] = _median_s(rr, runs)
    dr = rr.last
    P = int(c2.sum())
    K2 = w.K + 1

    def perm():
        src = O.row_sources(dr, P)
        for a in range(0, P, 1 << 17):
            O.rows_of(x_host, src, K2, a, min(P, a + (1 << 17)))
    t["permute"] = _median_s(perm, runs)
    total = sum(t.values())
    sample = (f"each step of the whole layer {runs} times, median ({total:.2f} s per pass): plan "
              f"{total - t['permute']:.2f} s, permute of all {w.R} ranks into the fused layout "
              f"{t['permute']:.2f} s; Python+numpy, BLAS/OpenMP pinned to one thread")
    return _cpu_line(w.N / total, t, sample, host)


@_one_thread
def cpu_baseline_lplb(w, ids, x_host, inst, ipr, rank_sample=4, runs=3):
    """The oracle, one thread, on the LPLB layer: load matrix, the fp64 simplex and
    largest-remainder quotas, reroute + assignment on those quotas, and the permute of
    `rank_sample` of the R source ranks (their rows produced in blocks from the oracle's
    row map), scaled by R / rank_sample for the whole group; median of `runs`."""
    import oracle as O
    host = host_cpu()
    t = {}
    f = lambda: O.load_matrix(ids, w.E)                               # noqa: E731
    t["load_matrix"] = _median_s(f, runs)
    counts, bp = f.last
    f = lambda: O.lplb(counts, inst, ipr)                             # noqa: E731
    t["lplb_simplex"] = _median_s(f, runs)
    q = f.last["inst_quota"]

    def rr():
        X, io, so = O.reroute(counts, inst, q, ipr)
        return O.assign(ids, bp, X, inst, ipr, io, so)[1]
    t["reroute_assign"] = _median_s(rr, runs)
    dr = rr.last
    sub = np.full_like(dr, -1)
    sub[:rank_sample] = dr[:rank_sample]

    def perm():
        src = O.row_sources(sub, w.P)
        rows = np.nonzero(src >= 0)[0]
        for a in range(0, rows.size, 1 << 17):
            blk = rows[a:a + (1 << 17)]
            O.rows_of(x_host, src[blk], w.K, 0, blk.size)
    t_sample = _median_s(perm, runs)
    t["permute"] = t_sample * w.R / rank_sample
    total = sum(t.values())
    sample = (f"each step {runs} times, median: plan {total - t['permute']:.2f} s for the whole "
              f"layer, permute of {rank_sample} of {w.R} source ranks {t_sample:.2f} s, scaled x"
              f"{w.R // rank_sample} to the group ({t['permute']:.2f} s); Python+numpy, "
              f"BLAS/OpenMP pinned to one thread")
    return _cpu_line(w.N / total, t, sample, host)


@_one_thread
def cpu_baseline_sweep(w, routings, layers=(0, 1, 2, 3), runs=1):
    """The oracle, one thread, on a sample of the sweep's layers: forward (load matrix,
    solve, reroute + assignment, whole-group permute, staging of the layer's slots into
    one shared slot set) and backward (staging again, gradient reduction) per layer;
    per-layer medians and the 94-layer sum scaled from the sample."""
    import oracle as O
    host = host_cpu()
    n = w.expert_elems
    rng = np.random.default_rng(9)
    x_host = rng.integers(0, 1 << 16, (w.R, w.T, w.H), dtype=np.uint16)
    slot_w = np.zeros((w.R, w.S, n), dtype=np.uint16)
    slot_g = np.zeros((w.R, w.S, n), dtype=np.float32)
    fwd, bwd, cached = [], [], []
    for l in layers:
        t0 = time.perf_counter()
        ids = routings[l]
        counts, bp = O.load_matrix(ids, w.E)
        plan = O.solve_quota(counts, w.S, w.q_min)
        ie, ipr = plan["inst_expert"], plan["inst_per_rank"]
        X, io, so = O.reroute(counts, ie, plan["inst_quota"], ipr)
        _, dr = O.assign(ids, bp, X, ie, ipr, io, so)
        O.permute(x_host, dr, 0, w.R, w.P)
        se = plan["slot_expert"]
        rep = sorted(set(int(e) for e in se.reshape(-1) if e >= 0))
        remap = {e: i for i, e in enumerate(rep)}
        se_c = np.vectorize(lambda e: remap.get(int(e), -1))(se).astype(np.int64)
        main_w = rng.integers(0, 1 << 16, (len(rep), n), dtype=np.uint16)
        t1 = time.perf_counter()
        O.stage_forward(se_c, main_w, slot_w)
        fwd.append(time.perf_counter() - t1 + (t1 - t0))
        cached.append((se_c, main_w, len(rep)))
    for se_c, main_w, nrep in reversed(cached):
        main_g = rng.standard_normal((nrep, n), dtype=np.float32)
        slot_g[se_c >= 0] = 1.0
        t0 = time.perf_counter()
        O.stage_forward(se_c, main_w, slot_w)
        O.grad_reduce(se_c, main_g, slot_g, w.E_loc)
        bwd.append(time.perf_counter() - t0)
    f, b = np.array(fwd), np.array(bwd)
    per_layer = float(np.median(f + b[::-1]))
    total = (f.sum() + b.sum()) * w.layers / len(layers)
    t = {"fwd_layer_p50": float(np.median(f)), "fwd_layer_max": float(f.max()),
         "bwd_layer_p50": float(np.median(b)), "bwd_layer_max": float(b.max()),
         "sweep_scaled_from_sample": total}
    sample = (f"layers {list(layers)} of {w.layers}, forward in order then backward in reverse "
              f"through one shared slot set, once each: forward {f.sum():.2f} s, backward "
              f"{b.sum():.2f} s; the {w.layers}-layer sum scaled from the sample is {total:.1f} s; "
              f"Python+numpy, BLAS/OpenMP pinned to one thread")
    return _cpu_line(w.N * w.layers / total, t, sample, host), per_layer


# ----------------------------------------------------------------------------- workloads
def bench_layer(args, torch, U, W, w, with_cpu):
    """UltraEP layer: plan + staging + whole-group permute."""
    log(f"workload {w.name}: R={w.R} E={w.E} S={w.S} T={w.T} K={w.K} H={w.H}")
    ids = W.routing(w)
    L = Layer(U, W, torch, w, ids)
    stream = torch.cuda.current_stream()
    tq, ts, tp = (Timer(torch, args.steps) for _ in range(3))

    def step(s, timers):
        if timers:
            timers[0].start(s)
        L.plan_step(s)
        if timers:
            timers[0].stop(s)
            timers[1].start(s)
        L.stage(s)
        if timers:
            timers[1].stop(s)
            timers[2].start(s)
        L.permute(s)
        if timers:
            timers[2].stop(s)

    ms = timed_steps(torch, args, step, stream, (tq, ts, tp))
    stats = L.plan["stats"].cpu().numpy()
    n_used = int(stats[0])
    pb = permute_bytes(w.N, w.P, w.H)
    perm_ms, stage_ms = tp.mean_ms(), ts.mean_ms()
    se_h = L.plan["slot_expert"].cpu().numpy()
    n_distinct = len(np.unique(se_h[se_h >= 0]))
    # each staged expert's main read once, each used slot written once
    stage_bytes = (n_distinct + n_used) * w.expert_elems * 2
    copy = copy_reference(torch, U)
    fill = fill_reference(torch, U)
    seq = sequential_permute_line(torch, U, L, perm_ms)
    comb = combine_figures(torch, U, W, L)
    floor = launch_floor(torch, U)
    grad = grad_reduce_figures(torch, U, L)
    if args.roofline_only:
        out = base_line(w, W, w.N / (ms * 1e-3), ms, args, "int32", {"ffn": list(w.ffn_shape)})
        out["roofline"] = roofline(pb, perm_ms, PERMUTE_CALL, measured_traffic(w.name))
        out["cpu_baseline"] = None
        out["extra"] = {"device_copy_gbs": copy["gbs"], "device_fill_gbs": fill["gbs"],
                        "stage_ms": stage_ms}
        return out
    # per-rank share, averaged over ranks (repetition i takes rank i mod R): the
    # whole-group plan, that rank's assignment, slot staging and permute

    def rank_share(s, i):
        r = i % w.R
        L.plan_step(s, r, r + 1)
        L.stage(s, r, r + 1)
        L.permute(s, r, r + 1, row_src=False)

    rank_us = graph_us(torch, rank_share, reps=w.R, replays=2, indexed=True)
    plan_us = graph_us(torch, lambda s: L.plan_step(s))
    plan_sep_us = graph_us(torch, lambda s: L.plan_separate(s))
    stage_kernel_us = graph_us(torch, lambda s: L.stage(s), reps=5)
    perm_rank_us = graph_us(torch, lambda s, i: L.permute(s, i % w.R, i % w.R + 1, row_src=False),
                            reps=w.R, replays=2, indexed=True)
    L.plan_step(stream)
    torch.cuda.synchronize()
    rl = L.plan["rank_load"].cpu().numpy()
    c = L.counts.cpu().numpy().sum(0)
    before = c.reshape(w.R, w.E_loc).sum(1)
    out = base_line(w, W, w.N / (ms * 1e-3), ms, args, "int32",
                    {"ffn": list(w.ffn_shape)})
    out["roofline"] = roofline(pb, perm_ms, PERMUTE_CALL, measured_traffic(w.name))
    cpu = None
    if with_cpu:
        log("cpu baseline (oracle) ...")
        x_host = L.x.view(torch.int16).cpu().numpy().view(np.uint16)
        cpu = cpu_baseline_layer(w, ids, x_host)
        del x_host
    out["cpu_baseline"] = cpu
    gpu_steps = {"load_matrix": graph_us(torch, L.load), "solve_quota": graph_us(torch, L.solve),
                 "reroute_assign": graph_us(torch, L.reroute), "permute": perm_ms * 1e3,
                 "stage_forward": stage_kernel_us, "grad_reduce": grad["grad_reduce_ms"] * 1e3}
    rank_bytes = permute_bytes(w.T, w.T * w.K, w.H) - w.T * w.K * 4
    out["extra"] = {
        "us_per_layer_rank_share": rank_us,
        "plan_us": plan_us,
        "plan_three_calls_us": plan_sep_us,
        "permute_rank_us": perm_rank_us,
        "permute_rank_gbs": rank_bytes / (perm_rank_us * 1e-6) / 1e9,
        "stage_ms": stage_ms,
        "stage_gbs": stage_bytes / (stage_ms * 1e-3) / 1e9 if n_used else 0.0,
        "replicas": n_used,
        "solver_steps": int(stats[1]),
        "imbalance_before": float(before.max() / before.mean()),
        "imbalance_after": float(rl.max() / rl.mean()),
        "device_copy_gbs": copy["gbs"],
        "device_fill_gbs": fill["gbs"],
        "permute_over_fill_line": (pb / (perm_ms * 1e-3) / 1e9) / fill["gbs"],
        **seq,
        **comb,
        **floor,
        **grad,
    }
    out["extra"]["stage_frac"] = out["extra"]["stage_gbs"] / HBM_PEAK_GBS
    # the staging kernel alone, graph-replayed back to back (no launch latency)
    out["extra"]["stage_kernel_us"] = stage_kernel_us
    out["extra"]["stage_kernel_gbs"] = stage_bytes / (stage_kernel_us * 1e-6) / 1e9 if n_used else 0.0
    out["extra"]["stage_kernel_frac"] = out["extra"]["stage_kernel_gbs"] / HBM_PEAK_GBS
    out["extra"]["steps_gpu_us_vs_oracle_ms"] = {
        k: {"gpu_us": v, "oracle_ms": cpu["per_step_ms_median"][k] if cpu else None}
        for k, v in gpu_steps.items()}
    return out


def waterfill_inst(w):
    ipr = w.E_loc + 1
    inst = np.full(w.R * ipr, -1, dtype=np.int32)
    for r in range(w.R):
        inst[r * ipr:r * ipr + w.E_loc] = np.arange(r * w.E_loc, (r + 1) * w.E_loc)
        inst[r * ipr + w.E_loc] = w.E + r
    return inst, ipr


def bench_waterfill(args, torch, U, W, w):
    """DeepSeek-V3 layer with Waterfill: routed load matrix (counts only) -> Waterfill ->
    fused (K+1)-column layout -> load matrix -> identity quotas -> reroute/assign ->
    permute."""
    log(f"workload {w.name}: R={w.R} E={w.E} T={w.T} K={w.K} H={w.H}")
    ids = W.routing(w)
    inst, ipr = waterfill_inst(w)
    E2, K2 = w.E + w.R, w.K + 1
    L = Layer(U, W, torch, w, None, E=E2, K=K2, ipr=ipr, weights=False)
    ids_d = torch.from_numpy(ids).to(DEV)
    counts1 = torch.empty(w.R, w.E, dtype=torch.int32, device=DEV)
    ws1 = torch.empty(max(U.load_matrix_workspace_size(w.R, w.T, w.K, w.E), 4), dtype=torch.uint8,
                      device=DEV)
    B = torch.full((w.R,), w.T, dtype=torch.int32, device=DEV)
    sh = torch.empty(w.R, w.T, dtype=torch.int32, device=DEV)
    wl = torch.empty(1, dtype=torch.int32, device=DEV)
    sl = torch.empty(w.R, dtype=torch.int32, device=DEV)
    rl = torch.empty(w.R, dtype=torch.int32, device=DEV)
    L.plan["inst_expert"].copy_(torch.from_numpy(inst))
    seed = W.waterfill_seed(w)

    def wf_plan(s, r_begin=0, r_end=None):
        U.load_matrix(ids_d, w.E, counts1, None, None, ws1, s, counts_only=True)
        U.waterfill(counts1, ids_d, B, seed, 0, 4, sh, wl, sl, rl, L.ids, stream=s)
        L.load(s)
        U.identity_quota(L.counts, L.plan["inst_expert"], L.plan["inst_quota"], stream=s)
        L.reroute(s, r_begin, r_end)

    tp = Timer(torch, args.steps)

    def step(s, timers):
        wf_plan(s)
        if timers:
            timers[0].start(s)
        L.permute(s)
        if timers:
            timers[0].stop(s)

    ms = timed_steps(torch, args, step, torch.cuda.current_stream(), (tp,))
    N = w.N
    pb = permute_bytes(N, L.P, w.H)
    out = base_line(w, W, N / (ms * 1e-3), ms, args, "int32",
                    {"top_k_fused": K2, "shared_slot_per_rank": 1})
    out["roofline"] = roofline(pb, tp.mean_ms(), PERMUTE_CALL,
                               measured_traffic(w.name))
    out["cpu_baseline"] = None
    if args.roofline_only:
        out["extra"] = {"device_copy_gbs": copy_reference(torch, U)["gbs"]}
        return out
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        x_host = L.x.view(torch.int16).cpu().numpy().view(np.uint16)
        out["cpu_baseline"] = cpu_baseline_waterfill(w, ids, x_host, inst, ipr, seed)
        del x_host
    seq = sequential_permute_line(torch, U, L, tp.mean_ms())
    plan_us = graph_us(torch, lambda s: wf_plan(s))
    wf_us = graph_us(torch, lambda s: U.waterfill(counts1, ids_d, B, seed, 0, 4, sh, wl, sl, rl,
                                                  L.ids, stream=s))
    rank_us = graph_us(torch, lambda s, i: (wf_plan(s, i % w.R, i % w.R + 1),
                                            L.permute(s, i % w.R, i % w.R + 1, row_src=False)),
                       reps=w.R, replays=2, indexed=True)
    torch.cuda.synchronize()
    L_r = rl.cpu().numpy().astype(np.float64)
    shared = np.bincount(sh.cpu().numpy().reshape(-1), minlength=w.R)
    local = np.full(w.R, w.T, dtype=np.float64)
    sh_all = torch.empty_like(sh)
    U.waterfill(counts1, ids_d, B, seed, 0, 4, sh_all, wl, sl, rl, None, want_ext=False,
                all_ranks=True)
    shared_all = np.bincount(sh_all.cpu().numpy().reshape(-1), minlength=w.R)
    out["extra"] = {**seq, "us_per_layer_rank_share": rank_us, "plan_us": plan_us,
                    "waterfill_us": wf_us,
                    "waterline": int(wl.item()),
                    "imbalance_routed_only": float(L_r.max() / L_r.mean()),
                    "imbalance_shared_local": float((L_r + local).max() / (L_r + local).mean()),
                    "imbalance_shared_waterfill": float((L_r + shared).max() / (L_r + shared).mean()),
                    "imbalance_shared_waterfill_all_ranks":
                        float((L_r + shared_all).max() / (L_r + shared_all).mean())}
    return out


def bench_lplb(args, torch, U, W, w):
    """LPLB layer: load matrix -> LP split -> reroute/assign on its quotas -> permute."""
    log(f"workload {w.name}: R={w.R} E={w.E} T={w.T} K={w.K} H={w.H} replicas={w.n_static_replicas}")
    ids = W.routing(w)
    inst = W.static_replica_placement(w)
    ipr = w.E_loc + 1
    L = Layer(U, W, torch, w, ids, ipr=ipr, weights=False)
    L.plan["inst_expert"].copy_(torch.from_numpy(inst))
    lp = U.lplb_prepare(inst, w.R, w.E, ipr, DEV)
    n_copies = int(sum((inst == e).sum() for e in range(w.E) if (inst == e).sum() >= 2))
    x = torch.empty(max(n_copies, 1), dtype=torch.float32, device=DEV)
    m = torch.empty(1, dtype=torch.float32, device=DEV)
    st = torch.zeros(4, dtype=torch.int32, device=DEV)

    lp_ws = torch.empty(max(U.lplb_plan_workspace_size(w.R, w.T, w.K, w.E, ipr), 4),
                        dtype=torch.uint8, device=DEV)
    lp_out = {"counts": L.counts, "bucket_pos": L.bp, "x": x, "m": m,
              "inst_quota": L.plan["inst_quota"], "stats": st, "xfer": L.xfer,
              "inst_offset": L.ioff, "dest_inst": L.dinst, "dest_row": L.drow}

    def lp_plan(s, r_begin=0, r_end=None):
        """The layer's plan in one uep_lplb_plan call (the LP overlapped with the ranking)."""
        U.lplb_plan(L.ids, lp, L.plan["inst_expert"], args.lp_iters, r_begin, r_end, lp_out,
                    None, lp_ws, s)

    def lp_plan_separate(s, r_begin=0, r_end=None):
        """The same plan as three calls: load matrix, LP split, reroute/assignment."""
        L.load(s)
        U.lplb(L.counts, lp, n_copies, len(inst), args.lp_iters, x, m, L.plan["inst_quota"], st,
               None, s)
        L.reroute(s, r_begin, r_end)

    tp = Timer(torch, args.steps)

    def step(s, timers):
        lp_plan(s)
        if timers:
            timers[0].start(s)
        L.permute(s)
        if timers:
            timers[0].stop(s)

    ms = timed_steps(torch, args, step, torch.cuda.current_stream(), (tp,))
    pb = permute_bytes(w.N, w.P, w.H)
    out = base_line(w, W, w.N / (ms * 1e-3), ms, args, "int32",
                    {"static_replicas": w.n_static_replicas, "lp_iters": args.lp_iters})
    out["roofline"] = roofline(pb, tp.mean_ms(), PERMUTE_CALL,
                               measured_traffic(w.name))
    out["cpu_baseline"] = None
    if args.roofline_only:
        out["extra"] = {"device_copy_gbs": copy_reference(torch, U)["gbs"]}
        return out
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        x_host = L.x.view(torch.int16).cpu().numpy().view(np.uint16)
        out["cpu_baseline"] = cpu_baseline_lplb(w, ids, x_host, inst, ipr)
        del x_host
    seq = sequential_permute_line(torch, U, L, tp.mean_ms(), reps=3)
    lp_us = graph_us(torch, lambda s: U.lplb(L.counts, lp, n_copies, len(inst), args.lp_iters, x,
                                             m, L.plan["inst_quota"], st, None, s), reps=5)
    plan_us = graph_us(torch, lambda s: lp_plan(s), reps=5)
    plan_sep_us = graph_us(torch, lambda s: lp_plan_separate(s), reps=5)
    rank_us = graph_us(torch, lambda s, i: (lp_plan(s, i % w.R, i % w.R + 1),
                                            L.permute(s, i % w.R, i % w.R + 1, row_src=False)),
                       reps=8, replays=2, indexed=True)
    # the per-token draw variant: LP split -> copy draw -> instance dispatch layout
    I = len(inst)
    di = torch.empty_like(L.ids)
    ident = torch.arange(I, dtype=torch.int32, device=DEV)
    ci = torch.empty(w.R, I, dtype=torch.int32, device=DEV)
    bpi = torch.empty_like(L.ids)
    wsi = torch.empty(max(U.load_matrix_workspace_size(w.R, w.T, w.K, I), 4), dtype=torch.uint8,
                      device=DEV)
    qi = torch.empty(I, dtype=torch.int32, device=DEV)
    xfi = torch.empty(w.R, I, dtype=torch.int32, device=DEV)
    ioi = torch.empty(I + 1, dtype=torch.int32, device=DEV)
    dii, dri = torch.empty_like(L.ids), torch.empty_like(L.ids)
    rri = torch.empty(max(U.reroute_workspace_size(w.R, I, ipr), 4), dtype=torch.uint8, device=DEV)

    def sample_plan(s):
        # the LP needs the loads only: the draws are ranked afterwards, as instance ids
        U.load_matrix(L.ids, L.E, L.counts, None, None, L.lm_ws, s, counts_only=True)
        U.lplb(L.counts, lp, n_copies, I, args.lp_iters, x, m, L.plan["inst_quota"], st, None, s)
        U.lplb_sample(L.ids, lp, x, 99, 0, di, None, s)
        U.load_matrix(di, I, ci, bpi, None, wsi, s)
        U.identity_quota(ci, ident, qi, stream=s)
        U.reroute_assign(ci, di, bpi, ipr, ident, qi, 0, None, xfi, ioi, dii, dri, None, rri, s)

    sample_us = graph_us(torch, sample_plan, reps=5)
    torch.cuda.synchronize()
    qs = qi.cpu().numpy()
    load_sampled = np.array([qs[r * ipr:(r + 1) * ipr].sum() for r in range(w.R)])
    torch.cuda.synchronize()
    c = L.counts.cpu().numpy().sum(0)
    # uniform split of every replicated expert (the static default the LP replaces)
    uni = np.zeros(w.R)
    for e in range(w.E):
        where = np.nonzero(inst == e)[0]
        for i in where:
            uni[i // ipr] += c[e] / len(where)
    out["extra"] = {**seq, "us_per_layer_rank_share": rank_us, "plan_us": plan_us,
                    "plan_three_calls_us": plan_sep_us, "lplb_us": lp_us,
                    "load_matrix_us": graph_us(torch, L.load, reps=5),
                    "lp_iterations_run": int(st[2].item()), "m": float(m.item()),
                    "max_load_uniform_split": float(uni.max()), "mean_load": float(c.sum() / w.R),
                    "sample_plan_us": sample_us, "max_load_sampled": int(load_sampled.max())}
    return out


def bench_sweep(args, torch, U, W, w):
    """94 Qwen3-235B-shaped layers: forward (plan, staging into the one shared slot set,
    whole-group permute) in layer order, then backward in reverse order replaying the
    cached plans (weights staged again, replica gradients reduced into the mains)."""
    from concurrent.futures import ProcessPoolExecutor
    log(f"workload {w.name}: {w.layers} layers, R={w.R} E={w.E} T={w.T} K={w.K} H={w.H}")
    with ProcessPoolExecutor(max_workers=8) as ex:
        routings = list(ex.map(W.routing, [w] * w.layers, range(w.layers)))
    layer0 = W.scaled(w, layers=1)
    L = Layer(U, W, torch, layer0, routings[0])
    pool = 4        # distinct main weight / gradient sets, cycled over the layers
    gen = torch.Generator(device=DEV).manual_seed(W.tensor_seed(w, 0, 2))
    mains = [L.main_w] + [(torch.randn(w.E, w.expert_elems, generator=gen, device=DEV,
                                       dtype=torch.bfloat16) * 0.02) for _ in range(pool - 1)]
    mgrads = [torch.zeros(w.E, w.expert_elems, dtype=torch.float32, device=DEV) for _ in range(pool)]
    slot_grad = torch.zeros(w.R, w.S, w.expert_elems, dtype=torch.float32, device=DEV)
    ids_d = [torch.from_numpy(r).to(DEV) for r in routings]
    slots = [torch.empty(w.R, w.S, dtype=torch.int32, device=DEV) for _ in range(w.layers)]
    s = torch.cuda.current_stream()
    fwd_t = Timer(torch, w.layers * (args.steps + args.warmup))
    bwd_t = Timer(torch, w.layers * (args.steps + args.warmup))
    perm_t = Timer(torch, w.layers * (args.steps + args.warmup))

    def sweep(st, timers):
        for l in range(w.layers):
            L.ids = ids_d[l]
            L.main_w = mains[l % pool]
            fwd_t.start(st)
            L.plan_step(st)
            L.stage(st)
            perm_t.start(st)
            L.permute(st)
            perm_t.stop(st)
            fwd_t.stop(st)
            slots[l].copy_(L.plan["slot_expert"][:, :w.S])
        for l in reversed(range(w.layers)):
            bwd_t.start(st)
            U.stage_replica_weights(U.STAGE_WEIGHTS, w.R, w.E, w.S, slots[l], w.expert_elems,
                                    main_w=mains[l % pool], slot_w=L.slot_w, stream=st)
            U.stage_replica_weights(U.STAGE_GRAD_REDUCE, w.R, w.E, w.S, slots[l], w.expert_elems,
                                    main_grad=mgrads[l % pool], slot_grad=slot_grad, stream=st)
            bwd_t.stop(st)

    ms = timed_steps(torch, args, sweep, s)
    f = np.array(fwd_t.all_ms()[w.layers * args.warmup:]) * 1e3
    b = np.array(bwd_t.all_ms()[w.layers * args.warmup:]) * 1e3
    out = base_line(w, W, w.N / (ms * 1e-3), ms, args, "int32",
                    {"layers": w.layers, "weight_sets_cycled": pool, "zipf_s": "0.8+0.6U per layer"})
    # the dominant kernel: every layer's whole-group permute call, timed on the launch
    # stream inside the sweep (no counter passes were taken on this command)
    perm_ms = float(np.mean(perm_t.all_ms()[w.layers * args.warmup:]))
    out["roofline"] = roofline(permute_bytes(w.N, w.P, w.H), perm_ms, PERMUTE_CALL)
    out["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"], _ = cpu_baseline_sweep(w, routings)
    out["extra"] = {"fwd_us_sum": float(f.sum() / args.steps), "fwd_us_p50": float(np.percentile(f, 50)),
                    "fwd_us_p99": float(np.percentile(f, 99)),
                    "bwd_us_sum": float(b.sum() / args.steps), "bwd_us_p50": float(np.percentile(b, 50)),
                    "bwd_us_p99": float(np.percentile(b, 99)),
                    "note": "per-layer times include the whole-group permute of 32 virtual ranks"}
    return out


def kernel_report(args, torch, U, W):
    """Graph-replayed GPU time of every kernel of the path, per workload."""
    rep = {}
    for w in (W.TINY, W.QWEN_LAYER):
        ids = W.routing(w)
        L = Layer(U, W, torch, w, ids)
        L.plan_step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        n_used = int(L.plan["stats"][0].item())
        d = {"load_matrix": graph_us(torch, L.load), "solve_quota": graph_us(torch, L.solve),
             "reroute_assign": graph_us(torch, L.reroute),
             "permute_whole": graph_us(torch, lambda s: L.permute(s), reps=5),
             "permute_rank": graph_us(torch, lambda s, i: L.permute(s, i % w.R, i % w.R + 1,
                                                                     row_src=False),
                                      reps=w.R, indexed=True),
             "stage_whole": graph_us(torch, lambda s: L.stage(s), reps=5),
             "stage_rank": graph_us(torch, lambda s, i: L.stage(s, i % w.R, i % w.R + 1),
                                    reps=w.R, indexed=True), "replicas": n_used}
        pb = permute_bytes(w.N, w.P, w.H)
        d["permute_whole_gbs"] = pb / (d["permute_whole"] * 1e-6) / 1e9
        se_h = L.plan["slot_expert"].cpu().numpy()
        n_distinct = len(np.unique(se_h[se_h >= 0]))
        d["stage_whole_gbs"] = ((n_distinct + n_used) * w.expert_elems * 2
                                / (d["stage_whole"] * 1e-6) / 1e9)
        rep[w.name] = d
        del L
        torch.cuda.empty_cache()
    # uep_device_copy and uep_device_fill of 4 GiB (the copy and write-only lines)
    a = torch.empty(1 << 31, dtype=torch.int16, device=DEV)
    b = torch.empty_like(a)
    cu = graph_us(torch, lambda s: U.device_copy(a, b, s), reps=5)
    rep["device_copy_4GiB"] = {"us": cu, "gbs": 2 * a.numel() * 2 / (cu * 1e-6) / 1e9}
    fu = graph_us(torch, lambda s: U.device_fill(b, 0, s), reps=5)
    rep["device_fill_4GiB"] = {"us": fu, "gbs": b.numel() * 2 / (fu * 1e-6) / 1e9}
    del a, b
    torch.cuda.empty_cache()
    print(json.dumps(rep), flush=True)


# ----------------------------------------------------------------------------- profiles
def _short(name):
    name = name.replace("void ", "")
    head = name.split("(")[0]
    return head if len(head) <= 60 else head[:57] + "..."


def _csv(directory, suffix):
    import csv
    import glob
    found = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not found:
        raise SystemExit(f"no *{suffix} under {directory}")
    with open(found[0]) as f:
        return list(csv.DictReader(f))


def _permute_calls(rows, name_key, order_key, whole_rs_blocks, blocks_of):
    """Group the launches of whole-group uep_permute calls: each call is a run of
    consecutive prefetch_kernel / permute_kernel launches closed by a row_src_kernel
    launch over every pair (whole_rs_blocks workgroups).  Returns a list of lists of
    rows, one list per call, in launch order."""
    calls, run = [], []
    for r in sorted(rows, key=lambda r: int(r[order_key])):
        name = r[name_key]
        if "prefetch_kernel" in name or "uep::permute_kernel" in name:
            run.append(r)
        elif "row_src_kernel" in name and blocks_of(r) == whole_rs_blocks and run:
            calls.append(run + [r])
            run = []
        else:
            run = []
    return calls


# the default bench's warm-up and timed steps (main()'s defaults)
_DEFAULT_WARMUP, _DEFAULT_STEPS = 3, 20
# (workload, pairs) of the whole-group permute calls the summaries look for
_TRACE_WORKLOADS = (("qwen3_235b_layer", 32 * 8192 * 8), ("dsv3_waterfill", 64 * 4096 * 9),
                    ("lplb_layer", 64 * 16384 * 8), ("tiny", 4 * 512 * 2))


def trace_summary(directory):
    """Markdown table of a rocprofv3 --kernel-trace --stats CSV run: rocprofv3's own
    per-name statistics, then the trace split by (kernel, workgroup count), since one
    kernel runs at several sizes in one bench (whole group vs one rank's share)."""
    stats = _csv(directory, "kernel_stats.csv")
    print("rocprofv3 kernel statistics (by kernel name, all launches):\n")
    print("| kernel | calls | avg us | min us | max us | % time |")
    print("|---|---|---|---|---|---|")
    for r in stats:
        if not r["Name"].startswith(("uep::", "void uep::")):
            continue
        print(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
              f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {r['Percentage']} |")
    trace = _csv(directory, "kernel_trace.csv")
    agg = {}
    for r in trace:
        if "uep::" not in r["Kernel_Name"]:
            continue
        wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
        blocks = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]) // max(wg, 1)
        key = (_short(r["Kernel_Name"]), blocks, wg)
        agg.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    print("\nkernel trace by (kernel, workgroups):\n")
    print("| kernel | workgroups x threads | launches | avg us | median us | min us | max us |")
    print("|---|---|---|---|---|---|---|")
    for (k, b, wg), d in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        d = np.array(d, dtype=np.float64) / 1e3
        print(f"| {k} | {b} x {wg} | {len(d)} | {d.mean():.2f} | {np.median(d):.2f} | "
              f"{d.min():.2f} | {d.max():.2f} |")

    def blocks_of(r):
        wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
        return int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]) // max(wg, 1)

    uep_rows = [r for r in trace if "uep::" in r["Kernel_Name"]]
    for workload, P in _TRACE_WORKLOADS:
        calls = _permute_calls(uep_rows, "Kernel_Name", "Start_Timestamp", (P + 255) // 256,
                               blocks_of)
        if not calls:
            continue
        busy = np.array([sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in c)
                         for c in calls], dtype=np.float64) / 1e3
        span = np.array([int(c[-1]["End_Timestamp"]) - int(c[0]["Start_Timestamp"]) for c in calls],
                        dtype=np.float64) / 1e3
        print(f"\nwhole-group uep_permute calls ({workload}, {P} pairs): {len(calls)} calls of "
              f"{len(calls[0])} launches; kernel time per call avg {busy.mean():.2f} us "
              f"(median {np.median(busy):.2f}); first start to last end avg {span.mean():.2f} us "
              f"(median {np.median(span):.2f})")
        w0, n = _DEFAULT_WARMUP, _DEFAULT_STEPS
        if len(calls) >= w0 + n:
            b, sp = busy[w0:w0 + n], span[w0:w0 + n]
            print(f"- calls {w0 + 1}-{w0 + n} (the default bench's {n} timed steps, after {w0} "
                  f"warm-up steps): kernel time per call avg {b.mean():.2f} us, first start to "
                  f"last end avg {sp.mean():.2f} us")
        if len(calls) > w0 + n:
            b = busy[w0 + n:]
            print(f"- calls {w0 + n + 1}-{len(calls)} (later calls of the same run, e.g. the "
                  f"sequential-row reference line): kernel time per call avg {b.mean():.2f} us")


def pmc_summary(fetch_dir, write_dir, workload="qwen3_235b_layer"):
    """Copy-calibrated HBM traffic of the permute call from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).  Each counter is scaled by
    true bytes / counter reading of uep_device_copy's 1 GiB copy in the same run."""
    w = None
    from moe_expert_load_amd import workload as W
    w = W.ALL[workload]

    def per_kernel(rows, counter):
        out = {}
        for r in rows:
            if r["Counter_Name"] != counter or "uep::" not in r["Kernel_Name"]:
                continue
            key = (_short(r["Kernel_Name"]), int(r["Grid_Size"]) // max(int(r["Workgroup_Size"]), 1))
            out.setdefault(key, []).append(float(r["Counter_Value"]))
        return {k: float(np.median(v)) for k, v in out.items()}

    fetch = per_kernel(_csv(fetch_dir, "counter_collection.csv"), "FETCH_SIZE")
    write = per_kernel(_csv(write_dir, "counter_collection.csv"), "WRITE_SIZE")
    copy_kib = (1 << 30) / 1024
    ck = [k for k in fetch if k[0].endswith("device_copy_kernel")]
    f_fetch = copy_kib / fetch[ck[0]]
    f_write = copy_kib / write[ck[0]]
    print("| kernel | workgroups | FETCH_SIZE KiB | WRITE_SIZE KiB | calibrated MiB read | "
          "calibrated MiB written |")
    print("|---|---|---|---|---|---|")
    for k in sorted(fetch, key=lambda k: -fetch[k] - write.get(k, 0)):
        fw = write.get(k, float("nan"))
        print(f"| {k[0]} | {k[1]} | {fetch[k]:.1f} | {fw:.1f} | {fetch[k] * f_fetch / 1024:.1f} | "
              f"{fw * f_write / 1024:.1f} |")
    P = w.N * (w.K + 1) if w.shared_expert else w.P

    def per_call(rows, counter):
        rows = [r for r in rows if r["Counter_Name"] == counter and "uep::" in r["Kernel_Name"]]
        order = "Dispatch_Id" if rows and "Dispatch_Id" in rows[0] else "Correlation_Id"
        calls = _permute_calls(rows, "Kernel_Name", order, (P + 255) // 256,
                               lambda r: int(r["Grid_Size"]) // max(int(r["Workgroup_Size"]), 1))
        sums = [sum(float(r["Counter_Value"]) for r in c) for c in calls]
        return float(np.median(sums)), len(calls), len(calls[0]) if calls else 0

    f_kib, nf, lf = per_call(_csv(fetch_dir, "counter_collection.csv"), "FETCH_SIZE")
    w_kib, nw, lw = per_call(_csv(write_dir, "counter_collection.csv"), "WRITE_SIZE")
    kib = f_kib * f_fetch + w_kib * f_write
    traffic = int(round(kib * 1024))
    H = w.H
    N = w.N
    alg = N * H * 2 + P * H * 2 + P * 4
    print(f"\ncalibration (uep_device_copy, 1 GiB read + 1 GiB written): FETCH_SIZE x {f_fetch:.5f}, "
          f"WRITE_SIZE x {f_write:.5f}\n")
    print(f"whole-group uep_permute calls: {nf} in the FETCH_SIZE run, {nw} in the WRITE_SIZE run, "
          f"{lf} launches each (prefetch and permute per chunk, then row_src); per call "
          f"(median): FETCH_SIZE {f_kib:.1f} KiB -> {f_kib * f_fetch / 1024:.1f} MiB read, "
          f"WRITE_SIZE {w_kib:.1f} KiB -> {w_kib * f_write / 1024:.1f} MiB written\n")
    print(f"- workload = {workload}")
    print(f"- kernels = {PERMUTE_CALL}")
    print(f"- algorithmic_bytes_per_launch = {alg}")
    print(f"- traffic_bytes_per_launch = {traffic}")
    print(f"- traffic_over_algorithmic = {traffic / alg:.4f}")
    print(f"- source_sha256 = {source_digest()}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="qwen3_235b_layer")
    ap.add_argument("--lp-iters", type=int, default=30)
    ap.add_argument("--kernels", action="store_true")
    ap.add_argument("--roofline-only", action="store_true",
                    help="timed steps, roofline and the 1 GiB copy reference only (for counter passes)")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="print the markdown summary of a rocprofv3 kernel-trace CSV run")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the copy-calibrated traffic of two rocprofv3 --pmc CSV runs")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, workload=args.workload)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the EP group is simulated as virtual ranks on a "
              "single device, so --gpus above 1 is not supported.", file=sys.stderr)
        sys.exit(2)
    import torch
    from moe_expert_load_amd import uep as U
    from moe_expert_load_amd import workload as W

    if args.kernels:
        kernel_report(args, torch, U, W)
        return
    w = W.ALL[args.workload]
    if w.name in ("qwen3_235b_layer", "tiny"):
        out = bench_layer(args, torch, U, W, w, with_cpu=not args.no_cpu_baseline)
    elif w.name == "dsv3_waterfill":
        out = bench_waterfill(args, torch, U, W, w)
    elif w.name == "lplb_layer":
        out = bench_lplb(args, torch, U, W, w)
    else:
        out = bench_sweep(args, torch, U, W, w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
