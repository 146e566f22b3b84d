"""Oracle: LPLB, the min-max split of replicated experts' load over their copies.

Waterfill/LPLB blog:
* section "速读" (summary) and "线性规划（LP）公式化构建": per layer and batch, minimise
  the largest rank load M; for every rank, its redundant-copy allocation plus the fixed
  load of its single-copy experts plus a slack equals M; for every replicated logical
  expert, the split over its copies sums to its true token count;
* section "决策变量与矩阵规模优化": the variables are the per-copy loads of replicated
  experts, one slack per rank and M; single-copy experts are constants, so the LP grows
  with the replicas and ranks, not with all experts; only the right-hand side changes
  per batch;
* section "从全局计数到LP求解的工程实现": per-expert counts are summed over the EP group
  and every rank solves the same LP (here: column sums of the load matrix);
* section "从LP解决方案到Token调度": the split is normalised into per-copy shares of each
  replicated expert, which then decide how its tokens go to its copies;
* with no redundant copies (red0) there is nothing to split (summary section).

Readings:
* the copies of a replicated expert include its main (per-copy load of each copy);
* integer quotas by largest remainder (Hamilton): w_p = rint(max(x_p, 0) * 256) as an
  integer, q_p = floor(c_e * w_p / W), the leftover units to the largest remainders
  (c_e * w_p mod W), lowest copy first on ties; W = 0 splits c_e evenly, the
  remainder to the lowest copies.  These quotas feed the local-first reroute.

Solver: a dense two-phase primal simplex in fp64 with Bland's rule (no cycling).
Pins: scipy's HiGHS, the max-flow/min-cut closed form
M* = max over rank sets T of (sum_{r in T} F_r + sum_{e: all copies in T} c_e) / |T|
on small R, red0 -> M* = max_r F_r, one expert split over two empty ranks -> c/2.

lplb_sample is the per-token variant of the same section "从LP解决方案到Token调度"
(each token draws a copy from the normalised split; see its docstring for the
readings).  Pins: Philox against numpy (full counters), the draw frequencies within
4 sigma of w_p / W, W = 0 -> uniform over copies, a zero-weight copy never drawn,
single-copy experts and empty slots mapped deterministically.
"""

import numpy as np

from .philox import philox4x64_10_np


def lplb_structure(inst_expert, inst_per_rank: int, E: int) -> dict:
    """Offline structure of the LP: copies of every expert and the replicated ones."""
    inst_expert = np.asarray(inst_expert, dtype=np.int64)
    copies = {e: [] for e in range(E)}
    for i, e in enumerate(inst_expert):
        if e >= 0:
            copies[int(e)].append(i)
    for e, lst in copies.items():
        ranks = [i // inst_per_rank for i in lst]
        if len(set(ranks)) != len(ranks):
            raise ValueError("two copies of one expert on one rank")
    replicated = [e for e in range(E) if len(copies[e]) >= 2]
    copy_inst, copy_rank, copy_group = [], [], []
    for g, e in enumerate(replicated):
        for i in copies[e]:
            copy_inst.append(i)
            copy_rank.append(i // inst_per_rank)
            copy_group.append(g)
    return {
        "copies": copies,
        "replicated": replicated,
        "copy_inst": np.array(copy_inst, dtype=np.int64),
        "copy_rank": np.array(copy_rank, dtype=np.int64),
        "copy_group": np.array(copy_group, dtype=np.int64),
        "inst_per_rank": inst_per_rank,
    }


def lplb_lp(counts, st: dict):
    """(A, b, cost, c_e, F): rows = R rank rows then one row per replicated expert;
    columns = copies x_p, then slacks s_r, then M."""
    counts = np.asarray(counts, dtype=np.int64)
    R, E = counts.shape
    c = counts.sum(axis=0)
    F = np.zeros(R, dtype=np.float64)
    for e in range(E):
        lst = st["copies"][e]
        if len(lst) == 0 and c[e] > 0:
            raise ValueError(f"expert {e} has load but no instance")
        if len(lst) == 1:
            F[lst[0] // st["inst_per_rank"]] += c[e]
    n = len(st["copy_inst"])
    G = len(st["replicated"])
    A = np.zeros((R + G, n + R + 1))
    b = np.zeros(R + G)
    for p in range(n):
        A[st["copy_rank"][p], p] = -1.0           # rank row: M - sum x_p - s_r = F_r
        A[R + st["copy_group"][p], p] = 1.0       # expert row: sum x_p = c_e
    for r in range(R):
        A[r, n + r] = -1.0
        A[r, n + R] = 1.0
        b[r] = F[r]
    for g, e in enumerate(st["replicated"]):
        b[R + g] = c[e]
    cost = np.zeros(n + R + 1)
    cost[n + R] = 1.0
    return A, b, cost, c, F


def simplex(A, b, cost, tol: float = 1e-9, max_pivots: int = 100000):
    """min cost.v s.t. A v = b, v >= 0 by a two-phase tableau simplex with Bland's rule."""
    A = np.array(A, dtype=np.float64)
    b = np.array(b, dtype=np.float64)
    m, n = A.shape
    neg = b < 0
    A[neg] *= -1.0
    b[neg] *= -1.0
    # phase 1 tableau: [A | I | b]
    T = np.hstack([A, np.eye(m), b[:, None]])
    basis = list(range(n, n + m))

    def run(cost_full, allowed):
        nonlocal T
        pivots = 0
        while True:
            cb = cost_full[basis]
            rc = cost_full - cb @ T[:, :-1]
            enter = -1
            for j in allowed:
                if rc[j] < -tol:
                    enter = j
                    break
            if enter < 0:
                return
            col = T[:, enter]
            best, leave = None, -1
            for i in range(m):
                if col[i] > tol:
                    ratio = T[i, -1] / col[i]
                    if best is None or ratio < best - tol or (abs(ratio - best) <= tol and basis[i] < basis[leave]):
                        best, leave = ratio, i
            if leave < 0:
                raise ValueError("LP unbounded")
            T[leave] /= T[leave, enter]
            for i in range(m):
                if i != leave and T[i, enter] != 0.0:
                    T[i] -= T[i, enter] * T[leave]
            basis[leave] = enter
            pivots += 1
            if pivots > max_pivots:
                raise RuntimeError("simplex pivot limit")

    cost1 = np.concatenate([np.zeros(n), np.ones(m)])
    run(cost1, range(n + m))
    if T[:, -1] @ cost1[basis] > tol * max(1.0, float(b.sum())):
        raise ValueError("LP infeasible")
    # drive zero-level artificials out of the basis
    for i in range(m):
        if basis[i] >= n:
            for j in range(n):
                if abs(T[i, j]) > tol:
                    T[i] /= T[i, j]
                    for k in range(m):
                        if k != i and T[k, j] != 0.0:
                            T[k] -= T[k, j] * T[i]
                    basis[i] = j
                    break
    keep_rows = [i for i in range(m) if basis[i] < n]          # redundant rows drop out
    T = np.hstack([T[keep_rows, :n], T[keep_rows, -1:]])
    basis = [basis[i] for i in keep_rows]
    m = len(keep_rows)
    run(np.asarray(cost, dtype=np.float64), range(n))
    v = np.zeros(n)
    for i, j in enumerate(basis):
        v[j] = T[i, -1]
    return v, float(np.asarray(cost) @ v)


def hamilton_quotas(x, c_groups, groups):
    """Integer quotas per copy by largest remainder on rint(max(x,0) * 256).

    x: per-copy split (any float type; the scaling by 256 is exact);
    c_groups[g]: true count of replicated expert g; groups[g]: its copy indices (ascending).
    """
    x = np.asarray(x)
    q = np.zeros(x.size, dtype=np.int64)
    for g, idx in enumerate(groups):
        c = int(c_groups[g])
        w = [int(np.rint(np.float64(max(x[p], 0)) * 256.0)) for p in idx]
        W = sum(w)
        if W == 0:
            n = len(idx)
            for k, p in enumerate(idx):
                q[p] = c // n + (1 if k < c % n else 0)
            continue
        base = [(c * wp) // W for wp in w]
        rem = [(c * wp) % W for wp in w]
        left = c - sum(base)
        order = sorted(range(len(idx)), key=lambda k: (-rem[k], k))
        for k in order[:left]:
            base[k] += 1
        for k, p in enumerate(idx):
            q[p] = base[k]
    return q


def lplb(counts, inst_expert, inst_per_rank: int):
    """Full LPLB step on the CPU: M*, the split x* and the integer quotas per instance."""
    counts = np.asarray(counts, dtype=np.int64)
    R, E = counts.shape
    st = lplb_structure(inst_expert, inst_per_rank, E)
    A, b, cost, c, F = lplb_lp(counts, st)
    n = len(st["copy_inst"])
    if n == 0:
        m_star = float(F.max()) if R else 0.0
        x = np.zeros(0)
    else:
        sigma = max(1.0, float(np.abs(b).max()))      # work on O(1) numbers
        v, m_star = simplex(A, b / sigma, cost)
        v *= sigma
        m_star *= sigma
        x = v[:n]
    groups = [list(np.nonzero(st["copy_group"] == g)[0]) for g in range(len(st["replicated"]))]
    c_groups = [int(c[e]) for e in st["replicated"]]
    qc = hamilton_quotas(x, c_groups, groups)
    inst_expert = np.asarray(inst_expert, dtype=np.int64)
    inst_quota = np.zeros(inst_expert.size, dtype=np.int64)
    for e in range(E):
        if len(st["copies"][e]) == 1:
            inst_quota[st["copies"][e][0]] = c[e]
    for p, i in enumerate(st["copy_inst"]):
        inst_quota[i] = qc[p]
    return {"m_star": m_star, "x": x, "inst_quota": inst_quota, "F": F, "c": c,
            "structure": st, "groups": groups}


def lplb_sample(topk_ids, inst_expert, inst_per_rank: int, E: int, x, seed: int, layer: int,
                ranks=None):
    """LPLB's dispatch-time copy draw (blog section "从LP解决方案到Token调度"): the LP
    split, normalised per replicated expert, is a probability distribution over its
    physical copies; every token routed to a replicated expert draws one copy from it,
    and a single-copy expert maps to its only instance.

    Readings: the distribution is taken on the integer weights w_p = rint(max(x_p, 0) *
    256) of the quota step (exact on both sides); the draw for slot k of global token
    g is word k mod 4 u of Philox4x64-10 at counter (g, floor(k / 4), 1, 0), key
    (seed, layer), so one block of the generator serves four slots of a token;
    v = floor(u * W / 2^64) with W = sum w_p, and the first copy (instance order) whose
    running weight exceeds v wins; with W = 0 the copy floor(u * n / 2^64) of the n
    copies.  x is indexed like lplb_structure's copies (replicated experts ascending,
    each expert's copies in instance order).

    Returns dest_inst [R][T][K] int64 (-1 for empty slots; ranks outside ``ranks``,
    if given, stay -1)."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    R, T, K = ids.shape
    st = lplb_structure(inst_expert, inst_per_rank, E)
    x = np.asarray(x)
    copies_of = {}
    for g_, e in enumerate(st["replicated"]):
        idx = np.nonzero(st["copy_group"] == g_)[0]
        w = [int(np.rint(np.float64(max(x[p], 0)) * 256.0)) for p in idx]
        copies_of[e] = ([int(st["copy_inst"][p]) for p in idx], w)
    out = np.full((R, T, K), -1, dtype=np.int64)
    for r in (range(R) if ranks is None else ranks):
        g = np.arange(r * T, (r + 1) * T, dtype=np.uint64)
        blocks = [philox4x64_10_np(g, (seed, layer), c1=b, c2=1) for b in range((K + 3) // 4)]
        u = [blocks[k // 4][:, k % 4] for k in range(K)]
        for t in range(T):
            for k in range(K):
                e = int(ids[r, t, k])
                if e < 0:
                    continue
                if e >= E:
                    raise ValueError("expert id out of range")
                lst = st["copies"][e]
                if len(lst) == 0:
                    raise ValueError("an expert with load has no instance")
                if len(lst) == 1:
                    out[r, t, k] = lst[0]
                    continue
                inst, w = copies_of[e]
                W = sum(w)
                uu = int(u[k][t])
                if W == 0:
                    out[r, t, k] = inst[(uu * len(inst)) >> 64]
                    continue
                v = (uu * W) >> 64
                run = 0
                for i, wi in zip(inst, w):
                    run += wi
                    if run > v:
                        out[r, t, k] = i
                        break
    return out
