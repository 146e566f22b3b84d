"""GPU parity of LPLB (Waterfill/LPLB blog, sections "线性规划（LP）公式化构建" and
"从LP解决方案到Token调度") against the fp64 simplex oracle.

The split x is not unique, so what is compared is: the objective m within 1e-3 of the
oracle's M* (and never below it), the split's validity (non-negative, each group
summing to its count), and the integer quotas, which must be exactly the largest
remainder rounding of the split the kernel returned.  The reroute/assignment driven by
the quotas is then checked bit-exact against the oracle on the oracle's own quotas, and
by its properties on the kernel's quotas.
"""

import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle as O                                       # noqa: E402
from moe_expert_load_amd import uep as U                 # noqa: E402
from moe_expert_load_amd import workload as W            # noqa: E402
from tests.gpu_helpers import (DEV, to_dev, host, err_word, say,  # noqa: E402
                               compare_dispatch_rows, random_routing)
from tests.test_oracle_reroute_permute import (check_reroute_properties,  # noqa: E402
                                               check_assign_properties)

pytestmark = pytest.mark.gpu

REL_TOL = 1e-3


def copy_groups(inst_expert, E):
    """Copies (instance ids) of every replicated expert, ascending expert then instance."""
    groups = []
    for e in range(E):
        insts = [i for i, v in enumerate(inst_expert) if v == e]
        if len(insts) >= 2:
            groups.append((e, insts))
    return groups


def check_largest_remainder(x, c, q):
    """q is the largest-remainder rounding of c over weights rint(max(x, 0) * 256)."""
    w = [int(np.rint(np.float64(max(float(v), 0.0)) * 256.0)) for v in x]
    W_ = sum(w)
    assert sum(q) == c
    if W_ == 0:
        n = len(q)
        assert q == [c // n + (1 if k < c % n else 0) for k in range(n)]
        return
    base = [(c * wi) // W_ for wi in w]
    rem = [(c * wi) % W_ for wi in w]
    plus = [qi - bi for qi, bi in zip(q, base)]
    assert all(p in (0, 1) for p in plus)
    # every +1 goes to a remainder at least as large as any copy without one
    got = [k for k in range(len(q)) if plus[k]]
    miss = [k for k in range(len(q)) if not plus[k]]
    for a in got:
        for b in miss:
            assert (rem[a], -a) > (rem[b], -b)


def run_lplb(counts_np, inst, ipr, iters=30):
    R, E = counts_np.shape
    lp = U.lplb_prepare(inst, R, E, ipr, DEV)
    groups = copy_groups(inst, E)
    n = sum(len(g[1]) for g in groups)
    err = err_word()
    x, m, q, st = U.lplb(to_dev(counts_np), lp, n, len(inst), iters=iters, err=err)
    return host(x), float(host(m)[0]), host(q), host(st), int(host(err)[0]), groups


def check_lplb(counts_np, inst, ipr, iters=30):
    R, E = counts_np.shape
    res = O.lplb(counts_np, inst, ipr)
    x, m, q, st, err, groups = run_lplb(counts_np, inst, ipr, iters)
    assert err == 0
    m_star = res["m_star"]
    assert m >= m_star * (1 - 1e-6) - 1e-3
    assert m <= m_star * (1 + REL_TOL) + 1e-3, (m, m_star)
    c = counts_np.sum(0)
    k = 0
    for e, insts in groups:
        xs = x[k:k + len(insts)]
        assert (xs >= 0).all()
        assert abs(float(xs.sum()) - c[e]) <= 1e-5 * max(1.0, c[e]) + 1e-3
        check_largest_remainder(xs, int(c[e]), [int(q[i]) for i in insts])
        k += len(insts)
    for e in range(E):                       # every expert's quotas sum to its load
        assert q[np.asarray(inst) == e].sum() == c[e]
    assert (q[np.asarray(inst) < 0] == 0).all()
    # the integer split stays within one token per copy of the objective
    ncopy = np.zeros(R, dtype=np.int64)
    for _, insts in groups:
        for i in insts:
            ncopy[i // ipr] += 1
    qload = np.array([q[r * ipr:(r + 1) * ipr].sum() for r in range(R)])
    assert (qload <= m_star * (1 + REL_TOL) + ncopy + 1).all()
    return res, x, m, q, st


@pytest.mark.parametrize("seed", range(12))
def test_lplb_random(seed):
    rng = np.random.default_rng(900 + seed)
    R = int(rng.choice([2, 3, 5, 8, 16, 31, 64]))
    E_loc = int(rng.integers(1, 5))
    E = R * E_loc
    ipr = E_loc + 1
    inst = np.full(R * ipr, -1, dtype=np.int32)
    for r in range(R):
        inst[r * ipr:r * ipr + E_loc] = np.arange(r * E_loc, (r + 1) * E_loc)
    hot = rng.choice(E, size=int(rng.integers(0, R + 1)), replace=False)
    free = list(rng.permutation(R))
    for e in hot:
        for r in free:
            if r != e // E_loc:
                inst[r * ipr + E_loc] = e
                free.remove(r)
                break
    counts = rng.multinomial(int(rng.integers(1, 2_000_000)),
                             rng.dirichlet(np.full(E, rng.choice([0.1, 0.3, 1.0]))), size=R)
    say(f"case: lplb random seed={seed} R={R} E={E} replicas={int((inst[E_loc::ipr] >= 0).sum())}")
    check_lplb(counts.astype(np.int32), inst, ipr)


@pytest.mark.parametrize("seed", range(40))
def test_lplb_random_multi_slot(seed):
    """Layers with 1-3 redundant slots per rank, so an expert can have up to four copies
    (larger groups, more rank pairs per group): M within the bound of the fp64 simplex
    optimum, the split summing to each count, largest-remainder quotas."""
    rng = np.random.default_rng(3000 + seed)
    R = int(rng.choice([4, 8, 13, 16, 32, 48, 64]))
    E_loc = int(rng.integers(1, 5))
    S2 = int(rng.integers(1, 4))
    E, ipr = R * E_loc, E_loc + S2
    inst = np.full(R * ipr, -1, dtype=np.int32)
    for r in range(R):
        inst[r * ipr:r * ipr + E_loc] = np.arange(r * E_loc, (r + 1) * E_loc)
    free = [S2] * R
    n_copies, n_groups = 0, 0
    target = int(rng.integers(0, R * S2 + 1))
    placed = 0
    for e in rng.permutation(E):
        if placed >= target or n_groups >= 120:
            break
        k = int(rng.integers(1, 4))
        ranks = [int(r) for r in rng.permutation(R) if r != e // E_loc and free[r] > 0][:k]
        if not ranks or n_copies + 1 + len(ranks) > 240:
            continue
        for r in ranks:
            inst[r * ipr + E_loc + (S2 - free[r])] = e
            free[r] -= 1
        placed += len(ranks)
        n_copies += 1 + len(ranks)
        n_groups += 1
    counts = rng.multinomial(int(rng.integers(1, 2_000_000)),
                             rng.dirichlet(np.full(E, rng.choice([0.1, 0.3, 1.0]))), size=R)
    say(f"case: lplb multi-slot seed={seed} R={R} E={E} S={S2} groups={n_groups} copies={n_copies}")
    check_lplb(counts.astype(np.int32), inst, ipr)


def test_lplb_special_cases():
    say("case: lplb special cases")
    # red0: no replicas -> M* = max fixed load, quotas = loads
    R, E_loc = 6, 3
    ipr = E_loc + 1
    inst = np.full(R * ipr, -1, dtype=np.int32)
    for r in range(R):
        inst[r * ipr:r * ipr + E_loc] = np.arange(r * E_loc, (r + 1) * E_loc)
    counts = np.random.default_rng(1).integers(0, 500, (R, R * E_loc)).astype(np.int32)
    res, x, m, q, st = check_lplb(counts, inst, ipr)
    assert m == counts.sum(0).reshape(R, E_loc).sum(1).max()
    assert st[0] == 0 and st[2] == 0
    # one expert over two otherwise empty ranks: M* = c / 2
    counts = np.array([[60, 0], [41, 0]], dtype=np.int32)
    check_lplb(counts, np.array([0, -1, 1, 0], dtype=np.int32), 2)
    # hand example: M* = 60 with a unique split
    counts = np.vstack([[90, 30, 60], np.zeros((2, 3))]).astype(np.int32)
    res, x, m, q, st = check_lplb(counts, np.array([0, 2, 1, 0, 2, -1], dtype=np.int32), 2)
    assert q.tolist() == [60, 0, 30, 30, 60, 0]
    # a replicated expert with no load at all
    counts = np.array([[0, 7], [0, 5]], dtype=np.int32)
    check_lplb(counts, np.array([0, 1, 1, 0], dtype=np.int32), 2)
    # all-zero layer
    check_lplb(np.zeros((4, 8), dtype=np.int32),
               np.array([0, 1, 5, 2, 3, -1, 4, 5, 0, 6, 7, 2], dtype=np.int32), 3)


def test_lplb_layer_full_size():
    """LPLB-shaped layer: R = 64, 256 experts + 32 static replicas, 16384 tokens per rank.
    M against the simplex optimum; reroute/assign on the oracle's quotas bit-exact and the
    whole group's permute on that plan compared on every one of its 8,388,608 rows;
    reroute on the kernel's own quotas by its properties."""
    w = W.LPLB_LAYER
    say("case: lplb layer full size", w)
    ids = W.routing(w)
    inst = W.static_replica_placement(w)
    ipr = w.E_loc + 1
    ids_d = to_dev(ids)
    err = err_word()
    counts, bp = U.load_matrix(ids_d, w.E, err=err)
    counts_o, bp_o = O.load_matrix(ids, w.E)
    assert np.array_equal(host(counts), counts_o)
    res, x, m, q, st = check_lplb(counts_o.astype(np.int32), inst, ipr)
    say(f"lplb: m={m} m*={res['m_star']} iterations={st[2]}")
    # reroute/assign on the oracle's quotas: bit-exact against the oracle
    inst_d = to_dev(inst)
    q_o = res["inst_quota"]
    X_o, io_o, so_o = O.reroute(counts_o, inst, q_o, ipr)
    di_o, dr_o = O.assign(ids, bp_o, X_o, inst, ipr, io_o, so_o)
    xfer, ioff, di, dr = U.reroute_assign(counts, ids_d, bp, ipr, inst_d, to_dev(q_o), err=err)
    assert host(err)[0] == 0
    assert np.array_equal(host(xfer), X_o) and np.array_equal(host(ioff), io_o)
    assert np.array_equal(host(di), di_o) and np.array_equal(host(dr), dr_o)
    # permute of the whole group (hidden 7168, 112 GiB) on that plan: every row compared
    gen = torch.Generator(device=DEV).manual_seed(W.tensor_seed(w, 0, 0))
    x_act = torch.randn(w.R, w.T, w.H, generator=gen, device=DEV, dtype=torch.bfloat16)
    out = torch.empty(w.P, w.H, dtype=torch.bfloat16, device=DEV)
    row_src = torch.empty(w.P, dtype=torch.int32, device=DEV)
    U.permute(x_act, dr, out, row_src)
    torch.cuda.synchronize()
    src_o = compare_dispatch_rows(x_act, out, dr_o)
    assert np.array_equal(host(row_src), src_o)
    del out, row_src, x_act
    torch.cuda.empty_cache()
    # reroute/assign on the kernel's own quotas: properties
    xfer, ioff, di, dr = U.reroute_assign(counts, ids_d, bp, ipr, inst_d, to_dev(q), err=err)
    assert host(err)[0] == 0
    Xg = host(xfer)
    check_reroute_properties(counts_o, inst, q, ipr, Xg)
    drh = host(dr)
    assert np.array_equal(np.sort(drh.reshape(-1)), np.arange(w.P))


# ---------------------------------------------------------------- per-token copy draw

def random_lplb_case(rng, R, E_loc, T, K, n_hot):
    E = R * E_loc
    ipr = E_loc + 1
    inst = np.full(R * ipr, -1, dtype=np.int32)
    for r in range(R):
        inst[r * ipr:r * ipr + E_loc] = np.arange(r * E_loc, (r + 1) * E_loc)
    hot = rng.choice(E, size=n_hot, replace=False)
    free = list(rng.permutation(R))
    for e in hot:
        for r in free:
            if r != e // E_loc:
                inst[r * ipr + E_loc] = e
                free.remove(r)
                break
    p = rng.dirichlet(np.full(E, 0.3))
    ids = np.stack([np.stack([rng.choice(E, K, replace=False, p=p) for _ in range(T)])
                    for _ in range(R)]).astype(np.int32)
    ids[rng.random(ids.shape) < 0.03] = -1
    return ids, inst, ipr, E


def instance_dispatch_oracle(dest_inst, inst_len, ipr):
    """Dispatch layout of sampled instance ids: each instance is a one-copy pseudo-expert."""
    ident = np.arange(inst_len, dtype=np.int64)
    c, bp = O.load_matrix(dest_inst, inst_len)
    q = O.identity_quota(c, ident)
    X, io, so = O.reroute(c, ident, q, ipr)
    _, dr = O.assign(dest_inst, bp, X, ident, ipr, io, so)
    return c, q, dr


@pytest.mark.parametrize("seed", range(5))
def test_lplb_sample_random(seed):
    rng = np.random.default_rng(1300 + seed)
    R = int(rng.choice([2, 4, 8, 16]))
    E_loc = int(rng.integers(1, 4))
    T, K = int(rng.integers(1, 200)), int(rng.integers(1, min(R * E_loc, 6) + 1))
    n_hot = int(rng.integers(0, R + 1))
    ids, inst, ipr, E = random_lplb_case(rng, R, E_loc, T, K, n_hot)
    say(f"case: lplb sample seed={seed} R={R} E={E} T={T} K={K} replicas={n_hot}")
    counts_o, _ = O.load_matrix(ids, E)
    x32 = np.asarray(O.lplb(counts_o, inst, ipr)["x"], dtype=np.float32)
    lp = U.lplb_prepare(inst, R, E, ipr, DEV)
    err = err_word()
    seed_, layer = 77 + seed, 3
    di = U.lplb_sample(to_dev(ids), lp, to_dev(x32 if x32.size else np.zeros(1), torch.float32),
                       seed_, layer, err=err)
    di_o = O.lplb_sample(ids, inst, ipr, E, x32, seed_, layer)
    assert host(err)[0] == 0
    assert np.array_equal(host(di), di_o)
    # the dispatch layout of the drawn instances, bit-exact
    I = len(inst)
    c_o, q_o, dr_o = instance_dispatch_oracle(di_o, I, ipr)
    c, bp = U.load_matrix(di, I, err=err)
    ident = to_dev(np.arange(I))
    q = U.identity_quota(c, ident)
    _, _, _, dr = U.reroute_assign(c, di, bp, ipr, ident, q, err=err)
    assert host(err)[0] == 0
    assert np.array_equal(host(c), c_o) and np.array_equal(host(q), q_o)
    assert np.array_equal(host(dr), dr_o)


def test_lplb_sample_errors_and_layouts():
    """An id out of range and an expert without an instance leave -1 on their pair and
    raise their error bits while every other pair is drawn as usual; a structure built
    for another R leaves every pair -1; ids and outputs that are not 16-byte aligned
    (K % 4 == 0) take the scalar loads and stores; K = 6 has a half-empty second quad."""
    for K in (4, 6):
        rng = np.random.default_rng(1400 + K)
        R, E_loc, T = 4, 3, 150
        ids, inst, ipr, E = random_lplb_case(rng, R, E_loc, T, K, 3)
        say(f"case: lplb sample errors and layouts R={R} E={E} T={T} K={K}")
        counts_o, _ = O.load_matrix(ids, E)
        # an expert with a single instance loses it; its pairs must come back -1
        single = [e for e in range(E) if (inst == e).sum() == 1 and (ids == e).any()]
        gone = single[0]
        inst2 = inst.copy()
        inst2[inst2 == gone] = -1
        x32 = np.asarray(O.lplb(counts_o, inst, ipr)["x"], dtype=np.float32)
        lp = U.lplb_prepare(inst2, R, E, ipr, DEV)
        xd = to_dev(x32 if x32.size else np.zeros(1), torch.float32)
        bad = ids.copy()
        bad[1, 7, 2] = E                                  # out of range
        ref_ids = np.where(bad == gone, -1, bad)
        ref_ids[1, 7, 2] = -1
        di_o = O.lplb_sample(ref_ids, inst2, ipr, E, x32, 5, 1)
        n = ids.size
        big = torch.zeros(n + 4, dtype=torch.int32, device=DEV)
        big[1:1 + n] = to_dev(bad).view(-1)
        out_big = torch.full((n + 4,), -9, dtype=torch.int32, device=DEV)
        for aligned in (True, False):
            err = err_word()
            if aligned:
                di = U.lplb_sample(to_dev(bad), lp, xd, 5, 1, err=err)
            else:
                di = U.lplb_sample(big[1:1 + n].view(R, T, K), lp, xd, 5, 1,
                                   dest_inst=out_big[1:1 + n].view(R, T, K), err=err)
            e = int(host(err)[0])
            assert e & U.ERR_ID_RANGE and e & U.ERR_LP
            assert np.array_equal(host(di), di_o)
        ob = host(out_big)
        assert ob[0] == -9 and (ob[1 + n:] == -9).all()
        # a structure built for 2 ranks, used with 4: the binding refuses it on the host;
        # with its record claiming 4 ranks, the kernel refuses the buffer itself
        inst_small = np.where(inst[:2 * ipr] < 2 * E_loc, inst[:2 * ipr], -1)
        lp2 = U.lplb_prepare(inst_small, 2, 2 * E_loc, ipr, DEV)
        ids_small = to_dev(np.where(ids < 2 * E_loc, ids, -1))
        with pytest.raises(TypeError):
            U.lplb_sample(ids_small, lp2, xd, 5, 1)
        err = err_word()
        di = U.lplb_sample(ids_small, dataclasses.replace(lp2, R=R), xd, 5, 1, err=err)
        assert host(err)[0] & U.ERR_LP and (host(di) == -1).all()


def test_lplb_sample_zero_weight_copy_ahead():
    """R = 4, E = 8 (two mains per rank), expert 0 on instances 0, 5 and 11 with weights
    (0, 1, 0): W = 1, every draw has v = 0 and must take instance 5, never the
    zero-weight copy ahead of it; the oracle agrees pair by pair."""
    say("case: lplb sample zero-weight copy ahead")
    ipr = 3
    inst = np.full(4 * ipr, -1, dtype=np.int32)
    for r in range(4):
        inst[r * ipr:r * ipr + 2] = [2 * r, 2 * r + 1]
    inst[1 * ipr + 2] = 0
    inst[3 * ipr + 2] = 0
    inst[0 * ipr + 2] = 5
    x = np.array([0.0, 1.0 / 256.0, 0.0, 1.0, 1.0], dtype=np.float32)
    ids = np.zeros((4, 300, 1), dtype=np.int32)
    lp = U.lplb_prepare(inst, 4, 8, ipr, DEV)
    err = err_word()
    di = host(U.lplb_sample(to_dev(ids), lp, to_dev(x, torch.float32), 3, 1, err=err))
    assert host(err)[0] == 0 and (di == 5).all()
    assert np.array_equal(di, O.lplb_sample(ids, inst, ipr, 8, x, seed=3, layer=1))


def test_lplb_refuses_a_foreign_structure():
    """A buffer that is not a structure from uep_lplb_prepare (all zeros, or a real one
    with its copy count overwritten beyond the LDS tables) is refused by both kernels:
    the solve writes nothing but UEP_ERR_LP, the draw leaves every pair -1."""
    rng = np.random.default_rng(1500)
    ids, inst, ipr, E = random_lplb_case(rng, 4, 2, 50, 3, 2)
    R = 4
    say("case: lplb foreign structure")
    good = U.lplb_prepare(inst, R, E, ipr, DEV)
    bad_n = good.buf.clone()
    bad_n.view(torch.int32)[6] = 1 << 20                   # n_copies beyond the tables
    for buf in (torch.zeros_like(good.buf), bad_n):
        lp = dataclasses.replace(good, buf=buf)
        err = err_word()
        x = torch.full((8,), -3.0, dtype=torch.float32, device=DEV)
        m = torch.full((1,), -3.0, dtype=torch.float32, device=DEV)
        q = torch.full((len(inst),), -3, dtype=torch.int32, device=DEV)
        st = torch.full((4,), -3, dtype=torch.int32, device=DEV)
        counts = to_dev(O.load_matrix(ids, E)[0])
        U.lplb(counts, lp, iters=30, x=x, m=m, inst_quota=q, stats=st, err=err)
        assert host(err)[0] == U.ERR_LP
        assert (host(x) == -3.0).all() and host(m)[0] == -3.0
        assert (host(q) == -3).all() and (host(st) == -3).all()
        err = err_word()
        di = U.lplb_sample(to_dev(ids), lp, x, 1, 2, err=err)
        assert host(err)[0] == U.ERR_LP and (host(di) == -1).all()


def test_lplb_sample_layer_full_size():
    """LPLB layer: the draw of three source ranks bit-exact on the oracle's split; with
    the kernel's own split, every pair lands on a copy of its expert and each copy's
    share of a replicated expert's tokens is within 5 sigma of w_p / W."""
    w = W.LPLB_LAYER
    say("case: lplb sample full size", w)
    ids = W.routing(w)
    inst = W.static_replica_placement(w)
    ipr = w.E_loc + 1
    counts_o, _ = O.load_matrix(ids, w.E)
    x32 = np.asarray(O.lplb(counts_o, inst, ipr)["x"], dtype=np.float32)
    lp = U.lplb_prepare(inst, w.R, w.E, ipr, DEV)
    ids_d = to_dev(ids)
    err = err_word()
    seed_, layer = 2024, 11
    di = U.lplb_sample(ids_d, lp, to_dev(x32, torch.float32), seed_, layer, err=err)
    some = [0, 40, w.R - 1]
    di_o = O.lplb_sample(ids, inst, ipr, w.E, x32, seed_, layer, ranks=some)
    assert host(err)[0] == 0
    assert np.array_equal(host(di)[some], di_o[some])
    # the kernel's own split, end to end
    groups = copy_groups(inst, w.E)
    n = sum(len(g[1]) for g in groups)
    x, m, q, st = U.lplb(to_dev(counts_o), lp, n, len(inst), iters=30, err=err)
    di = host(U.lplb_sample(ids_d, lp, x, seed_, layer, err=err))
    assert host(err)[0] == 0
    inst_np = np.asarray(inst)
    live = ids >= 0
    assert (inst_np[di[live]] == ids[live]).all() and (di[~live] == -1).all()
    xh = host(x)
    k = 0
    for e, insts in groups:
        wts = np.array([np.rint(max(float(v), 0.0) * 256.0) for v in xh[k:k + len(insts)]])
        k += len(insts)
        tot = int((ids == e).sum())
        if wts.sum() == 0 or tot == 0:
            continue
        p = wts / wts.sum()
        got = np.array([(di == i).sum() for i in insts])
        sigma = np.sqrt(tot * p * (1 - p))
        assert (np.abs(got - tot * p) <= 5 * sigma + 1).all()


def test_lplb_block_and_dense_solves():
    """The rank matrix is solved block by block when every component of the rank coupling
    graph has at most 16 ranks (lane groups of 8 or 16), densely otherwise: the LPLB
    layer's placement (components of at most 8 ranks), a chain of 12 ranks (groups of
    16) and a ring over all 64 ranks (dense) all reach the simplex optimum within the
    bound, and each reports the solve it took."""
    w = W.LPLB_LAYER
    R, E_loc = w.R, w.E_loc
    ipr = E_loc + 1
    ids = W.routing(w)
    counts = O.load_matrix(ids, w.E)[0].astype(np.int32)

    def mains():
        inst = np.full(R * ipr, -1, dtype=np.int32)
        for r in range(R):
            inst[r * ipr:r * ipr + E_loc] = np.arange(r * E_loc, (r + 1) * E_loc)
        return inst
    chain = mains()
    for r in range(11):                       # ranks 0..11 linked: one 12-rank component
        chain[(r + 1) * ipr + E_loc] = r * E_loc
    ring = mains()
    for r in range(R):                        # every rank linked to the next: one component
        ring[((r + 1) % R) * ipr + E_loc] = r * E_loc
    for name, inst, path in (("lplb placement", W.static_replica_placement(w), 8),
                             ("12-rank chain", chain, 16), ("64-rank ring", ring, 0)):
        say(f"case: lplb solve path, {name}")
        res, x, m, q, st = check_lplb(counts, inst, ipr)
        assert st[3] == path, (name, st)


def _placement(rng, R, E_loc, n_hot):
    """Static instance table: E_loc mains per rank and one redundant slot per rank,
    n_hot experts replicated on a rank other than their home."""
    E, ipr = R * E_loc, E_loc + 1
    inst = np.full(R * ipr, -1, dtype=np.int32)
    for r in range(R):
        inst[r * ipr:r * ipr + E_loc] = np.arange(r * E_loc, (r + 1) * E_loc)
    free = list(rng.permutation(R))
    for e in rng.choice(E, size=min(n_hot, R), replace=False):
        for r in free:
            if r != e // E_loc:
                inst[r * ipr + E_loc] = e
                free.remove(r)
                break
    return inst, ipr


def _fused_vs_separate(ids, E, inst, ipr, r_begin=0, r_end=None):
    R = ids.shape[0]
    ids_d, inst_d = to_dev(ids), to_dev(inst)
    lp = U.lplb_prepare(inst, R, E, ipr, DEV)
    e1, e2 = err_word(), err_word()
    counts, bp = U.load_matrix(ids_d, E, err=e1)
    x, m, q, st = U.lplb(counts, lp, iters=30, err=e1)
    xfer, ioff, di, dr = U.reroute_assign(counts, ids_d, bp, ipr, inst_d, q, r_begin, r_end,
                                          err=e1)
    o = U.lplb_plan(ids_d, lp, inst_d, iters=30, r_begin=r_begin, r_end=r_end, err=e2)
    torch.cuda.synchronize()
    assert int(host(e1)[0]) == 0 and int(host(e2)[0]) == 0
    for key, ref in (("counts", counts), ("bucket_pos", bp), ("inst_quota", q), ("stats", st),
                     ("xfer", xfer), ("inst_offset", ioff)):
        assert torch.equal(o[key], ref), key
    assert torch.equal(o["x"][:lp.n].view(torch.int32), x.view(torch.int32))
    assert torch.equal(o["m"].view(torch.int32), m.view(torch.int32))
    rb, re_ = r_begin, (R if r_end is None else r_end)
    assert torch.equal(o["dest_inst"][rb:re_], di[rb:re_])
    assert torch.equal(o["dest_row"][rb:re_], dr[rb:re_])
    return o


# (R, E_loc, T, K, replicated experts): 16-byte ids and the LDS-tiled ranking (K % 4 != 0),
# ranks long enough for many earlier chunks, a rank range, E = 1024 (the ranking's LDS
# close to the LP's whole block) and beyond what fits (the three calls in sequence)
LPLB_PLAN_GEOMS = [(4, 2, 600, 4, 3), (8, 4, 900, 8, 6), (16, 4, 1500, 6, 10),
                   (5, 3, 700, 9, 4), (8, 2, 5000, 4, 5), (5, 4, 300, 16, 3),
                   (16, 64, 300, 8, 8), (16, 128, 200, 8, 4)]


@pytest.mark.parametrize("geom", LPLB_PLAN_GEOMS, ids=[str(g) for g in LPLB_PLAN_GEOMS])
def test_lplb_plan_fused_matches_the_separate_calls(geom):
    """uep_lplb_plan (load matrix, the LP overlapped with the ranking, reroute/assignment
    in one call) gives the three separate calls' outputs bit for bit, the fp32 split and
    objective included; with a rank range it assigns exactly that range."""
    R, E_loc, T, K, n_hot = geom
    rng = np.random.default_rng(sum(geom) * 13 + 5)
    E = R * E_loc
    say(f"case: fused lplb plan R={R} E={E} T={T} K={K} replicated={n_hot}")
    inst, ipr = _placement(rng, R, E_loc, n_hot)
    ids = random_routing(rng, R, T, K, E, empty_frac=0.02)
    _fused_vs_separate(ids, E, inst, ipr)
    if R >= 4:
        _fused_vs_separate(ids, E, inst, ipr, r_begin=1, r_end=3)


def test_lplb_plan_layer_full_size():
    """The fused LPLB plan on the LPLB-shaped layer (R = 64, 256 experts + 32 static
    replicas, 16384 tokens per rank): bit for bit the separate calls' outputs."""
    w = W.LPLB_LAYER
    say("case: fused lplb plan, layer full size", w)
    ids = W.routing(w)
    inst = W.static_replica_placement(w)
    o = _fused_vs_separate(ids, w.E, inst, w.E_loc + 1)
    say(f"fused lplb plan: m={float(host(o['m'])[0])} iterations={int(host(o['stats'])[2])}")
