"""Pins of the oracle's reroute, assignment, permute and staging (CPU only).

Reroute/assignment: UltraEP article, section "Quota 同时决定专家副本与 token 分流".
Permute: section "流式通信算子加速动态权重分发" (dispatch follows the plan).
Staging: sections "共享冗余 slot 管理动态专家副本" and "复用前向方案，完成权重恢复与梯度归约".
"""

import numpy as np
import pytest

import oracle as O
from moe_expert_load_amd import workload as W
from tests.conftest import golden


def check_reroute_properties(counts, inst_expert, inst_quota, ipr, X):
    """Marginals + local-first + north-west-corner staircase (these fix X uniquely)."""
    C = np.asarray(counts)
    R, E = C.shape
    ie = np.asarray(inst_expert)
    q = np.asarray(inst_quota)
    assert (X >= 0).all()
    assert np.array_equal(X.sum(axis=0), q)                          # instance marginal
    for e in range(E):
        insts = np.nonzero(ie == e)[0]
        assert np.array_equal(X[:, insts].sum(axis=1), C[:, e])      # source marginal
        loc = {int(i) // ipr: int(i) for i in insts}
        remote = []
        for r in range(R):
            if r in loc:
                i = loc[r]
                assert X[r, i] == min(C[r, e], q[i])                 # local first
                if C[r, e] > X[r, i]:
                    assert X[r, i] == q[i]
            for i in insts:
                if loc.get(r) != int(i) and X[r, i] > 0:
                    remote.append((r, int(i)))
        # staircase: remote pieces sorted by source are sorted by instance too
        for (r1, i1), (r2, i2) in zip(remote, remote[1:]):
            assert r1 <= r2 and (r1 == r2 or i1 <= i2)
    assert (X[:, ie < 0] == 0).all()


def check_assign_properties(ids, bp, X, inst_offset, src_offset, ipr, dest_inst, dest_row):
    R, T, K = ids.shape
    ok = ids >= 0
    P = int(ok.sum())
    rows = dest_row[ok]
    assert np.array_equal(np.sort(rows), np.arange(P))                # bijection
    for r in range(R):
        for i in range(X.shape[1]):
            sel = (dest_inst[r] == i)
            assert sel.sum() == X[r, i]
            if X[r, i]:
                got = np.sort(dest_row[r][sel])
                lo = inst_offset[i] + src_offset[r, i]
                assert np.array_equal(got, np.arange(lo, lo + X[r, i]))   # one contiguous block
                t_idx, _ = np.nonzero(sel)
                order = np.argsort(dest_row[r][sel])
                assert (np.diff(t_idx[order]) > 0).all()               # token order inside
    # per (rank, expert), in token order: the local instance first, then the remote
    # instances in ascending physical id
    for r in range(R):
        for e in np.unique(ids[r][ok[r]]):
            t_idx, k_idx = np.nonzero(ids[r] == e)                     # ascending t
            seq = [(0 if int(i) // ipr == r else 1, int(i)) for i in dest_inst[r][t_idx, k_idx]]
            assert seq == sorted(seq)


def test_reroute_hand_example():
    g = golden("quota_ep4_hand.json")
    X, io, so = O.reroute(np.array(g["counts"]), np.array(g["inst_expert"]),
                          np.array(g["inst_quota"]), 3)
    assert X.tolist() == g["xfer"]
    assert io.tolist() == g["inst_offset"]


def test_assign_hand_example_two_remote_instances():
    """R = 3, one main per rank, one slot per rank (4 physical ids = r*2 + j).  Expert 0
    has its main (instance 0) and replicas on ranks 1 (instance 3) and 2 (instance 5)
    with quotas 1, 2, 2.  Rank 0 routes tokens 0..3 to expert 0, rank 2 routes token 0.
    Local pass: rank 0 keeps 1 (instance 0), rank 2 keeps 1 (instance 5, 1 left).
    Remote pass: rank 0's 3 remaining tokens fill instance 3 (2) then instance 5 (1).
    Rows: instance blocks at offsets 0 (i0), 1 (i3), 3 (i5); inside i5 rank 0 first."""
    ipr = 2
    ie = np.array([0, -1, 1, 0, 2, 0])
    q = np.array([1, 0, 0, 2, 0, 2])
    ids = np.full((3, 4, 1), -1, dtype=np.int64)
    ids[0, :, 0] = 0
    ids[2, 0, 0] = 0
    counts, bp = O.load_matrix(ids, 3)
    X, io, so = O.reroute(counts, ie, q, ipr)
    assert X[0].tolist() == [1, 0, 0, 2, 0, 1] and X[2].tolist() == [0, 0, 0, 0, 0, 1]
    assert io.tolist() == [0, 1, 1, 1, 3, 3, 5]
    di, dr = O.assign(ids, bp, X, ie, ipr, io, so)
    assert di[0, :, 0].tolist() == [0, 3, 3, 5] and dr[0, :, 0].tolist() == [0, 1, 2, 3]
    assert di[2, 0, 0] == 5 and dr[2, 0, 0] == 4
    assert (di[1] == -1).all() and (dr[2, 1:] == -1).all()
    check_assign_properties(ids, bp, X, io, so, ipr, di, dr)


@pytest.mark.parametrize("seed", range(8))
def test_reroute_assign_properties_random(seed):
    rng = np.random.default_rng(seed)
    R = int(rng.integers(2, 7))
    E = R * int(rng.integers(1, 4))
    K = int(rng.integers(1, min(E, 4) + 1))
    T = int(rng.integers(0, 60))
    S = int(rng.integers(0, 3))
    p = rng.dirichlet(np.full(E, 0.3))
    ids = np.zeros((R, T, K), dtype=np.int64)
    for r in range(R):
        for t in range(T):
            ids[r, t] = rng.choice(E, K, replace=False, p=p)
    ids[rng.random(ids.shape) < 0.05] = -1
    counts, bp = O.load_matrix(ids, E)
    plan = O.solve_quota(counts, S, int(rng.integers(1, 20)))
    ipr = plan["inst_per_rank"]
    X, io, so = O.reroute(counts, plan["inst_expert"], plan["inst_quota"], ipr)
    check_reroute_properties(counts, plan["inst_expert"], plan["inst_quota"], ipr, X)
    di, dr = O.assign(ids, bp, X, plan["inst_expert"], ipr, io, so)
    check_assign_properties(ids, bp, X, io, so, ipr, di, dr)
    assert (dr[ids < 0] == -1).all() and (di[ids < 0] == -1).all()
    for r in range(R):                          # each pair goes to an instance of its expert
        m = ids[r] >= 0
        assert np.array_equal(plan["inst_expert"][di[r][m]], ids[r][m])


def test_reroute_rejects_bad_quotas():
    counts = np.array([[5, 5], [5, 5]])
    inst = np.array([0, -1, 1, -1])
    with pytest.raises(ValueError):
        O.reroute(counts, inst, np.array([10, 0, 9, 0]), 2)     # quota sum mismatch
    with pytest.raises(ValueError):
        O.reroute(counts, np.array([0, 0, 1, -1]), np.array([5, 5, 10, 0]), 2)  # twice on a rank


def test_identity_quota():
    counts = np.array([[1, 2, 3], [4, 5, 6]])
    q = O.identity_quota(counts, np.array([2, -1, 0, 1]))
    assert q.tolist() == [9, 0, 5, 7]


def test_permute_matches_fancy_index():
    w = W.TINY
    ids = W.routing(w)
    counts, bp = O.load_matrix(ids, w.E)
    plan = O.solve_quota(counts, w.S, w.q_min)
    X, io, so = O.reroute(counts, plan["inst_expert"], plan["inst_quota"], plan["inst_per_rank"])
    _, dr = O.assign(ids, bp, X, plan["inst_expert"], plan["inst_per_rank"], io, so)
    rng = np.random.default_rng(0)
    x = rng.integers(0, 1 << 16, (w.R, w.T, 8), dtype=np.uint16)
    out, row_src, written = O.permute(x, dr, 0, w.R, w.P)
    assert written.all()
    assert np.array_equal(out, x.reshape(-1, 8)[row_src // w.K])
    assert np.array_equal(dr.reshape(-1)[row_src], np.arange(w.P))
    # a rank range writes exactly its own rows
    out1, rs1, wr1 = O.permute(x, dr, 1, 3, w.P)
    assert np.array_equal(np.sort(np.nonzero(wr1)[0]), np.sort(dr[1:3].reshape(-1)))
    assert np.array_equal(out1[wr1], out[wr1])
    exp, src = O.permute_rows(x, dr, np.array([0, 5, w.P - 1]))
    assert np.array_equal(exp, out[[0, 5, w.P - 1]]) and np.array_equal(src, row_src[[0, 5, w.P - 1]])
    # two pairs aimed at one row is an invalid plan, and the oracle says so
    bad = dr.copy()
    bad[0, 1, 0] = bad[0, 0, 0]
    with pytest.raises(ValueError):
        O.permute(x, bad, 0, w.R, w.P)
    # the row-order inverse used by full-size checks: the same map as the pair loop's,
    # and the same rows block by block
    assert np.array_equal(O.row_sources(dr, w.P), row_src)
    assert np.array_equal(np.concatenate([O.rows_of(x, row_src, w.K, a, min(w.P, a + 1000))
                                          for a in range(0, w.P, 1000)]), out)
    assert np.array_equal(O.rows_of(x, rs1, w.K, 0, w.P), out1)
    with pytest.raises(ValueError):
        O.row_sources(bad, w.P)
    with pytest.raises(ValueError):
        O.row_sources(dr, w.P - 1)


def test_row_sources_hand_example():
    """One rank, two tokens, top-2, an empty slot, a buffer of four rows: pair 0 -> row 2,
    pair 1 empty, pair 2 -> row 0, pair 3 -> row 1; row 3 is targeted by no pair."""
    dr = np.array([[[2, -1], [0, 1]]])
    assert O.row_sources(dr, 4).tolist() == [2, 3, 0, -1]


def test_slot_memory_arithmetic():
    """Qwen3-235B-A22B expert block 3 x 4096 x 1536 in bf16 with fp32 gradients gives the
    article's 36 MB + 72 MB = 108 MB per rank, and 9.9 GB when reserved for each of 94 layers."""
    g = golden("slot_memory.json")
    w = W.QWEN_SWEEP
    wb = w.expert_elems * 2
    gb = w.expert_elems * 4
    MiB = 1 << 20
    assert wb == g["weights_mb"] * MiB and gb == g["grads_mb"] * MiB
    assert (wb + gb) * w.S == g["total_mb"] * MiB
    assert round(w.layers * (wb + gb) * w.S / (1 << 30), 1) == g["per_layer_gb"]


def test_stage_forward_and_grad_reduce():
    rng = np.random.default_rng(3)
    R, S, E_loc, n = 4, 2, 2, 33
    slot_expert = np.array([[2, -1], [0, 5], [0, -1], [1, 0]])
    main_w = rng.integers(0, 1 << 16, (R * E_loc, n), dtype=np.uint16)
    slot_w = np.zeros((R, S, n), dtype=np.uint16)
    O.stage_forward(slot_expert, main_w, slot_w)
    for r in range(R):
        for s in range(S):
            e = slot_expert[r, s]
            assert np.array_equal(slot_w[r, s], main_w[e] if e >= 0 else np.zeros(n, np.uint16))
    # a rank range fills only its own ranks' slots
    part = np.full((R, S, n), 7, dtype=np.uint16)
    O.stage_forward(slot_expert, main_w, part, 1, 3)
    assert (part[[0, 3]] == 7).all()
    assert np.array_equal(part[1], slot_w[1]) and np.array_equal(part[2, 0], slot_w[2, 0])
    assert (part[2, 1] == 7).all()                       # empty slot untouched
    # integer-valued fp32 data: every partial sum is exact, so the result is the exact sum
    mg = rng.integers(-1000, 1000, (R * E_loc, n)).astype(np.float32)
    sg = rng.integers(-1000, 1000, (R, S, n)).astype(np.float32)
    exp = mg.astype(np.float64).copy()
    for r in range(R):
        for s in range(S):
            if slot_expert[r, s] >= 0:
                exp[slot_expert[r, s]] += sg[r, s]
    O.grad_reduce(slot_expert, mg, sg, E_loc)
    assert np.array_equal(mg.astype(np.float64), exp)
    assert (sg[slot_expert >= 0] == 0).all()
    assert not np.signbit(sg[slot_expert >= 0]).any()
    # general data: within the fp32 bound of the fp64 sum (3 adds at most)
    mg = rng.standard_normal((R * E_loc, n)).astype(np.float32)
    sg = rng.standard_normal((R, S, n)).astype(np.float32)
    exact = mg.astype(np.float64).copy()
    absum = np.abs(mg).astype(np.float64)
    for r in range(R):
        for s in range(S):
            if slot_expert[r, s] >= 0:
                exact[slot_expert[r, s]] += sg[r, s]
                absum[slot_expert[r, s]] += np.abs(sg[r, s])
    O.grad_reduce(slot_expert, mg, sg, E_loc)
    assert (np.abs(mg - exact) <= 4 * 2.0 ** -24 * absum + 1e-30).all()
    # order matters: expert 0 sums rank 1 then rank 2 then rank 3, one add at a time
    mg = np.zeros((R * E_loc, 1), np.float32)
    sg = np.zeros((R, S, 1), np.float32)
    mg[0] = 1.0
    sg[1, 0] = 2.0 ** 24        # slot 0 of rank 1 holds expert 0
    sg[2, 0] = 1.0
    sg[3, 1] = -(2.0 ** 24)
    O.grad_reduce(slot_expert, mg, sg, E_loc)
    # ((1 + 2^24) + 1) - 2^24 in fp32 RNE: 1 + 2^24 -> 2^24 (tie to even), + 1 -> 2^24, - 2^24 -> 0
    assert mg[0, 0] == 0.0
