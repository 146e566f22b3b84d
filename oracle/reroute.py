"""Oracle: local-first reroute and per-token assignment.

UltraEP article, section "Quota 同时决定专家副本与 token 分流": once quotas are fixed,
tokens first use the instance of their expert on their own rank; when that local
quota is used up, the rest go to instances on other ranks according to those
instances' remaining quota, which keeps every instance at its quota while cutting
cross-rank traffic; finally the aggregate quotas are realised per token, fixing the
instance every token is sent to.

Readings (the article prints no rule beyond the above):
* local pass: X[r][l] = min(C[r][e], q_l) for the instance l of e on rank r;
* remote pass "by remaining quota" = interval overlap (north-west-corner fill): for
  each expert, lay the residual demands end to end in ascending source rank and the
  remaining capacities end to end in ascending physical instance id; the tokens a
  source sends to an instance are the length of the overlap of their two intervals;
* per token: the tokens of (r, e), in ascending token index, fill first the local
  instance, then the remote instances of e in ascending physical id;
* dispatch layout: instance blocks in physical-id order, inside a block source rank
  ascending, then token index ascending.

Pins (tests/test_oracle_reroute.py): both marginals of X, the local-first property,
the monotone-staircase property (which, with the marginals, fixes the remote part
uniquely), dest_row a bijection with block/order properties, a hand-worked example.
"""

import numpy as np


def _instances_of(inst_expert: np.ndarray, e: int):
    return [int(i) for i in np.nonzero(np.asarray(inst_expert) == e)[0]]


def identity_quota(counts: np.ndarray, inst_expert: np.ndarray) -> np.ndarray:
    """Quota of each instance when every expert has exactly one instance: its total load."""
    c = np.asarray(counts, dtype=np.int64).sum(axis=0)
    inst_expert = np.asarray(inst_expert)
    q = np.zeros(inst_expert.size, dtype=np.int64)
    for i, e in enumerate(inst_expert):
        if e >= 0:
            q[i] = c[e]
    return q


def reroute(counts, inst_expert, inst_quota, inst_per_rank: int):
    """Transfer matrix X[r][i], inst_offset[I+1], src_offset[r][i]."""
    C = np.asarray(counts, dtype=np.int64)
    inst_expert = np.asarray(inst_expert, dtype=np.int64)
    q = np.asarray(inst_quota, dtype=np.int64)
    R, E = C.shape
    I = inst_expert.size
    if I != R * inst_per_rank:
        raise ValueError("instance table size mismatch")
    if (q < 0).any() or (q[inst_expert < 0] != 0).any():
        raise ValueError("invalid quotas")
    X = np.zeros((R, I), dtype=np.int64)
    for e in range(E):
        insts = _instances_of(inst_expert, e)              # ascending physical id
        ranks = [i // inst_per_rank for i in insts]
        if len(set(ranks)) != len(ranks):
            raise ValueError("two instances of one expert on one rank")
        if sum(int(q[i]) for i in insts) != int(C[:, e].sum()):
            raise ValueError(f"quotas of expert {e} do not sum to its load")
        local = {r: i for r, i in zip(ranks, insts)}
        demand = np.zeros(R, dtype=np.int64)
        cap = {i: int(q[i]) for i in insts}
        for r in range(R):                                  # local pass
            if r in local:
                i = local[r]
                x = min(int(C[r, e]), int(q[i]))
                X[r, i] += x
                demand[r] = C[r, e] - x
                cap[i] -= x
            else:
                demand[r] = C[r, e]
        d_lo = np.concatenate(([0], np.cumsum(demand)))     # remote pass: interval overlap
        q_lo = np.cumsum([0] + [cap[i] for i in insts])
        for r in range(R):
            for n, i in enumerate(insts):
                ov = min(d_lo[r + 1], q_lo[n + 1]) - max(d_lo[r], q_lo[n])
                if ov > 0:
                    X[r, i] += ov
    inst_offset = np.concatenate(([0], np.cumsum(q)))
    src_offset = np.vstack([np.zeros((1, I), dtype=np.int64), np.cumsum(X, axis=0)[:-1]])
    return X, inst_offset, src_offset


def assign(topk_ids, bucket_pos, X, inst_expert, inst_per_rank: int, inst_offset, src_offset):
    """dest_inst[r][t][k] and dest_row[r][t][k] (-1 for empty routing slots)."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    bp = np.asarray(bucket_pos, dtype=np.int64)
    X = np.asarray(X, dtype=np.int64)
    inst_expert = np.asarray(inst_expert, dtype=np.int64)
    R, T, K = ids.shape
    E = int(max(inst_expert.max(initial=-1), ids.max(initial=-1))) + 1
    insts_of = {e: _instances_of(inst_expert, e) for e in range(E)}
    dest_inst = np.full((R, T, K), -1, dtype=np.int64)
    dest_row = np.full((R, T, K), -1, dtype=np.int64)
    for r in range(R):
        # For every expert e, the table of (instance, row) that its bucket positions
        # 0, 1, 2, ... on rank r map to, laid out one expert after another.
        tab_inst, tab_row, base = [], [], np.zeros(E + 1, dtype=np.int64)
        for e in range(E):
            segs = []
            loc = [i for i in insts_of[e] if i // inst_per_rank == r]
            if loc:
                segs.append(loc[0])
            segs += [i for i in insts_of[e] if i // inst_per_rank != r]
            n = 0
            for i in segs:
                x = int(X[r, i])
                first = int(inst_offset[i] + src_offset[r, i])
                tab_inst.append(np.full(x, i, dtype=np.int64))
                tab_row.append(np.arange(first, first + x, dtype=np.int64))
                n += x
            base[e + 1] = base[e] + n
        tab_inst = np.concatenate(tab_inst) if tab_inst else np.zeros(0, np.int64)
        tab_row = np.concatenate(tab_row) if tab_row else np.zeros(0, np.int64)
        e_r = ids[r].reshape(-1)
        b_r = bp[r].reshape(-1)
        ok = e_r >= 0
        if (b_r[ok] >= (base[e_r[ok] + 1] - base[e_r[ok]])).any():
            raise ValueError("transfer matrix does not cover the routed tokens")
        slot = base[e_r[ok]] + b_r[ok]
        di = np.full(e_r.size, -1, dtype=np.int64)
        dr = np.full(e_r.size, -1, dtype=np.int64)
        di[ok] = tab_inst[slot]
        dr[ok] = tab_row[slot]
        dest_inst[r] = di.reshape(T, K)
        dest_row[r] = dr.reshape(T, K)
    return dest_inst, dest_row
