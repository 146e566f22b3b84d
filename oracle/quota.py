"""Oracle: joint replica placement + quota solve (the control plane's planner).

UltraEP article, section "Quota 同时决定专家副本与 token 分流" (quota decides both
replicas and the token split):
* a quota is the token load an expert instance receives after rerouting;
* one search solves replication and quotas together: every step may instantiate a
  new replica and updates the target quota distribution;
* constraints: a fixed number of redundant slots per rank, never two instances of one
  logical expert on one rank, and a new replica must get at least a minimum quota
  (1024 in production) so that no replica is made for a handful of tokens.
Section "共享冗余 slot 管理动态专家副本" (shared redundant slots): mains never move; a
logical expert has one main plus zero or more temporary replicas in the slots.
Section "在 Gate 之后获取当前层真实负载": every rank runs the same deterministic solve.

The article does not print the search.  Reading used here ("fill to the waterline"):

    c_e   = total load of expert e;  L_r = sum of c_e over the mains homed on r
    T*    = ceil(sum_e c_e / R)      (the force-balanced per-rank load)
    start from the identity plan (every main keeps its whole load, no replicas)
    repeat:
      h = the most loaded rank (lowest index on ties); stop if L_h <= T*
      try the mains of h in order (quota descending, expert id ascending), skipping
      empty ones; for a donor expert e: among ranks t != h with a free slot, no
      instance of e and L_t < T*, take the least loaded (lowest index on ties);
      d = min(q_main[e], L_h - T*, T* - L_t); only if d >= q_min put e into t's
      lowest free slot with quota d; the first donor that can move applies its move
      and the step ends.
      if no donor of h can move, try a relay (below); if none applies, stop.

    relay (the article's other kind of step, an update of the quota distribution):
      for the donors e of h in the same order, and the ranks x != h with a free slot, no
      instance of e and L_x >= T* (so no receiver by themselves) in ascending index: x
      qualifies when one of its mains f with a non-zero quota has a replica on a rank y
      with L_y < T*;  d2 = min(q_main[f], T* - L_y);  d = min(q_main[e], L_h - T*,
      T* - (L_x - d2));  if d >= q_min, move d2 of f from x's main to y's replica and
      open e in x's lowest free slot with quota d.  The first (e, x) that qualifies is
      the step.

No rank is ever pushed above T* and h's excess falls by d > 0 every step, so the
search ends; every step opens one replica, so there are at most R*S steps.

Relay lemma.  Call (f, y) a live pair when f's main has quota left and y < T* holds
a replica of f.  A rank above T* has only ever donated (ranks at or below T* never
rise above it), so it holds no replica.  A plain step leaves its receiver below T*
with quota left on the donor only when the donor h comes down to exactly T*; a relay
that opens e on x does the same only when h reaches T*.  So each rank gains a live
pair at most once, at the moment it reaches T* from above, and at that moment it
holds nothing.  A relay uses up the pair it takes (y reaches T* or f's main empties),
and its rank x, which needs a live pair of its own to qualify, is therefore exactly
at T*, holds no replica and has exactly one live pair; after the relay x holds only
e, whose pair is the donor's own.  Hence, by induction over the steps: every live
pair is the one its home rank gained on reaching T*, each rank has at most one, and
every qualifying relay rank sits at T* with a single (f, y).  The order of x's mains,
the choice among holders of f, the load order among relay ranks and a test that x
ends below T* therefore never decide anything; the search below states them not at
all and checks the lemma each time a relay rank qualifies.

Home of expert e: rank e // (E/R) (contiguous EP blocks).  Physical instance ids:
i = r*(E_loc+S) + j; j < E_loc is the main of expert r*E_loc + j, j >= E_loc is slot j-E_loc.

Pins (tests/test_oracle_load_quota.py): identity when balanced, S = 0 or q_min too large;
the one-hot-expert closed form; the constraints of the article as invariants;
the step bound; brute force over slot assignments on tiny inputs (quality report).
"""

import numpy as np


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def _relay(h, mains, L, q_main, slot_e, slot_q, free, t_star, q_min, E_loc, R, S) -> bool:
    """One relay step for the stuck heaviest rank h (see the module docstring): frees
    room on a rank x at T* by topping up the replica of one of x's mains on a rank y
    below T*, then opens a replica of h's donor on x."""
    for e in mains:
        for x in range(R):
            if x == h or free[x] == 0 or e in slot_e[x] or L[x] < t_star:
                continue
            pairs = [(f, y) for f in range(x * E_loc, (x + 1) * E_loc) if q_main[f] > 0
                     for y in range(R) if L[y] < t_star and f in slot_e[y]]
            if not pairs:
                continue
            if len(pairs) != 1 or L[x] != t_star:
                raise RuntimeError(f"relay lemma violated at rank {x}: L = {L[x]}, T* = {t_star}, "
                                   f"live pairs {pairs}")
            f, y = pairs[0]
            d2 = min(q_main[f], t_star - L[y])
            d = min(q_main[e], L[h] - t_star, t_star - (L[x] - d2))
            if d < q_min:
                continue
            slot_q[y][slot_e[y].index(f)] += d2
            q_main[f] -= d2
            L[y] += d2
            s = S - free[x]
            slot_e[x][s] = e
            slot_q[x][s] = d
            free[x] -= 1
            q_main[e] -= d
            L[h] -= d
            L[x] += d - d2
            return True
    return False


def solve_quota(counts: np.ndarray, S: int, q_min: int) -> dict:
    counts = np.asarray(counts, dtype=np.int64)
    R, E = counts.shape
    if E % R != 0:
        raise ValueError("E must be a multiple of R")
    E_loc = E // R
    c = [int(v) for v in counts.sum(axis=0)]
    L = [sum(c[r * E_loc:(r + 1) * E_loc]) for r in range(R)]
    t_star = _ceil_div(sum(c), R)
    q_main = list(c)
    slot_e = [[-1] * S for _ in range(R)]
    slot_q = [[0] * S for _ in range(R)]
    free = [S] * R
    steps = 0
    relays = 0
    stuck = False
    while True:
        h = max(range(R), key=lambda r: (L[r], -r))     # max load, lowest index on ties
        if L[h] <= t_star:
            break
        mains = [e for e in range(h * E_loc, (h + 1) * E_loc) if q_main[e] > 0]
        mains.sort(key=lambda e: (-q_main[e], e))
        moved = False
        for e in mains:
            over = L[h] - t_star
            news = [(L[t], t) for t in range(R)
                    if t != h and free[t] > 0 and e not in slot_e[t] and L[t] < t_star]
            if news:
                Lt, t = min(news)
                d = min(q_main[e], over, t_star - Lt)
                if d >= q_min:
                    s = S - free[t]          # slots fill in order and are never released
                    slot_e[t][s] = e
                    slot_q[t][s] = d
                    free[t] -= 1
                    q_main[e] -= d
                    L[h] -= d
                    L[t] += d
                    moved = True
                    break
        if not moved:
            moved = _relay(h, mains, L, q_main, slot_e, slot_q, free, t_star, q_min, E_loc, R, S)
            relays += int(moved)
        if not moved:
            stuck = True
            break
        steps += 1

    ipr = E_loc + S
    inst_expert = np.full(R * ipr, -1, dtype=np.int64)
    inst_quota = np.zeros(R * ipr, dtype=np.int64)
    for r in range(R):
        for j in range(E_loc):
            e = r * E_loc + j
            inst_expert[r * ipr + j] = e
            inst_quota[r * ipr + j] = q_main[e]
        for s in range(S):
            inst_expert[r * ipr + E_loc + s] = slot_e[r][s]
            inst_quota[r * ipr + E_loc + s] = slot_q[r][s]
    n_rep = sum(1 for r in range(R) for s in range(S) if slot_e[r][s] >= 0)
    return {
        "slot_expert": np.array(slot_e, dtype=np.int64).reshape(R, S),
        "inst_expert": inst_expert,
        "inst_quota": inst_quota,
        "rank_load": np.array(L, dtype=np.int64),
        "n_replicas": n_rep,
        "n_steps": steps,
        "n_relays": relays,
        "t_star": t_star,
        "stuck": stuck,
        "inst_per_rank": ipr,
    }
