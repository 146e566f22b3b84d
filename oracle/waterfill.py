"""Oracle: Waterfill placement of the shared expert's slot.

Waterfill/LPLB blog, section "Waterfill算法执行步骤" (Waterfill steps):
1. count the routed-expert load already assigned to every EP rank and use it as the
   rank's load score L_r (in dynamic mode after an EP collective, from the global
   routed-load vector plus every rank's local batch size);
2. add one shared-expert slot per participating token and set the waterline
   H = ceil((sum_r L_r + N) / R), N = number of shared slots, R = EP group size;
3. ranks under the waterline have slack S_r = max(H - L_r, 0);
4. for each token, sample the shared expert's rank among its candidates with
   probability proportional to slack, with a small preference for the local rank;
   if every candidate has zero slack, fall back to a clearly lighter candidate, again
   preferring the local rank.
Section "通信权衡与模式选择": the communication-conservative candidates are the ranks
the token already visits for its routed experts, with its source rank as fallback;
the all-rank mode lets every EP rank take the shared slot (more freedom to balance,
possibly one more destination per token).
Section "共享专家融合作为启用机制": the top-k output gains one extra column for the
shared expert and every rank keeps one shared-expert slot beside its routed experts.

Readings (the page gives no constants):
* L_r = routed pairs whose expert is homed on r (home(e) = e // (E/R)); the local batch
  sizes B_r enter only through N = sum_r B_r (adding them to L_r too would count the
  shared slots twice);
* candidates = the deduplicated set {home(e_k)} plus the source rank r0 (all-rank
  mode: every rank), in the order r0 first, then the others ascending;
* weights: 2^p * S_c for c != r0 and (2^p + 1) * S_r0 for the source (p = 4: a 1/16 bonus);
* with W = sum of weights > 0: u = word 0 of Philox4x64-10(counter = (g, 0, 0, 0),
  key = (seed, layer)) for the global token index g = r0*T + t; v = floor(u * W / 2^64);
  the first candidate whose running weight exceeds v wins;
* with W = 0: r0, unless some candidate c has (2^p + 1) * L_c < 2^p * L_r0; then the
  lightest such c (lowest rank on ties);
* slack is not updated token by token;
* tokens t >= B_r0 are absent: shared rank -1.

Pins: H and S_r closed form, sum_r S_r >= N, candidate set {r0} -> r0, the zero-slack
fallback on hand-made cases, the sampled distribution within 4 sigma of the weights;
all-rank mode without the local bonus: each rank's share of the shared slots within
4 sigma of N * S_r / sum S, so the expected load L_r + shared_r stays at or below H.
"""

import numpy as np

from .philox import philox4x64_10_np


def waterfill(counts, topk_ids, batch_size, seed: int, layer: int, local_pref_shift: int = 4,
              all_ranks: bool = False, ranks=None):
    """Returns (shared_rank [R][T] int64, H, S [R] int64, L [R] int64).

    ``ranks`` limits the per-token draws to those source ranks (others stay -1);
    H, S and L always cover the whole group."""
    counts = np.asarray(counts, dtype=np.int64)
    ids = np.asarray(topk_ids, dtype=np.int64)
    B = np.asarray(batch_size, dtype=np.int64)
    R, E = counts.shape
    _, T, K = ids.shape
    if E % R != 0:
        raise ValueError("E must be a multiple of R")
    if (B < 0).any() or (B > T).any():
        raise ValueError("batch sizes must lie in [0, T]")
    E_loc = E // R
    c = counts.sum(axis=0)
    L = np.array([int(c[r * E_loc:(r + 1) * E_loc].sum()) for r in range(R)], dtype=np.int64)
    N = int(B.sum())
    H = -(-(int(L.sum()) + N) // R)
    S = np.maximum(H - L, 0)
    big = 1 << local_pref_shift
    g = np.arange(R * T, dtype=np.uint64)
    u_all = philox4x64_10_np(g, (seed, layer))[:, 0]
    shared = np.full((R, T), -1, dtype=np.int64)
    for r0 in (range(R) if ranks is None else ranks):
        for t in range(int(B[r0])):
            if all_ranks:
                visited = [c_ for c_ in range(R) if c_ != r0]
            else:
                visited = sorted(set(int(e) // E_loc for e in ids[r0, t] if e >= 0) - {r0})
            cands = [r0] + visited
            w = [(big + 1) * int(S[r0])] + [big * int(S[c_]) for c_ in visited]
            W = sum(w)
            if W > 0:
                u = int(u_all[r0 * T + t])
                v = (u * W) >> 64
                run = 0
                for c_, wc in zip(cands, w):
                    run += wc
                    if run > v:
                        shared[r0, t] = c_
                        break
            else:
                lighter = [(int(L[c_]), c_) for c_ in visited
                           if (big + 1) * int(L[c_]) < big * int(L[r0])]
                shared[r0, t] = min(lighter)[1] if lighter else r0
    return shared, H, S, L


def extend_topk(topk_ids, shared_rank, E: int):
    """Top-k with one extra column: pseudo-expert E + d for the shared slot on rank d."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    sh = np.asarray(shared_rank, dtype=np.int64)
    col = np.where(sh >= 0, E + sh, -1)
    return np.concatenate([ids, col[:, :, None]], axis=2)
