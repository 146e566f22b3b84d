"""Oracle: the global load matrix of one layer.

UltraEP article, section "在 Gate 之后获取当前层真实负载" (real load after Gate):
after the Gate every expert's exact token count for the current microbatch and
layer is known; the routing metadata of the whole EP group is gathered into a
global load matrix.  The Waterfill/LPLB blog, section "从全局计数到LP求解的工程实现",
has each rank count its own tokens per logical expert in the same way.

Readings (the pages are silent):
* load unit = one (token, expert) pair, i.e. one GEMM row;
* an id of -1 marks an empty routing slot (a padded or absent token) and is not counted;
* ``bucket_pos`` is the stable position of a pair inside its (rank, expert) bucket,
  counting tokens in ascending index: the number of earlier tokens t' < t on the same
  rank that also route to that expert.  It is what fixes which concrete token goes to
  which instance later.

Pins: np.bincount totals, hand-worked example (tests/golden/load_matrix_hand.json),
bucket invariants (each bucket is exactly 0..count-1 in token order), brute force.
"""

import numpy as np


class OracleInputError(ValueError):
    """Routing that the path rejects: ids outside [-1, E) or an id twice in one token."""


def check_routing(topk_ids: np.ndarray, E: int) -> None:
    ids = np.asarray(topk_ids)
    if ids.ndim != 3:
        raise OracleInputError("topk_ids must be [R][T][K]")
    if ((ids < -1) | (ids >= E)).any():
        raise OracleInputError("expert id out of range")
    s = np.sort(ids, axis=2)
    if ((s[:, :, 1:] == s[:, :, :-1]) & (s[:, :, 1:] >= 0)).any():
        raise OracleInputError("an expert appears twice in one token's top-k")


def load_matrix(topk_ids: np.ndarray, E: int):
    """counts[r][e] and bucket_pos[r][t][k] (int64; -1 where the id is -1)."""
    ids = np.asarray(topk_ids).astype(np.int64)
    check_routing(ids, E)
    R, T, K = ids.shape
    counts = np.zeros((R, E), dtype=np.int64)
    bucket_pos = np.full((R, T, K), -1, dtype=np.int64)
    for r in range(R):
        flat = ids[r].reshape(-1)          # pair j = t*K + k, so pair order is token order
        valid = flat >= 0
        counts[r] = np.bincount(flat[valid], minlength=E)
        # A stable sort by expert keeps pairs of one expert in token order.  Ids are
        # distinct inside a token, so the j-th pair of a bucket is its j-th token.
        key = np.where(valid, flat, E)
        order = np.argsort(key, kind="stable")
        start = np.concatenate(([0], np.cumsum(counts[r])))   # bucket starts in sorted order
        pos_sorted = np.arange(flat.size) - start[key[order]]
        pos = np.empty(flat.size, dtype=np.int64)
        pos[order] = pos_sorted
        pos[~valid] = -1
        bucket_pos[r] = pos.reshape(T, K)
    return counts, bucket_pos
