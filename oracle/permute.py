"""Oracle: permute token activations into per-instance dispatch buffers.

UltraEP article, section "流式通信算子加速动态权重分发" (streaming weight distribution):
once replica weights are in their slots, token dispatch proceeds by the reroute plan.
On one device the local part of dispatch is the permutation itself: every (token,
expert) pair's activation row lands in the row ``dest_row`` of the buffer.

Activations are raw bf16 bits (uint16) and are copied bit for bit.
Pins: out equals x indexed by row_src (numpy fancy index), row_src inverse of dest_row.
"""

import numpy as np


def permute(x_bits: np.ndarray, dest_row: np.ndarray, r_begin: int, r_end: int, n_rows: int):
    """Returns (out [n_rows][H] uint16, row_src [n_rows] int64, written [n_rows] bool).

    Only sources r in [r_begin, r_end) are written; other rows stay 0 / -1 / False.
    """
    x = np.asarray(x_bits)
    R, T, H = x.shape
    K = dest_row.shape[2]
    out = np.zeros((n_rows, H), dtype=x.dtype)
    row_src = np.full(n_rows, -1, dtype=np.int64)
    written = np.zeros(n_rows, dtype=bool)
    for r in range(r_begin, r_end):
        for t in range(T):
            for k in range(K):
                d = int(dest_row[r, t, k])
                if d < 0:
                    continue
                if written[d]:
                    raise ValueError("two pairs target one dispatch row")
                out[d] = x[r, t]
                row_src[d] = (r * T + t) * K + k
                written[d] = True
    return out, row_src, written


def row_sources(dest_row: np.ndarray, n_rows: int) -> np.ndarray:
    """row_src of the whole buffer: for every dispatch row, the flat pair index
    j = (r*T + t)*K + k that targets it, -1 where no pair does.  The content of row d
    is then x[row_src[d] // K] (the token of that pair): the permute's definition with
    the row loop turned around, for full-size checks chunked over rows."""
    flat = np.asarray(dest_row).reshape(-1)
    pairs = np.nonzero(flat >= 0)[0]
    rows = flat[pairs]
    if rows.size and (rows.max() >= n_rows or np.bincount(rows, minlength=n_rows).max() > 1):
        raise ValueError("a pair targets a row outside the buffer, or two pairs one row")
    src = np.full(n_rows, -1, dtype=np.int64)
    src[rows] = pairs
    return src


def rows_of(x_bits: np.ndarray, row_src: np.ndarray, K: int, a: int, b: int) -> np.ndarray:
    """Content of dispatch rows [a, b) given row_sources' map: row d is the activation
    row of the token of pair row_src[d] (rows no pair targets stay zero).  The permute
    written over output rows, so a buffer too large to hold can be produced block by
    block."""
    x = np.asarray(x_bits)
    H = x.shape[-1]
    flat = x.reshape(-1, H)
    src = np.asarray(row_src[a:b])
    out = np.zeros((b - a, H), dtype=x.dtype)
    live = src >= 0
    out[live] = flat[src[live] // K]
    return out


def permute_rows(x_bits: np.ndarray, dest_row: np.ndarray, rows: np.ndarray) -> tuple:
    """Expected content of selected dispatch rows only (for full-size sampled checks).

    Returns (expected rows [len(rows)][H], expected row_src [len(rows)]), found by
    looking the rows up in dest_row.
    """
    x = np.asarray(x_bits)
    R, T, H = x.shape
    K = dest_row.shape[2]
    flat = np.asarray(dest_row).reshape(-1)
    where = {}
    want = set(int(v) for v in rows)
    for j in np.nonzero(np.isin(flat, np.asarray(rows)))[0]:
        where[int(flat[j])] = int(j)
    if set(where) != want:
        raise ValueError("some sampled rows are not targeted by any pair")
    src = np.array([where[int(v)] for v in rows], dtype=np.int64)
    tok = src // K
    return x.reshape(R * T, H)[tok], src
