"""Oracle: combine (un-permute) expert outputs from the dispatch buffer back to tokens.

Waterfill/LPLB blog, section "背景知识与设计原则": DeepEP sends each token to the few
routed experts the router chose and brings their outputs back with its combine kernel;
section "共享专家融合作为启用机制": with shared-expert fusion the shared expert is one more
column of the same layout and shares the same dispatch and combine.  The pages do not
write the combine out; the reading here is the standard MoE output, a weighted sum of
the token's expert outputs with the router weights as an input:

    y[r][t] = sum over k with dest_row[r][t][k] >= 0 of  g[r][t][k] * out[dest_row[r][t][k]]

Arithmetic, fixed so that the device kernel can match it bit for bit:
  * bf16 rows are widened to fp32 exactly;
  * each term is one fp32 product, rounded to nearest even;
  * terms are added in ascending k, starting from +0.0, each addition rounded to
    nearest even (no fused multiply-add anywhere);
  * the fp32 sum is rounded to bf16, nearest even (a NaN becomes a quiet NaN with its
    sign kept).

Pins (tests/test_oracle_combine.py): the bf16 rounding against torch's float32 ->
bfloat16 cast, exact ties included; one-hot weights undo the permutation bit for bit;
power-of-two weights on equal rows are exact; the fp32 sum lies within the recursive
summation error bound of the exact sum (math.fsum of exact products); a hand example.
"""

import numpy as np


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    is_nan = ((u >> 23) & 0xFF == 0xFF) & (u & 0x7FFFFF != 0)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    quiet = (u >> 16) | 0x40
    return (np.where(is_nan, quiet, rounded) & 0xFFFF).astype(np.uint16)


def _combine_rows_f32(y_disp_bits, d, g):
    """fp32 sums for a set of tokens: d [n][K] dispatch rows, g [n][K] fp32 weights."""
    n, K = d.shape
    H = y_disp_bits.shape[1]
    acc = np.zeros((n, H), dtype=np.float32)
    for k in range(K):
        live = d[:, k] >= 0
        if not live.any():
            continue
        rows = bf16_bits_to_f32(y_disp_bits[d[live, k]])
        term = g[live, k].astype(np.float32)[:, None] * rows     # fp32 product, RNE
        acc[live] = acc[live] + term                                # fp32 sum, RNE
    return acc


def combine_f32(y_disp_bits: np.ndarray, dest_row: np.ndarray, gate_w: np.ndarray,
                r_begin: int = 0, r_end: int = None) -> np.ndarray:
    """The fp32 sums before the final rounding, [R][T][H] float32 (0 outside the range)."""
    R, T, K = dest_row.shape
    H = y_disp_bits.shape[1]
    r_end = R if r_end is None else r_end
    out = np.zeros((R, T, H), dtype=np.float32)
    for r in range(r_begin, r_end):
        out[r] = _combine_rows_f32(y_disp_bits, np.asarray(dest_row[r]), np.asarray(gate_w[r]))
    return out


def combine(y_disp_bits: np.ndarray, dest_row: np.ndarray, gate_w: np.ndarray,
            r_begin: int = 0, r_end: int = None) -> np.ndarray:
    """y [R][T][H] bf16 bits (uint16) for the sources in [r_begin, r_end); other
    ranks' rows are 0."""
    R, T, K = dest_row.shape
    r_end = R if r_end is None else r_end
    acc = combine_f32(y_disp_bits, dest_row, gate_w, r_begin, r_end)
    y = np.zeros(acc.shape, dtype=np.uint16)
    y[r_begin:r_end] = f32_to_bf16_bits(acc[r_begin:r_end])
    return y


def combine_tokens(y_disp_bits: np.ndarray, dest_row: np.ndarray, gate_w: np.ndarray,
                   tokens: np.ndarray) -> np.ndarray:
    """Expected output rows of selected global tokens g = r*T + t only (for sampled
    checks at full size), [len(tokens)][H] bf16 bits."""
    R, T, K = dest_row.shape
    d = np.asarray(dest_row).reshape(R * T, K)[tokens]
    g = np.asarray(gate_w).reshape(R * T, K)[tokens]
    return f32_to_bf16_bits(_combine_rows_f32(y_disp_bits, d, g))
