"""Pins of the combine oracle against facts that do not come from the oracle itself."""

import math

import numpy as np
import pytest

import oracle as O
from oracle.combine import bf16_bits_to_f32, combine_f32, f32_to_bf16_bits


def _bits_of(values):
    return np.asarray(values, dtype=np.float32).view(np.uint32)


def test_bf16_rounding_matches_torch_cast():
    """Round-to-nearest-even of float32 -> bfloat16 is what torch's CPU cast does; the
    cases include exact ties (low half 0x8000) with even and odd kept bits, values
    that round up into the next binade and to infinity, subnormals and zeros."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    hi = rng.integers(0, 1 << 16, 4000, dtype=np.uint32)
    lo = rng.integers(0, 1 << 16, 4000, dtype=np.uint32)
    special_lo = np.array([0x8000, 0x7FFF, 0x8001, 0x0000, 0xFFFF], dtype=np.uint32)
    lo[:5 * 400] = np.repeat(special_lo, 400)
    u = (hi << 16) | lo
    exp = (u >> 23) & 0xFF
    u = u[exp != 0xFF]                                   # finite inputs
    u = np.concatenate([u, _bits_of([0.0, -0.0, 3.3895314e38, 1e-40, -1e-45])])
    x = u.view(np.float32)
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), want)


def test_bf16_widening_is_exact():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = bf16_bits_to_f32(bits)
    finite = ~np.isnan(f)
    assert np.array_equal(f32_to_bf16_bits(f[finite]), bits[finite])


def test_nan_is_quieted_with_sign():
    x = np.array([0x7F800001, 0xFF800001, 0x7FC00000], dtype=np.uint32).view(np.float32)
    out = f32_to_bf16_bits(x)
    assert out.tolist() == [0x7FC0, 0xFFC0, 0x7FC0]


def _toy(rng, R=3, T=7, K=4, E=6, H=24, empty=0.15):
    ids = np.stack([np.stack([rng.choice(E, K, replace=False) for _ in range(T)]) for _ in range(R)])
    ids = ids.astype(np.int32)
    ids[rng.random(ids.shape) < empty] = -1
    counts, bp = O.load_matrix(ids, E)
    plan = O.solve_quota(counts, 1, 1)
    X, io, so = O.reroute(counts, plan["inst_expert"], plan["inst_quota"], plan["inst_per_rank"])
    _, dr = O.assign(ids, bp, X, plan["inst_expert"], plan["inst_per_rank"], io, so)
    x = f32_to_bf16_bits(rng.standard_normal((R, T, H)).astype(np.float32))
    P = int((dr >= 0).sum())
    out, _, _ = O.permute(x, dr, 0, R, P)
    return ids, dr, x, out


@pytest.mark.parametrize("seed", range(3))
def test_one_hot_weights_undo_the_permutation(seed):
    """With weight 1 on one live slot and 0 elsewhere, combine(permute(x)) == x bit for
    bit: every other term is a signed zero and x + 0 = x."""
    rng = np.random.default_rng(seed)
    ids, dr, x, out = _toy(rng)
    R, T, K = dr.shape
    g = np.zeros((R, T, K), dtype=np.float32)
    has = np.zeros((R, T), dtype=bool)
    for r in range(R):
        for t in range(T):
            live = np.nonzero(dr[r, t] >= 0)[0]
            if len(live):
                g[r, t, rng.choice(live)] = 1.0
                has[r, t] = True
    y = O.combine(out, dr, g)
    assert np.array_equal(y[has], x[has])
    assert (y[~has] == 0).all()                 # no live slot: +0.0


def test_power_of_two_weights_on_equal_rows_are_exact():
    """Rows equal to one vector v with weights 1/2, 1/4, 1/8, 1/8 give v exactly."""
    rng = np.random.default_rng(11)
    H = 40
    v = f32_to_bf16_bits(rng.standard_normal(H).astype(np.float32))
    y_disp = np.tile(v, (4, 1))
    dr = np.arange(4, dtype=np.int32).reshape(1, 1, 4)
    g = np.array([[[0.5, 0.25, 0.125, 0.125]]], dtype=np.float32)
    assert np.array_equal(O.combine(y_disp, dr, g)[0, 0], v)


def test_hand_example():
    """Two slots: 0.75 * 1.5 + 0.25 * (-2.25) = 1.125 - 0.5625 = 0.5625 (bf16 0x3F10);
    a third slot with dest -1 is ignored; a rank outside the range stays 0."""
    vals = np.array([[1.5, 3.0], [-2.25, 1.0]], dtype=np.float32)
    y_disp = f32_to_bf16_bits(vals)
    dr = np.array([[[0, 1, -1]], [[1, 0, -1]]], dtype=np.int32)
    g = np.array([[[0.75, 0.25, 9.0]], [[1.0, 1.0, 1.0]]], dtype=np.float32)
    y = O.combine(y_disp, dr, g, 0, 1)
    # column 0: 0.5625; column 1: 0.75 * 3 + 0.25 * 1 = 2.5
    assert y[0, 0].tolist() == [0x3F10, 0x4020]
    assert (y[1] == 0).all()


def test_summation_order_is_ascending_k_in_fp32():
    """Terms 1, 2^-8, 0.75*2^-24, 0.75*2^-24 (rows 1.0, 2^-8, 2^-24, 2^-24; weights 1, 1,
    0.75, 0.75).  In k order each small term is below half an ulp of 1 + 2^-8 (2^-24)
    and is lost: the fp32 sum is 1 + 2^-8, the exact midpoint of the bf16 neighbours
    1.0 and 1 + 2^-7, which rounds to even, 0x3F80.  Adding the two small terms first
    (any other order) or in a wider type gives 1 + 2^-8 + 1.5*2^-24, which rounds to
    1 + 2^-8 + 2^-23 in fp32 and to 0x3F81 in bf16."""
    y_disp = np.array([[0x3F80], [0x3B80], [0x3380], [0x3380]], dtype=np.uint16)
    assert bf16_bits_to_f32(y_disp).ravel().tolist() == [1.0, 2.0 ** -8, 2.0 ** -24, 2.0 ** -24]
    dr = np.arange(4, dtype=np.int32).reshape(1, 1, 4)
    g = np.array([[[1.0, 1.0, 0.75, 0.75]]], dtype=np.float32)
    assert combine_f32(y_disp, dr, g)[0, 0, 0] == np.float32(1 + 2.0 ** -8)
    assert O.combine(y_disp, dr, g)[0, 0].tolist() == [0x3F80]
    # the same terms in reverse slot order: the small ones meet first
    dr_rev = dr[:, :, ::-1].copy()
    g_rev = g[:, :, ::-1].copy()
    assert combine_f32(y_disp, dr_rev, g_rev)[0, 0, 0] == np.float32(1 + 2.0 ** -8 + 2.0 ** -23)
    assert O.combine(y_disp, dr_rev, g_rev)[0, 0].tolist() == [0x3F81]


def test_fp32_sum_within_recursive_summation_bound():
    """|fl(sum) - exact| <= gamma_K * sum |g_k x_k| with gamma_K = K u / (1 - K u),
    u = 2^-24: the bound for K rounded products summed left to right."""
    rng = np.random.default_rng(5)
    ids, dr, x, out = _toy(rng, R=2, T=40, K=6, E=10, H=16, empty=0.1)
    R, T, K = dr.shape
    g = rng.random((R, T, K)).astype(np.float32)
    acc = combine_f32(out, dr, g)
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    rows = bf16_bits_to_f32(out).astype(np.float64)
    for r in range(R):
        for t in range(T):
            for h in range(out.shape[1]):
                terms = [float(g[r, t, k]) * rows[dr[r, t, k], h]
                         for k in range(K) if dr[r, t, k] >= 0]
                exact = math.fsum(terms)
                bound = gamma * sum(abs(v) for v in terms)
                assert abs(float(acc[r, t, h]) - exact) <= bound


def test_rank_range_leaves_other_ranks_zero():
    rng = np.random.default_rng(9)
    ids, dr, x, out = _toy(rng)
    R, T, K = dr.shape
    g = rng.random((R, T, K)).astype(np.float32)
    whole = O.combine(out, dr, g)
    part = O.combine(out, dr, g, 1, 2)
    assert np.array_equal(part[1], whole[1])
    assert (part[0] == 0).all() and (part[2] == 0).all()


def test_combine_tokens_matches_whole():
    rng = np.random.default_rng(8)
    ids, dr, x, out = _toy(rng)
    R, T, K = dr.shape
    g = rng.random((R, T, K)).astype(np.float32)
    y = O.combine(out, dr, g)
    tok = np.array([0, 5, R * T - 1])
    assert np.array_equal(O.combine_tokens(out, dr, g, tok), y.reshape(R * T, -1)[tok])
