"""Property-based pins of the oracle (hypothesis): invariants that hold for every input, each chosen so that a
plausible slip in the oracle (a wrong rounding direction, a dropped sign, an off-by-one in a tie rule, a missing
max subtraction) breaks one of them.  The pages' FP4 format (MarkTechPost retelling, paragraph 4: E2M1 values,
one E4M3 scale per 16 channels), the indexer's Top-K (paragraph 3) and the attention merge (HN summary key
points: window plus sparse retrieval) are the subjects.
"""
import numpy as np
from hypothesis import given, settings, strategies as st, HealthCheck

from oracle import attention as OA
from oracle import formats as OF
from oracle import topk as OT

SETTINGS = settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])

# bf16-representable values over a wide magnitude range, with exact zeros of both signs
bf16_value = st.builds(
    lambda m, e, s: float(np.float32(s * m * 2.0 ** e)),
    st.integers(0, 255), st.integers(-40, 20), st.sampled_from([-1.0, 1.0]))


def _bf16(xs):
    return OF.bf16_to_float(OF.bf16_round(np.asarray(xs, dtype=np.float64)))


@SETTINGS
@given(st.lists(bf16_value, min_size=16, max_size=16))
def test_fp4_block_round_trip_bounds(vals):
    x = _bf16(vals)[None, :]
    codes, scales = OF.fp4_pack(x)
    y = OF.fp4_unpack(codes, scales)[0]
    s = float(OF.e4m3_decode(scales)[0, 0])
    # the scale is the E4M3 value nearest amax / 6 (ties to even): no other code is closer
    amax6 = np.abs(x).max() / 6.0
    grid = OF.e4m3_decode(np.arange(127))
    assert abs(s - amax6) <= np.abs(grid - min(amax6, 448.0)).min() + 1e-300 or amax6 > 448.0
    # every element is within half an E2M1 step of its value (clamped at 6 s), sign kept unless it rounds to 0
    for xi, yi in zip(x[0], y):
        if s == 0.0:
            assert yi == 0.0
            continue
        r = min(abs(xi) / s, 6.0)
        mags = OF.E2M1_MAG
        assert abs(abs(yi) / s - r) <= np.abs(mags - r).min() + 1e-12
        if yi != 0.0:
            assert np.sign(yi) == np.sign(xi)
    # re-packing the dequantised block changes nothing (its values lie on the grid of the same scale)
    c2, s2 = OF.fp4_pack(y[None, :])
    assert np.array_equal(OF.fp4_unpack(c2, s2), y[None, :])


@SETTINGS
@given(st.lists(bf16_value, min_size=16, max_size=16))
def test_fp4_rounding_is_monotone_within_a_block(vals):
    x = _bf16(vals)
    y = OF.fp4_unpack(*OF.fp4_pack(x[None, :]))[0]
    order = np.argsort(np.abs(x), kind="stable")
    assert np.all(np.diff(np.abs(y)[order]) >= 0.0)


@SETTINGS
@given(st.floats(-1000.0, 1000.0, allow_nan=False))
def test_e4m3_encode_is_nearest_and_saturating(v):
    code = int(OF.e4m3_encode(np.array([v]))[0])
    d = float(OF.e4m3_decode(np.array([code]))[0])
    grid = OF.e4m3_decode(np.arange(127))
    a = min(abs(v), 448.0)
    assert abs(abs(d) - a) <= np.abs(grid - a).min()
    assert (code >> 7) == (1 if np.signbit(v) else 0)


@SETTINGS
@given(st.lists(st.integers(-20, 20), min_size=1, max_size=200), st.integers(1, 64), st.randoms())
def test_topk_is_the_ordered_top_set_with_low_position_ties(ints, k, rnd):
    s = np.array(ints, dtype=np.float64)
    # a few invisible candidates
    for i in range(len(s)):
        if rnd.random() < 0.1:
            s[i] = -np.inf
    idx = OT.topk(s, k)
    sel = idx[idx >= 0]
    visible = np.flatnonzero(np.isfinite(s))
    assert len(idx) == k and np.all(idx[len(sel):] == -1)
    assert len(sel) == min(k, len(visible))
    assert np.all(np.diff(sel) > 0)                           # ascending, unique
    rest = np.setdiff1d(visible, sel)
    if len(sel) and len(rest):
        assert s[sel].min() >= s[rest].max()                 # a top set
        tau = s[sel].min()
        # at the boundary value, the lowest positions are taken
        eq_sel = sel[s[sel] == tau]
        eq_rest = rest[s[rest] == tau]
        if len(eq_rest):
            assert eq_sel.max() < eq_rest.min()


@SETTINGS
@given(st.lists(st.integers(-50, 50), min_size=1, max_size=120), st.integers(1, 40), st.randoms())
def test_topk_index_map_follows_positions(ints, k, rnd):
    s = np.array(ints, dtype=np.float64)
    n = len(s)
    positions = np.array(sorted(rnd.sample(range(10 * n + 10), n)), dtype=np.int64)
    perm = np.array(rnd.sample(range(n), n))
    # scores listed in a shuffled slot order with the map naming each slot's position
    got = OT.topk(s[perm], k, index_map=positions[perm])
    want = OT.topk(s, k, index_map=positions)
    assert np.array_equal(got, want)


@SETTINGS
@given(st.integers(1, 4), st.integers(1, 12), st.integers(0, 12), st.integers(0, 2 ** 31 - 1))
def test_merge_of_a_split_equals_attention_over_the_union(H, na, nb, seed):
    g = np.random.default_rng(seed)
    C = 8
    q = g.normal(size=(H, C))
    a = g.normal(size=(na, C)) * 3
    b = g.normal(size=(nb, C)) * 3
    oa, la = OA.attend(q, a, 0.7)
    ob, lb = OA.attend(q, b, 0.7)
    o, l = OA.merge(oa, la, ob, lb)
    ou, lu = OA.attend(q, np.concatenate([a, b]), 0.7)
    assert np.allclose(o, ou, rtol=1e-12, atol=1e-12) and np.allclose(l, lu, rtol=1e-12, atol=1e-12)
    # the merge is symmetric
    o2, l2 = OA.merge(ob, lb, oa, la)
    assert np.allclose(o, o2, rtol=1e-13, atol=1e-13) and np.allclose(l, l2, rtol=1e-13, atol=1e-13)


@SETTINGS
@given(st.integers(1, 4), st.integers(1, 20), st.integers(0, 2 ** 31 - 1))
def test_attention_shift_of_every_row(H, n, seed):
    # adding one vector v to every key/value row adds sigma q.v to every score (the softmax is unchanged), so
    # o moves by v and lse by sigma q.v; o is a convex combination of the rows
    g = np.random.default_rng(seed)
    C = 8
    q = g.normal(size=(H, C))
    rows = g.normal(size=(n, C)) * 4
    v = g.normal(size=C) * 10
    o, l = OA.attend(q, rows, 0.5)
    o2, l2 = OA.attend(q, rows + v, 0.5)
    assert np.allclose(o2, o + v, rtol=1e-10, atol=1e-10)
    assert np.allclose(l2, l + 0.5 * (q @ v), rtol=1e-10, atol=1e-10)
    assert np.all(o <= rows.max(axis=0) + 1e-12) and np.all(o >= rows.min(axis=0) - 1e-12)
