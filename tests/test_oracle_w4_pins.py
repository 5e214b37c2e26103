"""Pins of the oracle's 4-bit weights (ref.quantize_w4, pack_w4,
sparse_mlp_w4): exact round trips of weights that are codes times an fp16
scale, the rounding bound, ties to even, zero groups, the nibble order, and
the sparse MLP on exactly representable weights against the fp16 one."""
import numpy as np

from oracle import ref


def exact_matrix(rows, cols, seed, s_exp=-6):
    """Weights v * 2^s_exp with integer codes in [-7, 7], each group holding
    a +-7 (so its scale is exactly 2^s_exp)."""
    g = np.random.default_rng(seed)
    v = g.integers(-7, 8, size=(rows, cols)).astype(np.int8)
    v[:, ::ref.W4_GROUP] = np.where(g.random((rows, cols // ref.W4_GROUP)) < 0.5, 7, -7)
    return v, (v.astype(np.float64) * 2.0 ** s_exp).astype(np.float16)


def test_codes_times_an_fp16_scale_round_trip_exactly():
    v, w = exact_matrix(6, 512, 1)
    q, s = ref.quantize_w4(w)
    assert np.array_equal(q, v)
    assert np.all(s == np.float16(2.0 ** -6))
    assert np.array_equal(ref.dequantize_w4(q, s), w.astype(np.float64))


def test_rounding_error_is_at_most_half_a_scale():
    w = (np.random.default_rng(2).standard_normal((8, 1024)) * 0.02).astype(np.float16)
    q, s = ref.quantize_w4(w)
    assert q.min() >= -8 and q.max() <= 7
    err = np.abs(ref.dequantize_w4(q, s) - w.astype(np.float64))
    bound = np.repeat(s.astype(np.float64), ref.W4_GROUP, axis=1) * 0.5 * (1 + 2.0 ** -9)
    assert np.all(err <= bound)
    # the largest entry of each group takes code +-7
    big = np.abs(q.reshape(8, -1, ref.W4_GROUP)).max(axis=2)
    assert np.all(big == 7)


def test_ties_round_to_even_and_zero_groups():
    s = 2.0 ** -4
    row = np.zeros(ref.W4_GROUP)
    row[0] = 7 * s
    row[1:7] = np.array([2.5, 3.5, -2.5, -0.5, 0.5, 6.5]) * s
    w = np.stack([row, np.zeros(ref.W4_GROUP)]).astype(np.float16)
    q, sc = ref.quantize_w4(w)
    assert q[0, :7].tolist() == [7, 2, 4, -2, 0, 0, 6]
    assert sc[0, 0] == np.float16(s) and sc[1, 0] == 0 and not q[1].any()


def test_nibble_order():
    v = np.array([[-8, 7, 0, -1] + [0] * 124], np.int8)
    p = ref.pack_w4(v)
    assert p.shape == (1, 64) and p[0, 0] == 0xF0 and p[0, 1] == 0x78 and p[0, 2] == 0x88


def test_sparse_mlp_on_representable_weights_is_the_fp16_mlp():
    N, d = 64, 256
    _, w1 = exact_matrix(N, d, 3)
    _, w2 = exact_matrix(N, d, 4, s_exp=-7)
    g = np.random.default_rng(5)
    b1 = (g.standard_normal(N) * 0.02).astype(np.float16)
    b2 = (g.standard_normal(d) * 0.02).astype(np.float16)
    y = g.standard_normal((2, d))
    idx = np.sort(g.choice(N, 20, replace=False))
    v1, s1 = ref.quantize_w4(w1)
    v2, s2 = ref.quantize_w4(w2)
    got, a = ref.sparse_mlp_w4(y, v1, s1, b1, v2, s2, b2, idx, residual=y, skip_nonpos=True)
    want, a2 = ref.sparse_mlp(y, w1, b1, w2, b2, idx, residual=y, skip_nonpos=True)
    assert np.allclose(got, want, rtol=0, atol=1e-12) and np.allclose(a, a2, rtol=0, atol=1e-12)
