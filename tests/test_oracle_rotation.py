"""Pins of the rotated TQ3 variant in the oracle (oracle/rotation.py).

The Sylvester-Hadamard matrix is checked against its closed-form properties,
the fast transform against the explicit matrix product (exactly, on integer
inputs small enough that every fp32 sum is exact), the scale and the inverse
by round trips and one-hot vectors, the query rotation by the invariance of
q . k, and the pool path (demote with signs, page reads) by comparing the
rotated pool's page values with the rotation's own definition.
"""
import numpy as np
import pytest

from oracle import attention as OA, pool as OP, rotation as R, tq3 as OT


@pytest.mark.parametrize("d", [2, 8, 16, 128, 256])
def test_sylvester_closed_form(d):
    H = R.sylvester(d)
    assert H.shape == (d, d) and set(np.unique(H)) <= {-1, 1}
    assert np.array_equal(H, H.T)
    assert np.array_equal(H @ H, d * np.eye(d, dtype=np.int64))
    if d >= 2:                                          # H_2n = [[H_n, H_n], [H_n, -H_n]]
        h = R.sylvester(d // 2)
        assert np.array_equal(H, np.block([[h, h], [h, -h]]))


@pytest.mark.parametrize("d", [8, 128, 256])
def test_fwht_exact_on_integers(d):
    rng = np.random.default_rng(d)
    x = rng.integers(-1000, 1001, (50, d))             # every partial sum stays below 2^24
    got = R.fwht_f32(x.astype(np.float32))
    assert np.array_equal(got.astype(np.int64), x @ R.sylvester(d).T)


def test_fwht_stage_order_is_fixed():
    # the first stage pairs channels 0 and 1: a value with only a 2^-24-sized
    # difference shows the order through fp32 rounding (different orders give
    # different bits); this pins the order used by the byte format
    x = np.zeros(4, dtype=np.float32)
    x[:] = [1.0, 2.0 ** -24, -1.0, 2.0 ** -24]
    got = R.fwht_f32(x)
    a0, a1 = np.float32(1.0) + np.float32(2.0 ** -24), np.float32(1.0) - np.float32(2.0 ** -24)
    b0, b1 = np.float32(-1.0) + np.float32(2.0 ** -24), np.float32(-1.0) - np.float32(2.0 ** -24)
    want = np.array([a0 + b0, a1 + b1, a0 - b0, a1 - b1], dtype=np.float32)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("d", [128, 256])
def test_rotation_scale_and_inverse(d):
    assert R.rot_scale(256) == 1 / 16 and R.rot_scale(128) == 1 / 8
    s = R.random_signs(d, 3)
    assert set(np.unique(s)) <= {-1, 1}
    # one-hot rows: c * s_k * column k of H, exactly
    for k in (0, 1, d // 2 + 3, d - 1):
        e = np.zeros(d, dtype=np.float32)
        e[k] = 1.0
        y = R.rotate_f32(e, s)
        assert np.array_equal(y.astype(np.float64), R.rot_scale(d) * s[k] * R.sylvester(d)[:, k])
    rng = np.random.default_rng(d + 1)
    x = rng.standard_normal((20, d)).astype(np.float32)
    back = R.unrotate_f64(R.rotate_f32(x, s), s)
    assert np.abs(back - x).max() <= 4e-6 * np.abs(x).max()
    if d == 256:                                        # orthonormal at d = 256: norms kept
        y = R.rotate_f32(x, s).astype(np.float64)
        assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x.astype(np.float64), axis=1), rtol=1e-6)


@pytest.mark.parametrize("d", [128, 256])
def test_query_rotation_keeps_scores(d):
    rng = np.random.default_rng(7 * d)
    s = R.random_signs(d, 5)
    q = rng.standard_normal((6, d))
    k = rng.standard_normal((9, d))
    qr = R.rotate_query_f64(q, s)
    y = np.stack([(R.sylvester(d) @ (s * kk)) * R.rot_scale(d) for kk in k])   # exact fp64 rotation of k
    assert np.allclose(qr @ y.T, q @ k.T, rtol=1e-12, atol=1e-12)
    assert np.allclose(R.unrotate_f64(y, s), k, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("d", [128, 256])
def test_pool_demote_with_signs(d):
    hkv = 2
    rng = np.random.default_rng(11 + d)
    n = 3
    s = R.random_signs(d, d)
    plain = OP.Pool(hkv, d, n, n, 0.5, 2.0)
    rot = OP.Pool(hkv, d, n, n, 0.5, 2.0, signs=s)
    raw = rng.integers(0, 256, (n, plain.fp8.shape[1])).astype(np.uint8)
    raw[(raw & 0x7F) == 0x7F] = 0x7E
    plain.fp8[:] = raw
    rot.fp8[:] = raw
    OP.demote(plain, np.arange(n), n + np.arange(n))
    OP.demote(rot, np.arange(n), n + np.arange(n))
    assert not np.array_equal(plain.tq3, rot.tq3)
    for p in range(n):
        x = OP.fp8_page_values(rot, p)                   # fp32 [Hkv][2][16][d]
        y = R.rotate_f32(x, s)
        G = d // OT.GROUP
        u, sc = OT.quantize_groups(y.reshape(hkv, 2, 16, G, OT.GROUP))
        want = R.unrotate_f64(OT.dequantize_groups(u, sc).reshape(hkv, 2, 16, d), s)
        assert np.array_equal(OP.page_values(rot, n + p), want)
        # the rotated cache approximates the FP8 values: the TQ3 error is at
        # most half a scale step per rotated element, and the rotation keeps
        # (d = 256) or scales (d = 128: by 1/sqrt 2 back) the row norms
        err = np.linalg.norm(OP.page_values(rot, n + p) - x, axis=-1)
        bound = np.linalg.norm(0.5 * np.repeat(sc, OT.GROUP, axis=-1).reshape(hkv, 2, 16, d), axis=-1)
        assert (err <= bound * (1.0 if d == 256 else np.sqrt(2)) * (1 + 1e-9) + 1e-12).all()


def test_value_path_matches_pool_path_with_signs():
    d, T = 128, 40
    rng = np.random.default_rng(2)
    s = R.random_signs(d, 9)
    x = rng.standard_normal((T, d)).astype(np.float32) * 3
    is_tq3 = np.array([True, False, True])
    got = OP.quantized_values(x, is_tq3, 1.0, s)
    # byte path: one head, K = V = x
    pool = OP.Pool(1, d, 3, 3, 1.0, 1.0, signs=s)
    k = x.reshape(1, T, 1, d)
    OP.append(pool, k, k, np.array([0, 3]), np.arange(3), [0])
    OP.demote(pool, np.array([0, 2]), np.array([3, 5]))
    bt = np.array([3, 1, 5])
    K, V = OP.gather_kv(pool, np.array([0, 3]), bt, 0, T)
    assert np.array_equal(got, K[:, 0]) and np.array_equal(got, V[:, 0])
    # and attention over it equals attention with the rotated query over the rotated keys
    q = rng.standard_normal((3, d)).astype(np.float32)
    o, lse = OA.decode_attention(q, K, V)
    assert np.isfinite(o).all() and np.isfinite(lse).all()


# ---- unrotate_f32: the dense value of a rotated TQ3 element -----------------

@pytest.mark.parametrize("d", [128, 256])
def test_unrotate_f32_spikes_are_exact(d):
    # y = v e_k: every butterfly adds a zero, so x = signs . H[:, k] v / (c d) exactly
    s = R.random_signs(d, 3 + d)
    H = R.sylvester(d)
    for k, v in ((0, 1.5), (1, -0.375), (d - 1, 6144.0), (d // 3, 2.0 ** -20)):
        y = np.zeros(d, dtype=np.float32)
        y[k] = v
        want = (s.astype(np.float64) * H[:, k] * v / (R.rot_scale(d) * d)).astype(np.float32)
        assert np.array_equal(R.unrotate_f32(y, s), want)


@pytest.mark.parametrize("d", [128, 256])
def test_unrotate_f32_inverts_the_rotation_on_integers(d):
    # small integers: every fp32 sum of both transforms is exact, c and 1/(c d)
    # are powers of two, so the round trip returns x bit for bit
    rng = np.random.default_rng(5)
    s = R.random_signs(d, 9)
    x = rng.integers(-64, 65, (7, d)).astype(np.float32)
    assert np.array_equal(R.unrotate_f32(R.rotate_f32(x, s), s), x)


@pytest.mark.parametrize("d", [128, 256])
def test_unrotate_f32_within_the_butterfly_bound(d):
    # each of the log2(d) stages rounds every element once, by at most 2^-24 of
    # a partial sum, itself at most sum |y|: |fp32 - exact| <= log2(d) 2^-24 sum|y| / (c d)
    rng = np.random.default_rng(6)
    s = R.random_signs(d, 10)
    y = (rng.standard_normal((50, d)) * np.exp(rng.uniform(-8, 8, (50, 1)))).astype(np.float32)
    got = R.unrotate_f32(y, s).astype(np.float64)
    exact = R.unrotate_f64(y, s)
    bound = np.log2(d) * 2.0 ** -24 * np.abs(y.astype(np.float64)).sum(axis=-1, keepdims=True) / (R.rot_scale(d) * d)
    assert (np.abs(got - exact) <= bound * (1 + 1e-12)).all()
    assert (np.abs(got - exact) > 0).any()                 # the fp32 path does round somewhere


def test_dense_values_of_a_rotated_page_take_the_fp32_inverse():
    from oracle import dense as OD
    d, hkv, n = 128, 2, 2
    rng = np.random.default_rng(12)
    s = R.random_signs(d, 4)
    rot = OP.Pool(hkv, d, n, n, 0.75, 1.25, signs=s)
    raw = rng.integers(0, 256, (n, rot.fp8.shape[1])).astype(np.uint8)
    raw[(raw & 0x7F) == 0x7F] = 0x7E
    rot.fp8[:] = raw
    OP.demote(rot, np.arange(n), n + np.arange(n))
    for p in range(n):
        y = OP.tq3_page_codes_values(rot, n + p)
        got = OD.page_fp32(rot, n + p)
        assert got.dtype == np.float32
        assert np.array_equal(got, R.unrotate_f32(y.astype(np.float32), s))
        # and it is the fp64 page value to within the butterfly bound
        bound = np.log2(d) * 2.0 ** -24 * np.abs(y).sum(axis=-1, keepdims=True) / 16
        assert (np.abs(got - OP.page_values(rot, n + p)) <= bound * (1 + 1e-12)).all()
