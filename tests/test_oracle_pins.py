"""Pins of the CPU oracle against what the pages and mathematics fix (no GPU).

Each test ties one oracle function to something other than itself: a worked
value printed on a page, a closed form, an invariant, a library routine, or
exact rational arithmetic.  A plausible slip (dropped term, wrong sign or
index, transposed operand, wrong summation order) fails at least one of them.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


def _sylvester_pm1(d):
    H = np.array([[1]], dtype=np.int64)
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    return H


# --------------------------------------------------------------------- builders


def test_bit_reversal_worked_values():
    g = json.load(open(os.path.join(GOLDEN, "bit_reversal_d128.json")))
    beta = O.bit_reversal(g["d"])
    for rank, pos in g["rank_to_position"].items():
        assert beta[int(rank) - 1] == pos


def test_bit_reversal_balances_every_power_of_two_group():
    beta = O.bit_reversal(128)
    assert sorted(beta) == list(range(128))
    assert all(beta[beta[k]] == k for k in range(128))  # involution
    for G in (64, 32, 16, 8, 4, 2):
        n = 128 // G
        groups = {int(beta[k]) // G for k in range(n)}
        assert len(groups) == n


def test_bit_reversal_matrix_places_column_k_at_beta_k():
    X = RNG.standard_normal((3, 128))
    P = O.bit_reversal_matrix(128)
    beta = O.bit_reversal(128)
    Y = X @ P
    for k in range(128):
        assert np.array_equal(Y[:, beta[k]], X[:, k])


def test_hadamard_sylvester_entries_and_orthogonality():
    H = O.hadamard(128)
    assert np.array_equal(np.sign(H), _sylvester_pm1(128))
    assert np.allclose(np.abs(H), 1 / np.sqrt(128), rtol=0, atol=1e-17)
    assert np.abs(H.T @ H - np.eye(128)).max() < 1e-14


def test_lemma1_hadamard_equalizes_a_diagonal():
    lam = RNG.exponential(size=128) ** 3
    H = O.hadamard(128)
    diag = np.diag(H.T @ np.diag(lam) @ H)
    assert np.allclose(diag, lam.sum() / 128, rtol=1e-12)


def test_qr_factor_is_orthonormal_upper_triangular_positive():
    G = synth.rotation_gaussian(synth.WORKLOADS["tiny_1h_4k"], "k")
    Q = O.orthonormal_from_gaussian(G)
    Rt = Q.T @ G
    assert np.abs(Q.T @ Q - np.eye(128)).max() < 1e-13
    assert np.abs(np.tril(Rt, -1)).max() < 1e-12
    assert (np.diag(Rt) > 0).all()
    assert np.abs(Q @ Rt - G).max() < 1e-12


def test_oscar_rotation_orthogonal_and_preserves_dot_products():
    wl = synth.WORKLOADS["tiny_1h_4k"]
    R = O.oscar_rotation(synth.rotation_gaussian(wl, "k"))
    assert np.abs(R.T @ R - np.eye(128)).max() < 1e-13
    q, k = RNG.standard_normal((2, 128))
    assert abs((q @ R) @ (k @ R) - q @ k) < 1e-12 * (1 + abs(q @ k))
    R32 = R.astype(np.float32).astype(np.float64)
    assert np.abs(R32.T @ R32 - np.eye(128)).max() < 1e-6


def test_oscar_factor_order_gives_a_constant_importance_diagonal():
    # [OSCAR] §3.4.2: with U the eigenbasis of C, diag(R^T C R) = tr(C)/d only for U.H.P order.
    wl = synth.WORKLOADS["tiny_1h_4k"]
    U = O.orthonormal_from_gaussian(synth.rotation_gaussian(wl, "v"))
    lam = np.sort(RNG.exponential(size=128) ** 4)[::-1]
    C = U @ np.diag(lam) @ U.T
    R = O.oscar_rotation(synth.rotation_gaussian(wl, "v"))
    d = np.diag(R.T @ C @ R)
    assert np.allclose(d, lam.sum() / 128, rtol=1e-10)
    wrong = O.hadamard() @ U @ O.bit_reversal_matrix()
    assert np.abs(np.diag(wrong.T @ C @ wrong) - lam.sum() / 128).max() > 1e-3 * lam.sum() / 128


def test_oscar_rotation_with_identity_basis_is_permuted_hadamard():
    R = O.oscar_rotation(np.diag(np.arange(1.0, 129.0)))
    H = O.hadamard()
    beta = O.bit_reversal()
    for k in range(128):
        assert np.allclose(R[:, beta[k]], H[:, k], atol=1e-15)


# --------------------------------------------------------------------- rotation


def test_rotate_dense_is_exact_when_the_sum_is_representable():
    x = RNG.integers(-8, 9, size=(6, 128)).astype(np.float32)
    R = (_sylvester_pm1(128) * 2.0 ** -4).astype(np.float32)
    exact = (x.astype(np.int64) @ _sylvester_pm1(128)).astype(np.float64) * 2.0 ** -4
    assert np.array_equal(O.rotate_dense(x, R), exact.astype(np.float32))


def test_rotate_dense_sums_in_increasing_channel_order():
    # products 2^53, 1, -2^53: increasing order rounds 2^53+1 to 2^53 (tie to even) -> 0;
    # decreasing order gives 1; the exact sum is 1.
    x = np.zeros((1, 128), np.float32)
    x[0, :3] = [2.0 ** 26, 1.0, -(2.0 ** 26)]
    R = np.zeros((128, 128), np.float32)
    R[:3, 0] = [2.0 ** 27, 1.0, 2.0 ** 27]
    assert O.rotate_dense(x, R)[0, 0] == 0.0


def test_rotate_dense_within_one_ulp_of_exact_and_usually_equal():
    wl = synth.WORKLOADS["tiny_1h_4k"]
    R = O.oscar_rotation(synth.rotation_gaussian(wl, "k")).astype(np.float32)
    x = O.bf16_value(synth.to_bf16_bits(RNG.standard_normal((3, 128)).astype(np.float32)))
    got = O.rotate_dense(x, R)
    n_eq = 0
    for t in range(3):
        for j in range(0, 128, 5):
            ex = O.round_fraction_to_f32(O.exact_dot(x[t], R[:, j]))
            ulp = np.spacing(np.float32(abs(ex)))
            assert abs(float(got[t, j]) - float(ex)) <= ulp
            n_eq += got[t, j] == ex
    assert n_eq >= 0.97 * 3 * len(range(0, 128, 5))


def test_round_fraction_to_f32_matches_ieee_casts():
    for v in RNG.standard_normal(200):
        assert O.round_fraction_to_f32(Fraction(float(v))) == np.float32(v)
    # ties go to even
    one = Fraction(1)
    assert O.round_fraction_to_f32(one + Fraction(1, 2 ** 24)) == np.float32(1.0)
    assert O.round_fraction_to_f32(one + Fraction(3, 2 ** 24)) == np.float32(1.0 + 2 ** -22)


def test_rotate_hadamard_matches_integer_hadamard_and_is_an_involution():
    sign = synth.sign_vector(synth.WORKLOADS["saw_int4_b16_16k"], "k")
    x = RNG.integers(-100, 101, size=(4, 128)).astype(np.float32)
    S = (x.astype(np.int64) * sign[None, :]) @ _sylvester_pm1(128)
    want = (S.astype(np.float64) * (np.sqrt(2.0) / 16)).astype(np.float32)
    assert np.array_equal(O.rotate_hadamard(x, sign), want)
    y = O.fwht_fp64(O.fwht_fp64(x.astype(np.float64)))
    assert np.array_equal(y, 128 * x.astype(np.float64))


def test_rotate_hadamard_close_to_dense_fp64():
    sign = synth.sign_vector(synth.WORKLOADS["saw_int4_b16_16k"], "v")
    x = O.bf16_value(synth.to_bf16_bits(RNG.standard_normal((8, 128)).astype(np.float32)))
    dense = x.astype(np.float64) @ O.saw_rotation_matrix(sign)
    assert np.abs(O.rotate_hadamard(x, sign) - dense).max() < 1e-6


# --------------------------------------------------------------------- clip


def test_clip_index_at_the_pages_ratios():
    j, f = O.clip_index(0.96)
    assert j == 121 and abs(float(f) - 0.92) < 1e-5
    j, f = O.clip_index(0.92)
    assert j == 116 and abs(float(f) - 0.84) < 1e-5
    assert O.clip_index(1.0) == (127, np.float32(0.0))
    with pytest.raises(ValueError):
        O.clip_index(0.0)


def test_clip_threshold_is_the_linear_quantile():
    x = RNG.standard_normal((64, 128)).astype(np.float32) * RNG.exponential(size=(1, 128)).astype(np.float32)
    for rho in (0.96, 0.92, 0.5):
        tau = O.clip_threshold(x, rho)
        lib = np.quantile(np.abs(x).astype(np.float64), float(np.float32(rho)), axis=1, method="linear")
        assert np.allclose(tau, lib, rtol=3e-7, atol=0)
        ys = np.sort(np.abs(x), axis=1)
        j, _ = O.clip_index(rho)
        assert (tau >= ys[:, j]).all() and (tau <= ys[:, j + 1]).all()


def test_clip_tokens_changes_only_values_beyond_tau():
    x = RNG.standard_normal((32, 128)).astype(np.float32)
    c = O.clip_tokens(x, 0.96)
    tau = O.clip_threshold(x, 0.96)[:, None]
    inside = np.abs(x) <= tau
    assert np.array_equal(c[inside], x[inside])
    assert np.array_equal(np.abs(c[~inside]), np.broadcast_to(tau, x.shape)[~inside])
    assert np.array_equal(np.sign(c), np.sign(x))
    assert ((~inside).sum(axis=1) <= 127 - 121).all()
    assert np.array_equal(O.clip_tokens(x, 1.0), x)


# --------------------------------------------------------------------- quantizers


def test_int2_codes_of_a_group_on_the_grid():
    s = np.float32(2.0 ** -3)
    n = RNG.integers(0, 4, size=(128, 128))
    n[:4, :] = np.arange(4)[:, None]          # every level appears in every channel
    zoff = np.array([0.0, 1.0, 1.5, 2.0, 3.0])[RNG.integers(0, 5, size=128)]
    x = (s * (n - zoff[None, :])).astype(np.float32)
    q, s16, z16 = O.quantize_int2_channel_group(x)
    assert np.array_equal(q, n)
    assert (O.bf16_value(s16) == s).all()
    assert np.array_equal(O.bf16_value(z16).astype(np.float64), zoff)
    assert np.array_equal(O.dequantize(q, s16[None], z16[None]), x.astype(np.float64))


def test_int2_symmetric_levels_closed_form():
    x = np.tile(np.array([-1.5, -0.5, 0.5, 1.5], np.float32), 32)[:, None].repeat(128, 1)
    q, s16, z16 = O.quantize_int2_channel_group(x)
    assert (O.bf16_value(s16) == 1.0).all() and (O.bf16_value(z16) == 1.5).all()
    assert np.array_equal(q[:4, 0], [0, 1, 2, 3])


def test_int2_ties_round_half_to_even_and_constant_channel():
    x = np.zeros((128, 128), np.float32)
    x[0, :] = 0.0
    x[1, :] = 3.0                               # a = 0, b = 3 -> s = 1, z = 0
    x[2:, :] = 0.5
    x[3, 0], x[4, 0], x[5, 0] = 1.5, 2.5, 2.0
    x[:, 7] = 0.3                                # constant channel -> s = 1
    q, s16, z16 = O.quantize_int2_channel_group(x)
    assert q[2, 0] == 0 and q[3, 0] == 2 and q[4, 0] == 2 and q[5, 0] == 2
    assert O.bf16_value(s16)[7] == 1.0 and q[0, 7] == 0
    assert O.bf16_value(z16)[7] == O.bf16_value(O.bf16_rne(np.float32(-0.3)))


def test_int2_reconstruction_error_bound():
    x = O.clip_tokens(RNG.standard_normal((128, 128)).astype(np.float32), 0.96)
    q, s16, z16 = O.quantize_int2_channel_group(x)
    xh = O.dequantize(q, s16[None], z16[None])
    sp = O.bf16_value(s16).astype(np.float64)
    zp = np.abs(O.bf16_value(z16)).astype(np.float64)
    bound = 0.5 * sp + sp * (zp + 3) * 2.0 ** -7
    assert (np.abs(xh - x) <= bound[None, :]).all()
    assert q.max() == 3 and q.min() == 0


def test_int4_codes_on_the_grid_and_eq4_rounding_order():
    s = np.float32(2.0 ** -2)
    n = RNG.integers(0, 16, size=(16, 128))
    n[:, 0], n[:, 1] = 0, 15
    x = (s * (n - 8)).astype(np.float32)
    q, s16, z16 = O.quantize_int4_token(x)
    assert np.array_equal(q, n)
    assert (O.bf16_value(z16) == 8).all() and (O.bf16_value(s16) == s).all()
    # eq. (4) rounds x/s first, then adds z: x/s = 2.5, z = 1 -> 2 + 1 = 3 (not rint(3.5) = 4)
    y = np.zeros((1, 128), np.float32)
    y[0, 0], y[0, 1], y[0, 2] = -1.0, 14.0, 2.5
    q, s16, z16 = O.quantize_int4_token(y)
    assert O.bf16_value(s16)[0] == 1.0 and O.bf16_value(z16)[0] == 1.0
    assert q[0, 2] == 3


def test_int4_integer_zero_point_has_one_zero():
    """[SAW] eq. (3): z = round(-min / s) is an integer, so a zero zero point is stored as +0 whatever the
    sign of a zero minimum, or of -min / s below one half."""
    rows = np.zeros((5, 128), np.float32)
    rows[1, :] = -0.0                                 # all -0: b = a, s = 1, -a / s = +0
    rows[2, 1:] = np.linspace(0.25, 3.75, 127)        # minimum +0: -a / s = -0
    rows[3, 0], rows[3, 1:] = -0.0, np.linspace(0.25, 3.75, 127)
    rows[4, 1:] = np.linspace(3.0, 18.0, 127)         # minimum 2^-... > 0 below s / 2: rint(-a / s) = -0
    rows[4, 0] = 0.5
    q, s16, z16 = O.quantize_int4_token(rows)
    assert (z16 == 0).all(), z16                      # bf16 bits of +0
    assert O.bf16_value(s16)[0] == 1.0 and O.bf16_value(s16)[1] == 1.0
    assert (q[0] == 0).all() and (q[1] == 0).all()
    sp = O.bf16_value(s16)[2]
    assert q[2, 0] == 0 and q[2, -1] == 15 and np.array_equal(q[2], q[3])
    assert q[4, 0] == int(np.rint(np.float32(0.5) / O.bf16_value(s16)[4]))


def test_bf16_rne_against_exact_rounding():
    x = (RNG.standard_normal(2000) * 10.0 ** RNG.integers(-20, 20, 2000)).astype(np.float32)
    got = O.bf16_value(O.bf16_rne(x))
    for v, g in zip(x[:300], got[:300]):
        # nearest bf16: 8 significant bits, ties to even
        m, e = np.frexp(np.float64(v))
        scaled = Fraction(float(m)) * 256
        n = scaled.numerator // scaled.denominator
        rem = scaled - n
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
            n += 1
        assert float(g) == float(Fraction(n, 256) * Fraction(2) ** int(e))


# --------------------------------------------------------------------- layout


def test_group_and_band_layout_small_cases():
    assert O.n_groups(4, 4, 128) == 0
    assert O.n_groups(259, 4, 128) == 0
    assert O.n_groups(260, 4, 128) == 1
    assert list(O.band_positions(260, 4, 128)) == list(range(4)) + list(range(132, 260))
    assert list(O.band_positions(3, 4, 128)) == [0, 1, 2]
    T = 4096
    ng = O.n_groups(T, 4, 128)
    assert ng == 30 and T - 4 - 128 * ng in range(128, 256)


# --------------------------------------------------------------------- attention


def test_attend_equal_keys_give_the_mean_value():
    k = np.tile(RNG.standard_normal(128), (7, 1))
    v = RNG.standard_normal((7, 128))
    o = O.attend(RNG.standard_normal((2, 128)), k, v)
    assert np.allclose(o, v.mean(axis=0)[None], atol=1e-14)


def test_attend_two_tokens_sigmoid_and_dominant_token():
    k = np.zeros((2, 128)); k[0, 0] = 1.0
    v = RNG.standard_normal((2, 128))
    q = np.zeros((1, 128)); q[0, 0] = 3.0
    p0 = 1 / (1 + np.exp(-3.0 / np.sqrt(128)))
    assert np.allclose(O.attend(q, k, v)[0], p0 * v[0] + (1 - p0) * v[1], atol=1e-14)
    q[0, 0] = 1e4
    assert np.allclose(O.attend(q, k, v)[0], v[0], atol=1e-12)


def test_attend_offset_invariance_and_library_sdpa():
    import torch
    k = RNG.standard_normal((50, 128)); v = RNG.standard_normal((50, 128))
    q = RNG.standard_normal((4, 128))
    o = O.attend(q, k, v)
    # a shift of all keys by c changes every logit of one query by q.c: per-query invariance
    c = RNG.standard_normal(128)
    for h in range(4):
        assert np.allclose(O.attend(q[h:h + 1], k + c[None], v), o[h:h + 1], atol=1e-12)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None])[0].numpy()
    assert np.allclose(o, ref, atol=1e-12)


def test_pure_band_cache_is_exact_attention_on_bf16_values():
    wl = synth.scaled(synth.WORKLOADS["tiny_1h_4k"], seq_len=100)
    R = O.oscar_rotation(synth.rotation_gaussian(wl, "k")).astype(np.float32)
    k = synth.kv_tokens(wl, 0, 0, 100, "k")[:, 0]
    v = synth.kv_tokens(wl, 0, 0, 100, "v")[:, 0]
    q = synth.queries(wl)[0]
    o, st = O.decode_int2(q, k, v, 100, 4, 128, 0.96, 0.92, R, R)
    assert st["n_groups"] == 0
    kb = O.bf16_value(O.bf16_rne(k)).astype(np.float64)
    vb = O.bf16_value(O.bf16_rne(v)).astype(np.float64)
    assert np.allclose(o, O.attend(q.astype(np.float64), kb, vb), atol=1e-13)


def test_int4_reconstruction_uses_the_transposed_rotation():
    wl = synth.WORKLOADS["saw_int4_b16_16k"]
    sk, sv = synth.sign_vector(wl, "k"), synth.sign_vector(wl, "v")
    x = O.bf16_value(synth.to_bf16_bits(RNG.standard_normal((64, 128)).astype(np.float32)))
    st = O.int4_state(synth.to_bf16_bits(x), synth.to_bf16_bits(x), 64, sk, sv)
    K, V = O.int4_keys_values(st, sk, sv)
    rel = np.linalg.norm(K - x) / np.linalg.norm(x)
    assert rel < 0.12
    wrongK = O.dequantize(st["k_codes"], st["k_s16"][:, None], st["k_z16"][:, None]) @ O.saw_rotation_matrix(sk)
    assert np.linalg.norm(wrongK - x) / np.linalg.norm(x) > 0.8


def test_int2_reconstruction_uses_the_transposed_rotation():
    wl = synth.WORKLOADS["tiny_1h_4k"]
    R = O.oscar_rotation(synth.rotation_gaussian(wl, "k")).astype(np.float32)
    T = 4 + 128 + 128
    k = synth.kv_tokens(wl, 0, 0, T, "k")[:, 0]
    st = O.int2_state(k, k, T, 4, 128, 1.0, 1.0, R, R)
    K, _ = O.int2_keys_values(st, R, R)
    ref = O.bf16_value(O.bf16_rne(k[4:132])).astype(np.float64)
    rel = np.linalg.norm(K[-128:] - ref) / np.linalg.norm(ref)
    xh = O.dequantize(st["k_codes"][0], st["k_s16"][0][None], st["k_z16"][0][None])
    wrong = np.linalg.norm(xh @ R.astype(np.float64) - ref) / np.linalg.norm(ref)
    assert rel < 0.6 and wrong > 1.0


def test_int2_token_quantizer_is_the_channel_quantizer_transposed():
    """Per-token INT2 applies R5's arithmetic along the other axis: the same codes and scale/zero bits as
    the (pinned) per-channel quantizer on the transposed group."""
    r = np.random.default_rng(21)
    x = (r.standard_normal((128, 128)) * r.uniform(0.1, 5.0, size=(128, 1))).astype(np.float32)
    x[7] = 0.25  # a constant token: b == a, so s = 1
    q, s16, z16 = O.quantize_int2_token(x)
    qc, sc, zc = O.quantize_int2_channel_group(x.T)
    assert np.array_equal(q, qc.T) and np.array_equal(s16, sc) and np.array_equal(z16, zc)
    assert O.bf16_value(s16[7]) == 1.0


def test_int2_token_codes_on_the_grid():
    """Tokens built as a + s n with n in {0..3} (s a power of two) get codes n and dequantize exactly."""
    r = np.random.default_rng(22)
    n = r.integers(0, 4, size=(64, 128))
    n[:, 0], n[:, 1] = 0, 3  # every token spans the full range
    a = -r.integers(1, 8, size=(64, 1)).astype(np.float32)
    s = (2.0 ** r.integers(-3, 3, size=(64, 1))).astype(np.float32)
    x = (a + s * n).astype(np.float32)
    q, s16, z16 = O.quantize_int2_token(x)
    assert np.array_equal(q, n)
    assert np.array_equal(O.dequantize(q, s16[:, None], z16[:, None]), x.astype(np.float64))


def test_key_only_state_is_the_identity_rotation_state():
    """R_V = None (key-only rotation) quantizes the bf16 values themselves: the same state as R_V = I,
    whose fp64 rotation is exact; per channel and per token."""
    r = np.random.default_rng(23)
    k = r.standard_normal((600, 128)).astype(np.float32)
    v = r.standard_normal((600, 128)).astype(np.float32)
    RK = O.oscar_rotation(r.standard_normal((128, 128))).astype(np.float32)
    for axis in ("channel", "token"):
        a = O.int2_state(k, v, 600, 4, 128, 0.96, 0.92, RK, None, axis=axis)
        b = O.int2_state(k, v, 600, 4, 128, 0.96, 0.92, RK, np.eye(128, dtype=np.float32), axis=axis)
        for key in ("k_codes", "v_codes", "k_s16", "k_z16", "v_s16", "v_z16"):
            assert np.array_equal(a[key], b[key])
        Ka, Va = O.int2_keys_values(a, RK, None)
        Kb, Vb = O.int2_keys_values(b, RK, np.eye(128, dtype=np.float32))
        assert np.array_equal(Ka, Kb) and np.array_equal(Va, Vb)
    sk = np.where(r.integers(0, 2, 128) == 1, 1, -1).astype(np.int8)
    st = O.int4_state(k, v, 600, sk, None)
    qv, sv, zv = O.quantize_int4_token(O.bf16_value(O.source_to_bf16(v)))
    assert np.array_equal(st["v_codes"], qv) and np.array_equal(st["v_s16"], sv)


@pytest.mark.parametrize("block", [16, 32, 64, 128])
def test_block_hadamard_structure_and_normalization(block):
    """[SAW] eq. (1): diag(sign) . diag(H_h, ..., H_h) is orthogonal, zero outside its h x h blocks, and
    every block is the same normalized Hadamard (entries +-1/sqrt(h), signs flipped by row)."""
    r = np.random.default_rng(block)
    sign = np.where(r.integers(0, 2, 128) == 1, 1, -1).astype(np.int8)
    R = O.saw_rotation_matrix(sign, block)
    assert np.abs(R.T @ R - np.eye(128)).max() < 1e-13
    blk = np.arange(128) // block
    assert np.all(R[blk[:, None] != blk[None, :]] == 0)
    assert np.allclose(np.abs(R[blk[:, None] == blk[None, :]]), 1 / np.sqrt(block), atol=0, rtol=1e-15)
    Hh = O.hadamard(block)
    for i in range(0, 128, block):
        assert np.array_equal(R[i:i + block, i:i + block], sign[i:i + block, None] * Hh)
    assert O.hadamard_scale(block) == pytest.approx(1 / np.sqrt(block), rel=1e-16)


@pytest.mark.parametrize("block", [16, 32, 64])
def test_block_fwht_matches_an_integer_block_hadamard(block):
    """With integer inputs every butterfly is exact: the block FWHT equals x . diag(s) . diag(H_int) exactly,
    then one fp64 multiply by 1/sqrt(h) and one fp32 rounding (reading R2)."""
    r = np.random.default_rng(40 + block)
    x = r.integers(-300, 300, size=(20, 128)).astype(np.float32)
    sign = np.where(r.integers(0, 2, 128) == 1, 1, -1).astype(np.int8)
    Hint = np.rint(O.hadamard(block) * np.sqrt(block)).astype(np.int64)
    want = np.zeros((20, 128), np.int64)
    xs = x.astype(np.int64) * sign[None, :]
    for i in range(0, 128, block):
        want[:, i:i + block] = xs[:, i:i + block] @ Hint
    got = O.rotate_hadamard(x, sign, block)
    assert np.array_equal(got, (want.astype(np.float64) * O.hadamard_scale(block)).astype(np.float32))
    # a vector supported on one block stays there
    e = np.zeros((1, 128), np.float32)
    e[0, block + 3] = 1.0
    y = O.rotate_hadamard(e, sign, block)
    assert np.all(y[0, :block] == 0) and np.all(y[0, 2 * block:] == 0)


def test_block_128_is_the_full_hadamard():
    r = np.random.default_rng(50)
    x = r.standard_normal((10, 128)).astype(np.float32)
    sign = np.where(r.integers(0, 2, 128) == 1, 1, -1).astype(np.int8)
    assert np.array_equal(O.rotate_hadamard(x, sign, 128), O.rotate_hadamard(x, sign))
    assert O.hadamard_scale(128) == O.INV_SQRT128_F64


def test_causal_attention_reduces_to_decode_and_to_prefixes():
    """Prefill attention: the last query (position T-1) sees the whole cache, so it equals the decode
    output; a query at position p equals attention over the first p+1 source tokens in an all-bf16
    cache (no quantized group: S0 + W covers the length)."""
    r = np.random.default_rng(61)
    T = 700
    k = r.standard_normal((T, 128)).astype(np.float32)
    v = r.standard_normal((T, 128)).astype(np.float32)
    q = r.standard_normal((5, 4, 128)).astype(np.float32)
    RK = O.oscar_rotation(r.standard_normal((128, 128))).astype(np.float32)
    RV = O.oscar_rotation(r.standard_normal((128, 128))).astype(np.float32)
    pos = np.array([3, 131, 132, 400, T - 1])
    got = O.prefill_int2(q, pos, k, v, T, 4, 128, 0.96, 0.92, RK, RV)
    want_last, _ = O.decode_int2(q[-1], k, v, T, 4, 128, 0.96, 0.92, RK, RV)
    assert np.abs(got[-1] - want_last).max() < 1e-12
    # all-bf16 cache (W large): causal attention over exact bf16 prefixes
    got_b = O.prefill_int2(q, pos, k, v, T, 4, 1024, 0.96, 0.92, RK, RV)
    kb, vb = O.bf16_value(O.bf16_rne(k)).astype(np.float64), O.bf16_value(O.bf16_rne(v)).astype(np.float64)
    for i, p in enumerate(pos):
        assert np.abs(got_b[i] - O.attend(q[i], kb[:p + 1], vb[:p + 1])).max() < 1e-12
    # positions of a state: band first (sink + tail), then the groups
    st = O.int2_state(k, v, T, 4, 128, 0.96, 0.92, RK, RV)
    tp = O.token_positions(st, T, 4, 128)
    assert sorted(tp.tolist()) == list(range(T))


def test_int4_prefill_is_decode_over_each_prefix():
    """INT4 per token quantizes every token on its own, so the cache after a chunk's write holds the same
    codes for a prefix as a cache of that prefix alone: the query at position p equals the decode over the
    first p + 1 tokens (the last query the decode over all T); and a query at position 0 reads exactly the
    dequantized, inverse-rotated first value, whatever its logit."""
    r = np.random.default_rng(67)
    T = 300
    k = r.standard_normal((T, 128)).astype(np.float32)
    v = r.standard_normal((T, 128)).astype(np.float32)
    q = r.standard_normal((5, 4, 128)).astype(np.float32)
    sk = np.where(r.random(128) < 0.5, -1.0, 1.0).astype(np.float32)
    sv = np.where(r.random(128) < 0.5, -1.0, 1.0).astype(np.float32)
    pos = np.array([0, 63, 64, 200, T - 1])
    for block, svv in ((128, sv), (32, sv), (128, None)):
        got = O.prefill_int4(q, pos, k, v, T, sk, svv, block)
        for i, p in enumerate(pos):
            want, _ = O.decode_int4(q[i], k, v, int(p) + 1, sk, svv, block)
            assert np.abs(got[i] - want).max() < 1e-12
        # position 0: the first value back in its own frame, within the rounding of one 15-step code per
        # rotated channel (the inverse rotation is orthonormal) and of the bf16 source
        st = O.int4_state(k, v, 1, sk, svv, block=block)
        step = float(O.bf16_value(st["v_s16"][:1])[0])
        bound = 0.5 * step * np.sqrt(128) * 1.01 + 2.0 ** -8 * np.linalg.norm(v[0])
        err = np.linalg.norm(got[0] - v[0].astype(np.float64)[None, :], axis=1).max()  # L2 over channels
        assert err <= bound, (block, err, bound)


def test_int4_channel_quantizer_closed_forms():
    """Per-channel INT4 (15 levels): channels built as a + s n, n in {0..15} and s a power of two, give codes
    n and dequantize exactly; the 3-level instance is the pinned INT2 quantizer."""
    r = np.random.default_rng(71)
    n = r.integers(0, 16, size=(128, 128))
    n[0, :], n[1, :] = 0, 15
    a = -r.integers(1, 9, size=(1, 128)).astype(np.float32)
    s = (2.0 ** r.integers(-3, 2, size=(1, 128))).astype(np.float32)
    x = (a + s * n).astype(np.float32)
    q, s16, z16 = O.quantize_int2_channel_group(x, 15)
    assert np.array_equal(q, n)
    assert np.array_equal(O.dequantize(q, s16[None, :], z16[None, :]), x.astype(np.float64))
    y = r.standard_normal((128, 128)).astype(np.float32)
    for got, want in zip(O.quantize_int2_channel_group(y, 3), O.quantize_int2_channel_group(y)):
        assert np.array_equal(got, want)
    # the reconstruction error of 4 bits is within half a step of the 15-level grid
    q, s16, z16 = O.quantize_int2_channel_group(y, 15)
    err = np.abs(O.dequantize(q, s16[None, :], z16[None, :]) - y)
    step = O.bf16_value(s16).astype(np.float64)
    assert np.all(err <= step[None, :] * 0.5 * (1 + 1e-2) + 1e-6)
