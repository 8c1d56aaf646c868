"""Rotation from a calibration covariance ([OSCAR] summary page §3.2 offline steps 2-3, §3.4.2 Factor 1
and Lemma 1): the oracle pinned to closed forms and to the factor-order property the page proves, then
the library's host builders (covariances, Jacobi eigensolver, R = U.H.P_br) against the oracle.  CPU only.
"""
import numpy as np
import pytest

import oracle as O
import synth

D = 128


def _spd(seed, decay=0.5):
    """A generic symmetric positive definite matrix with a decaying, well-separated spectrum."""
    r = np.random.default_rng(seed)
    Q, _ = np.linalg.qr(r.standard_normal((D, D)))
    lam = (np.arange(D) + 1.0) ** -decay * (1.0 + 0.01 * r.random(D))
    return (Q * lam[None, :]) @ Q.T, Q, lam


# ---------------------------------------------------------------- oracle pins


def test_eigenbasis_of_a_permuted_diagonal_is_the_permuted_identity():
    r = np.random.default_rng(3)
    lam = r.permutation(np.arange(1.0, D + 1.0))
    U, got = O.eigenbasis(np.diag(lam))
    assert np.array_equal(got, np.sort(lam)[::-1])
    # column k is +e_i where lam[i] is the k-th largest
    want = np.zeros((D, D))
    want[np.argsort(-lam), np.arange(D)] = 1.0
    assert np.abs(U - want).max() < 1e-12


def test_eigenbasis_of_a_hadamard_spectrum():
    """C = H diag(lam) H^T: eigenvectors are the Hadamard columns (up to sign), eigenvalues as given."""
    H = O.hadamard()
    lam = np.linspace(5.0, 0.1, D)
    U, got = O.eigenbasis(H @ np.diag(lam) @ H.T)
    assert np.abs(got - lam).max() < 1e-12
    for k in range(D):
        assert min(np.abs(U[:, k] - H[:, k]).max(), np.abs(U[:, k] + H[:, k]).max()) < 1e-10
        assert U[np.argmax(np.abs(U[:, k])), k] > 0


def test_eigenbasis_diagonalizes_and_sorts():
    C, _, lam_true = _spd(11)
    U, lam = O.eigenbasis(C)
    assert np.abs(U.T @ U - np.eye(D)).max() < 1e-12
    Lam = U.T @ C @ U
    assert np.abs(Lam - np.diag(np.diag(Lam))).max() < 1e-12
    assert np.all(np.diff(lam) <= 0)
    assert np.abs(lam - np.sort(lam_true)[::-1]).max() < 1e-12


def test_rotation_from_covariance_equalizes_the_importance_diagonal():
    """Lemma 1 through the factor order U first, H second: diag(R^T C R) = tr(C)/d for every channel, while
    the Hadamard alone (no eigenbasis) leaves it uneven on the same C."""
    for seed in (1, 2, 3):
        C, _, _ = _spd(seed)
        R = O.oscar_rotation_from_covariance(C)
        assert np.abs(R.T @ R - np.eye(D)).max() < 1e-12
        diag = np.diag(R.T @ C @ R)
        assert np.abs(diag - np.trace(C) / D).max() < 1e-12 * np.trace(C)
        Rh = O.hadamard() @ O.bit_reversal_matrix()
        dh = np.diag(Rh.T @ C @ Rh)
        assert dh.max() / dh.mean() > 1.05


def test_rotation_from_covariance_places_the_kth_eigenvector_at_beta_k():
    """Before the Hadamard mixing, P_br puts the eigenvector of the k-th largest eigenvalue at column
    beta(k) (top-1 -> 0, top-2 -> 64, top-3 -> 32, top-4 -> 96 as the page lists)."""
    C, _, _ = _spd(5)
    U, _ = O.eigenbasis(C)
    UP = U @ O.bit_reversal_matrix()
    beta = O.bit_reversal()
    for k in range(D):
        assert np.array_equal(UP[:, beta[k]], U[:, k])
    assert [int(beta[k]) for k in range(4)] == [0, 64, 32, 96]


def test_covariances_closed_forms():
    q = np.zeros((4, D), dtype=np.float32)
    q[0, 3], q[1, 3], q[2, 7], q[3, 9] = 2.0, -2.0, 3.0, 1.0
    C = O.query_covariance(q)
    want = np.zeros((D, D))
    want[3, 3], want[7, 7], want[9, 9] = 8.0 / 4, 9.0 / 4, 1.0 / 4
    assert np.array_equal(C, want)
    r = np.random.default_rng(0)
    v = r.standard_normal((6, D)).astype(np.float32)
    # identity scores: C_S = V^T V / N
    assert np.abs(O.score_value_covariance(v, np.eye(6)) - v.astype(np.float64).T @ v / 6).max() < 1e-12
    # uniform scores: every row of S V is the mean value m, so C_S = m m^T
    m = v.astype(np.float64).mean(axis=0)
    assert np.abs(O.score_value_covariance(v, np.full((3, 6), 1.0 / 6)) - np.outer(m, m)).max() < 1e-12


# ---------------------------------------------------------------- library (host) against the oracle


@pytest.fixture(scope="module")
def K():
    import decode_attention_15_amd as K
    return K


def test_library_covariances_match_the_oracle(K):
    q, v, s = synth.calibration_activations(2000, seed=1)
    Cq = K.query_covariance(q)
    Cq_o = O.query_covariance(q)
    assert np.abs(Cq - Cq_o).max() <= 1e-12 * np.abs(Cq_o).max()
    assert np.array_equal(Cq, Cq.T)
    Cs = K.score_value_covariance(v, s)
    Cs_o = O.score_value_covariance(v, s)
    assert np.abs(Cs - Cs_o).max() <= 1e-12 * np.abs(Cs_o).max()


def test_library_eigenbasis_matches_the_oracle(K):
    for seed in (7, 8):
        C, _, _ = _spd(seed)
        U, lam = K.eigenbasis(C)
        Uo, lamo = O.eigenbasis(C)
        assert np.abs(lam - lamo).max() <= 1e-12 * lamo[0]
        assert np.abs(U - Uo).max() < 1e-9
        assert np.abs(U.T @ U - np.eye(D)).max() < 1e-12
        assert np.abs(C @ U - U * lam[None, :]).max() < 1e-12 * lamo[0]


def test_library_rotation_from_calibration_data(K):
    """End to end on seeded calibration activations: C_Q and C_S, their eigenbases and the two rotations,
    against the oracle; the library's rotations satisfy the Lemma 1 property on their own covariance."""
    q, v, s = synth.calibration_activations(4000, seed=2)
    for C_lib, C_or in ((K.query_covariance(q), O.query_covariance(q)),
                        (K.score_value_covariance(v, s), O.score_value_covariance(v, s))):
        R = K.build_oscar_rotation_from_covariance(C_lib)
        Ro = O.oscar_rotation_from_covariance(C_or)
        assert np.abs(R - Ro).max() < 1e-8
        assert np.abs(R.T @ R - np.eye(D)).max() < 1e-12
        diag = np.diag(R.T @ C_lib @ R)
        assert np.abs(diag - np.trace(C_lib) / D).max() < 1e-10 * np.trace(C_lib)
        assert np.array_equal(R, K.compose_oscar_rotation(K.eigenbasis(C_lib)[0]))


def test_library_eigenbasis_of_repeated_eigenvalues(K):
    """Identity and a two-level spectrum: the basis is not unique, its invariants are."""
    U, lam = K.eigenbasis(np.eye(D))
    assert np.array_equal(lam, np.ones(D)) and np.array_equal(U, np.eye(D))
    C, Q, _ = _spd(9)
    lam2 = np.where(np.arange(D) < 40, 3.0, 1.0)
    C2 = (Q * lam2[None, :]) @ Q.T
    U, lam = K.eigenbasis(C2)
    assert np.abs(lam - np.sort(lam2)[::-1]).max() < 1e-12
    assert np.abs(U.T @ U - np.eye(D)).max() < 1e-12
    assert np.abs(C2 @ U - U * lam[None, :]).max() < 1e-12
    R = K.build_oscar_rotation_from_covariance(C2)
    assert np.abs(np.diag(R.T @ C2 @ R) - np.trace(C2) / D).max() < 1e-12 * np.trace(C2)


def test_library_calibration_errors(K):
    C, _, _ = _spd(4)
    bad = C.copy()
    bad[0, 1] += 1e-6
    with pytest.raises(K.KvqError):
        K.eigenbasis(bad)
    nan = C.copy()
    nan[5, 5] = np.nan
    with pytest.raises(K.KvqError):
        K.build_oscar_rotation_from_covariance(nan)
    with pytest.raises(K.KvqError):
        K.query_covariance(np.zeros((0, D), dtype=np.float32))
    with pytest.raises(K.KvqError):
        K.query_covariance(np.full((2, D), np.inf, dtype=np.float32))
