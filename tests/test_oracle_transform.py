"""Pins for the oracle's query-aware key transform (NOVA-KV summary,
Methodology, Key Transform Derivation: Theorem 1 and Proposition 1).

The oracle builds the transform from an eigendecomposition; these checks tie
it to other routes to the same numbers: the score error measured straight
from the queries and keys (eq. 5's left side), a brute-force search over every
rank-1 reconstruction map in two dimensions, numpy's SVD where the query
moment is the identity (the transform is then plain PCA), the generalized
Parseval relation on random coefficient vectors, and softmax's invariance to a
per-query shift.  The last tests plant plausible mistakes in copies of the
construction and show that some pin catches each one.
"""
import math

import numpy as np
import pytest

from oracle import lrkv_oracle as O


def _data(seed, d=12, nq=150, nk=240, mean=0.7):
    """Anisotropic queries (a skewed, rotated second moment) and keys with a
    decaying spectrum and a non-zero mean."""
    rng = np.random.default_rng(seed)
    rot = np.linalg.qr(rng.standard_normal((d, d)))[0]
    Q = rng.standard_normal((nq, d)) @ np.diag(np.geomspace(0.2, 4.0, d)) @ rot
    K = rng.standard_normal((nk, d)) * (0.8 ** np.arange(d)) @ np.linalg.qr(rng.standard_normal((d, d)))[0]
    return Q, K + mean * rng.standard_normal(d)


def _score_error_by_loops(Q, K, K_hat):
    """sum over queries i and keys j of (q_i . k_j - q_i . k_hat_j)^2, term by term."""
    tot = 0.0
    for q in Q:
        for k, kh in zip(K, K_hat):
            tot += (float(q @ k) - float(q @ kh)) ** 2
    return tot


def test_score_error_equals_the_term_by_term_sum():
    """O.score_error (the yardstick of the optimality and brute-force pins
    below) equals the sum over queries and keys of the squared logit
    differences taken one term at a time, for reconstructions from the
    transform, from an unrelated map, and the empty reconstruction K_hat = 0."""
    rng = np.random.default_rng(8)
    for seed, (d, nq, nk) in enumerate([(5, 7, 9), (12, 20, 31), (3, 1, 1)]):
        Q, K = _data(100 + seed, d=d, nq=nq, nk=nk)
        p = max(1, d // 2)
        enc, dec, _ = O.query_aware_key_transform(Q, K, p) if nq >= d else (None, None, None)
        hats = [np.zeros_like(K), K @ rng.standard_normal((d, d)) / d, K + rng.standard_normal(K.shape)]
        if enc is not None:
            hats.append(K @ enc @ dec.T)
        for K_hat in hats:
            ref = _score_error_by_loops(Q, K, K_hat)
            assert abs(O.score_error(Q, K, K_hat) - ref) <= 1e-12 * max(1.0, ref)
    # a single query and key by hand: q = (1, 2), k = (3, -1), k_hat = (1, 1):
    # q.k = 1, q.k_hat = 3, error (1 - 3)^2 = 4
    assert O.score_error(np.array([[1.0, 2.0]]), np.array([[3.0, -1.0]]), np.array([[1.0, 1.0]])) == 4.0


def _centred(K):
    return K - K.mean(axis=0, keepdims=True)


def test_decoder_is_biorthogonal_to_encoder():
    """dec^T enc = I_p, so k -> (k enc) dec^T is a projection; at p = d it is the identity."""
    Q, K = _data(1)
    d = K.shape[1]
    for p in (1, 4, d):
        enc, dec, _ = O.query_aware_key_transform(Q, K, p)
        assert np.max(np.abs(dec.T @ enc - np.eye(p))) <= 1e-11
        P = enc @ dec.T
        assert np.max(np.abs(P @ P - P)) <= 1e-10
    enc, dec, _ = O.query_aware_key_transform(Q, K, d)
    assert np.max(np.abs(enc @ dec.T - np.eye(d))) <= 1e-10
    # the transform is not orthogonal for anisotropic queries
    assert np.max(np.abs(enc - dec)) > 0.1


def test_generalized_parseval():
    """Proposition 1: with k = r R^-1 and k_hat = r_hat R^-1 (R the full transform),
    ||r - r_hat||^2 equals sum_i (q_i . (k - k_hat))^2, the score error over the queries."""
    Q, K = _data(2)
    d = K.shape[1]
    enc, dec, _ = O.query_aware_key_transform(Q, K, d)
    rng = np.random.default_rng(3)
    for _ in range(20):
        r, r_hat = rng.standard_normal(d), rng.standard_normal(d)
        k, k_hat = r @ dec.T, r_hat @ dec.T           # R^-1 = dec^T at p = d
        lhs = float(np.sum((r - r_hat) ** 2))
        rhs = float(np.sum((Q @ (k - k_hat)) ** 2))
        assert abs(lhs - rhs) <= 1e-10 * rhs
        assert np.max(np.abs(k @ enc - r)) <= 1e-10   # the transform recovers the coefficients


def test_truncation_error_is_the_eigenvalue_tail():
    """Keeping p coefficients of centred keys costs exactly the discarded
    eigenvalues in score error (eq. 5 with Theorem 1's transform), measured
    term by term from the queries and keys; the eigenvalues sum to the total
    score energy sum_ij (q_i . k_j)^2 of the centred keys."""
    Q, K = _data(4, d=8, nq=40, nk=60)
    Kc = _centred(K)
    d = K.shape[1]
    _, _, lam = O.query_aware_key_transform(Q, K, d)
    energy = _score_error_by_loops(Q, Kc, np.zeros_like(Kc))
    assert abs(lam.sum() - energy) <= 1e-10 * energy
    assert np.all(np.diff(lam) <= 1e-9 * lam[0])
    for p in range(d + 1):
        enc, dec, lam_p = O.query_aware_key_transform(Q, K, p)
        err = _score_error_by_loops(Q, Kc, Kc @ enc @ dec.T)
        assert abs(err - lam_p[p:].sum()) <= 1e-9 * energy, p


def test_transform_beats_pca_and_nearby_rank_p_maps():
    """Theorem 1's optimality: at every rank the score error is no larger than
    the orthogonal PCA basis's (top right singular vectors of the centred keys,
    numpy's SVD), strictly smaller somewhere, and no larger than that of
    random rank-p maps near the optimum."""
    Q, K = _data(5)
    Kc = _centred(K)
    d = K.shape[1]
    vt = np.linalg.svd(Kc, full_matrices=False)[2]
    strictly = False
    rng = np.random.default_rng(6)
    for p in (1, 3, 6, 9):
        enc, dec, _ = O.query_aware_key_transform(Q, K, p)
        best = O.score_error(Q, Kc, Kc @ enc @ dec.T)
        pca = vt[:p].T
        e_pca = O.score_error(Q, Kc, Kc @ pca @ pca.T)
        assert best <= e_pca * (1 + 1e-12)
        strictly |= best < 0.95 * e_pca
        for _ in range(200):
            A = enc + 0.05 * rng.standard_normal(enc.shape)
            B = dec + 0.05 * rng.standard_normal(dec.shape)
            assert best <= O.score_error(Q, Kc, Kc @ A @ B.T) * (1 + 1e-12)
    assert strictly


def test_brute_force_rank1_in_two_dimensions():
    """d = 2, p = 1: every rank-1 reconstruction is k -> (k . a) b.  For each
    unit direction a on a fine half-circle grid the best b is a linear least
    squares problem (numpy's lstsq) over all (query, key) pairs; the grid
    minimum agrees with the oracle's transform."""
    rng = np.random.default_rng(7)
    Q = rng.standard_normal((30, 2)) @ np.array([[2.0, 0.6], [0.0, 0.4]])
    K = rng.standard_normal((40, 2)) @ np.array([[1.0, 0.3], [0.2, 0.7]]) + np.array([0.5, -1.0])
    Kc = _centred(K)
    enc, dec, _ = O.query_aware_key_transform(Q, K, 1)
    opt = O.score_error(Q, Kc, Kc @ enc @ dec.T)
    target = (Q @ Kc.T).reshape(-1)                 # q_i . k_j, i major
    best = math.inf
    for t in np.linspace(0.0, math.pi, 4001):
        a = np.array([math.cos(t), math.sin(t)])
        proj = Kc @ a                               # k_j . a
        feats = (Q[:, None, :] * proj[None, :, None]).reshape(-1, 2)   # (k_j . a) q_i
        b, *_ = np.linalg.lstsq(feats, target, rcond=None)
        best = min(best, float(np.sum((feats @ b - target) ** 2)))
    assert opt <= best * (1 + 1e-9)
    assert best <= opt * (1 + 1e-5) + 1e-12


def test_identity_query_moment_is_pca():
    """With M_q = c I the weighting is uniform: the reconstruction is the
    orthogonal projection onto the top-p right singular vectors of the
    centred keys (numpy's SVD), and encoder and decoder are parallel."""
    rng = np.random.default_rng(8)
    d, p, c = 10, 4, 2.5
    Q = math.sqrt(c) * np.eye(d)                    # Q^T Q = c I
    K = rng.standard_normal((80, d)) * (0.7 ** np.arange(d)) + 0.2
    enc, dec, lam = O.query_aware_key_transform(Q, K, p)
    vt = np.linalg.svd(_centred(K), full_matrices=False)[2]
    assert np.max(np.abs(enc @ dec.T - vt[:p].T @ vt[:p])) <= 1e-10
    assert np.max(np.abs(enc - c * dec)) <= 1e-10
    sv = np.linalg.svd(_centred(K), compute_uv=False)
    assert np.max(np.abs(lam - c * sv ** 2)) <= 1e-9 * lam[0]


def test_psd_square_root():
    rng = np.random.default_rng(9)
    a = rng.standard_normal((9, 9))
    m = a @ a.T + 0.1 * np.eye(9)
    r, ri = O.psd_sqrt(m), O.psd_sqrt(m, inverse=True)
    assert np.max(np.abs(r @ r - m)) <= 1e-10 * np.abs(m).max()
    assert np.max(np.abs(r - r.T)) <= 1e-12 * np.abs(r).max()
    assert np.max(np.abs(ri @ m @ ri - np.eye(9))) <= 1e-9
    assert np.all(np.linalg.eigvalsh(r) > 0)
    with pytest.raises(ValueError):
        O.psd_sqrt(-np.eye(3))


def test_key_mean_shifts_every_score_of_a_query_equally():
    """Why the decode path needs no key mean: reconstructing mu + (k - mu) P
    instead of k P adds q . mu (I - P) to every score of query q.  Softmax
    ignores a per-query shift, so the output is unchanged and lse moves by
    that shift times the scale (checked on the oracle's textbook attention)."""
    Q, K = _data(10, d=8, nq=20, nk=50)
    enc, dec, _ = O.query_aware_key_transform(Q, K, 3)
    mu = K.mean(axis=0)
    P = enc @ dec.T
    V = np.random.default_rng(11).standard_normal((50, 8))
    scale = 1 / math.sqrt(8)
    for q in Q[:5]:
        o1, l1, _, _ = O.softmax_attention(q, K @ P, V, scale)
        o2, l2, _, _ = O.softmax_attention(q, mu + (K - mu) @ P, V, scale)
        assert np.max(np.abs(o1 - o2)) <= 1e-12 * np.max(np.abs(o1))
        shift = float(q @ (mu - mu @ P)) * scale
        assert abs((l2 - l1) - shift) <= 1e-10 * max(1.0, abs(shift))


# ----------------------------------------------------------------------------
# planted mistakes
# ----------------------------------------------------------------------------

def _mutant(kind):
    def transform(queries, keys, p):
        Q = np.asarray(queries, dtype=np.float64)
        K = np.asarray(keys, dtype=np.float64)
        m = Q.T @ Q
        root, root_inv = O.psd_sqrt(m), O.psd_sqrt(m, inverse=True)
        if kind == "moment_not_root":
            root, root_inv = m, np.linalg.inv(m)
        kc = K if kind == "uncentred_scatter" else K - K.mean(axis=0, keepdims=True)
        a = root @ (kc.T @ kc) @ root
        lam, e = np.linalg.eigh(a)
        order = np.argsort(lam) if kind == "smallest_first" else np.argsort(lam)[::-1]
        lam, e = lam[order], e[:, order]
        if kind == "transposed_frame":
            e = e.T
        enc = root @ e[:, :p]
        dec = enc if kind == "decoder_is_encoder" else root_inv @ e[:, :p]
        return enc, dec, lam
    return transform


PINS = [test_decoder_is_biorthogonal_to_encoder, test_generalized_parseval,
        test_truncation_error_is_the_eigenvalue_tail, test_transform_beats_pca_and_nearby_rank_p_maps,
        test_brute_force_rank1_in_two_dimensions, test_identity_query_moment_is_pca]


def _some_pin_fails():
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            return True
    return False


def test_unmutated_transform_passes_pins():
    assert not _some_pin_fails()


@pytest.mark.parametrize("kind", ["moment_not_root", "uncentred_scatter", "smallest_first",
                                  "transposed_frame", "decoder_is_encoder"])
def test_planted_transform_mistake_is_caught(monkeypatch, kind):
    monkeypatch.setattr(O, "query_aware_key_transform", _mutant(kind))
    assert _some_pin_fails()
