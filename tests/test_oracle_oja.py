"""Pins for the oracle's Oja subspace update ("OjaKV" README, Method Summary,
OjaKV: the low-rank subspace is updated online with Oja's algorithm).

Each pin is a property the rule has by its mathematics, checked against
something other than the oracle's own formula: an exact algebraic identity,
a fixed point, the per-token (sequential) rule to second order in the step,
the principal subspace from numpy's eigendecomposition, and Oja's
single-neuron rule.
"""
import numpy as np
import pytest

from oracle import lrkv_oracle as O


def _orthonormal(rng, d, r):
    q, rr = np.linalg.qr(rng.standard_normal((d, r)))
    return q * np.sign(np.diag(rr))[None, :]


def _sequential(basis, x, eta):
    """The per-token rule, one token after another: y = x B, B <- B + eta (x - y B^T)^T y."""
    B = np.array(basis, dtype=np.float64)
    for t in range(x.shape[0]):
        xt = x[t:t + 1]
        y = xt @ B
        B = B + eta * (xt - y @ B.T).T @ y
    return B


def test_orthonormality_is_kept_to_first_order_exactly():
    # for B^T B = I: B^T dB = B^T X^T Y - B^T B Y^T Y = Y^T Y - Y^T Y = 0, so
    # (B + dB)^T (B + dB) - I is exactly dB^T dB
    rng = np.random.default_rng(1)
    for d, r, n, eta in ((16, 4, 50, 1e-3), (128, 64, 300, 1e-4), (64, 1, 20, 0.05)):
        B = _orthonormal(rng, d, r)
        X = rng.standard_normal((n, d))
        Bn = O.oja_update(B, X, eta)
        dB = Bn - B
        assert np.abs(B.T @ dB).max() < 1e-12 * max(1.0, np.abs(dB).max())
        assert np.abs(Bn.T @ Bn - np.eye(r) - dB.T @ dB).max() < 1e-12
        assert np.abs(dB).max() > 0


def test_tokens_inside_the_span_leave_the_basis_unchanged():
    rng = np.random.default_rng(2)
    B = _orthonormal(rng, 32, 6)
    X = rng.standard_normal((40, 6)) @ B.T          # every residual is zero
    np.testing.assert_allclose(O.oja_update(B, X, 0.3), B, atol=1e-13)


def test_batched_step_matches_the_per_token_rule_to_second_order():
    rng = np.random.default_rng(3)
    B = _orthonormal(rng, 24, 5)
    X = rng.standard_normal((30, 24))
    gaps = []
    for eta in (1e-3, 5e-4, 2.5e-4, 1.25e-4):
        batched = O.oja_update(B, X, eta)
        seq = _sequential(B, X, eta)
        gaps.append(np.abs(batched - seq).max())
        # both moved by O(eta); they differ by O(eta^2)
        assert np.abs(batched - B).max() > 20 * gaps[-1]
    ratios = [gaps[i] / gaps[i + 1] for i in range(len(gaps) - 1)]
    assert all(3.6 < q < 4.4 for q in ratios), ratios


def test_repeated_steps_converge_to_the_principal_subspace():
    # tokens with a planted covariance U diag(lam) U^T: repeated steps take a
    # random orthonormal basis onto the span of the top-r eigenvectors that
    # numpy finds for the tokens' second moment
    rng = np.random.default_rng(4)
    d, r = 16, 3
    U = _orthonormal(rng, d, d)
    lam = np.array([9.0, 7.0, 5.0] + [1.0] * (d - 3))
    X = (rng.standard_normal((4000, d)) * np.sqrt(lam)[None, :]) @ U.T
    B = _orthonormal(rng, d, r)
    eta = 2e-4
    for it in range(300):
        batch = X[(it * 200) % 4000:(it * 200) % 4000 + 200]
        B = O.oja_update(B, batch, eta)
    mu, V = np.linalg.eigh(X.T @ X)
    top = V[:, np.argsort(mu)[::-1][:r]]
    # sine of the largest principal angle between span(B) and span(top)
    Qb = np.linalg.qr(B)[0]
    s = np.linalg.svd(top.T @ Qb, compute_uv=False)
    assert np.sqrt(max(0.0, 1.0 - s.min() ** 2)) < 0.05
    assert np.abs(B.T @ B - np.eye(r)).max() < 0.02


def test_single_component_is_ojas_neuron_rule():
    # r = 1, one token: w <- w + eta y (x - y w), y = x . w (Oja's original rule)
    rng = np.random.default_rng(5)
    w = rng.standard_normal(10)
    w /= np.linalg.norm(w)
    x = rng.standard_normal(10)
    y = float(x @ w)
    expected = w + 0.07 * y * (x - y * w)
    np.testing.assert_allclose(O.oja_update(w[:, None], x[None, :], 0.07)[:, 0], expected, rtol=1e-13)


def test_heads_are_independent_and_batch_order_does_not_matter():
    rng = np.random.default_rng(6)
    Bs = np.stack([_orthonormal(rng, 16, 4) for _ in range(3)])
    x = rng.standard_normal((2, 9, 3, 16))          # [B, T, Hkv, d]
    out = O.oja_update_heads(Bs, x, 0.01)
    x2 = x.copy()
    x2[:, :, 1] += 5.0                              # another head's tokens
    out2 = O.oja_update_heads(Bs, x2, 0.01)
    np.testing.assert_array_equal(out[0], out2[0])
    np.testing.assert_array_equal(out[2], out2[2])
    assert np.abs(out[1] - out2[1]).max() > 1e-3
    np.testing.assert_allclose(O.oja_update_heads(Bs, x[::-1], 0.01), out, atol=1e-14)
    # one call over both batch rows is one step over their concatenated tokens
    np.testing.assert_allclose(out[2], O.oja_update(Bs[2], np.concatenate([x[0, :, 2], x[1, :, 2]]), 0.01),
                               atol=1e-14)


def _mutants():
    def plus_decay(B, X, eta):
        Y = X @ B
        return B + eta * (X.T @ Y + B @ (Y.T @ Y))

    def no_decay(B, X, eta):
        Y = X @ B
        return B + eta * (X.T @ Y)

    def mean_step(B, X, eta):
        Y = X @ B
        return B + eta / X.shape[0] * (X.T @ Y - B @ (Y.T @ Y))

    def away(B, X, eta):
        Y = X @ B
        return B - eta * (X.T @ Y - B @ (Y.T @ Y))

    def rounded_projection(B, X, eta):
        Y = O.round_bf16(X @ B)
        return B + eta * (X.T @ Y - B @ (Y.T @ Y))

    return [plus_decay, no_decay, mean_step, away, rounded_projection]


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_planted_oja_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(O, "oja_update", mutant)
    checks = [test_orthonormality_is_kept_to_first_order_exactly,
              test_tokens_inside_the_span_leave_the_basis_unchanged,
              test_batched_step_matches_the_per_token_rule_to_second_order,
              test_repeated_steps_converge_to_the_principal_subspace,
              test_single_component_is_ojas_neuron_rule]
    failed = 0
    with np.errstate(all="ignore"):
        for check in checks:
            try:
                check()
            except (AssertionError, np.linalg.LinAlgError):
                failed += 1
    assert failed > 0, f"{mutant.__name__} passed every pin"


def test_old_rows_read_through_an_updated_basis_drift_in_proportion_to_the_step():
    """Rows compressed with the starting basis keep their coefficients after an
    update, so decoding them through the updated bases moves the output.  The
    move is first order in eta (doubling eta doubles it, to within the
    second-order term) and vanishes when the update's tokens lie in the span
    (the fixed point): the size of the drift that leaving old rows as stored
    causes."""
    rng = np.random.default_rng(31)
    d, rk, rv, n, T = 16, 6, 8, 40, 12
    bk0 = _orthonormal(rng, d, rk)[None]
    bv0 = _orthonormal(rng, d, rv)[None]
    ck = rng.standard_normal((1, 1, n, rk))
    cv = rng.standard_normal((1, 1, n, rv))
    q = rng.standard_normal((1, 2, d))
    xk = rng.standard_normal((1, T, 1, d))
    xv = rng.standard_normal((1, T, 1, d))
    o0, _ = O.decode(q, bk0, ck, bv0, cv, n)

    def drift(eta, xk=xk, xv=xv):
        o1, _ = O.decode(q, O.oja_update_heads(bk0, xk, eta), ck, O.oja_update_heads(bv0, xv, eta), cv, n)
        return np.abs(o1 - o0).max()

    d1, d2, d4 = drift(1e-5), drift(2e-5), drift(4e-5)
    assert d1 > 0
    assert abs(d2 / d1 - 2) < 0.01 and abs(d4 / d2 - 2) < 0.01
    # tokens inside the span leave the bases, and so the output, unchanged
    in_k = (rng.standard_normal((1, T, 1, rk)) @ bk0[0].T)
    in_v = (rng.standard_normal((1, T, 1, rv)) @ bv0[0].T)
    assert drift(1e-2, in_k, in_v) < 1e-12
