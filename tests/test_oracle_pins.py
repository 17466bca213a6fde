"""Pins that tie the CPU oracle to something other than itself.

Each check compares the oracle with an independent route to the same number:
a library routine (torch's scaled_dot_product_attention, numpy's SVD), a
closed form, a brute-force search, or an invariant of the mathematics.  The
mutation tests at the end plant plausible mistakes in copies of the oracle and
show that some pin catches each one.
"""
import math

import numpy as np
import pytest
import torch

import lrkv_synth as synth
from oracle import lrkv_oracle as O


def _rand_orthonormal(rng, d, r):
    q, rr = np.linalg.qr(rng.standard_normal((d, d)))
    q = q * np.sign(np.diag(rr))[None, :]
    return q[:, :r]


def _sdpa(q, K, V, scale=None):
    """Dense GQA attention from torch (float64, CPU).

    q [B, Hq, d]; K, V [B, Hkv, N, d].  torch repeats kv head h for query
    heads h*g .. h*g+g-1 and scales by 1/sqrt(q.shape[-1]) by default.
    """
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))[:, :, None, :]
    Kt = torch.from_numpy(np.asarray(K, dtype=np.float64))
    Vt = torch.from_numpy(np.asarray(V, dtype=np.float64))
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale, enable_gqa=True)
    return o[:, :, 0, :].numpy()


def _sdpa_lse(q, K, group, scale):
    """log-sum-exp of the dense scores via torch.logsumexp."""
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))
    Kt = torch.from_numpy(np.asarray(K, dtype=np.float64)).repeat_interleave(group, dim=1)
    s = torch.einsum("bhd,bhnd->bhn", qt, Kt) * scale
    return torch.logsumexp(s, dim=-1).numpy()


def _case(seed, B=2, Hq=8, Hkv=2, d=16, rk=6, rv=10, N=37, orthonormal=True):
    rng = np.random.default_rng(seed)
    if orthonormal:
        bk = np.stack([_rand_orthonormal(rng, d, rk) for _ in range(Hkv)])
        bv = np.stack([_rand_orthonormal(rng, d, rv) for _ in range(Hkv)])
    else:
        bk = rng.standard_normal((Hkv, d, rk))
        bv = rng.standard_normal((Hkv, d, rv))
    ck = rng.standard_normal((B, Hkv, N, rk))
    cv = rng.standard_normal((B, Hkv, N, rv))
    q = rng.standard_normal((B, Hq, d))
    return q, bk, ck, bv, cv


# ----------------------------------------------------------------------------
# I1: latent-space attention equals reconstructed-space attention
# ----------------------------------------------------------------------------

def _latent_decode(q, bk, ck, bv, cv, n, scale):
    """Attention computed entirely in the latent space (associativity route)."""
    B, Hq, d = q.shape
    Hkv = bk.shape[0]
    g = Hq // Hkv
    o = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    for b in range(B):
        for hq in range(Hq):
            h = hq // g
            qp = (q[b, hq] @ bk[h]) * scale           # fold the query into the key latent space
            s = ck[b, h, :n] @ qp                      # latent scores
            m = s.max()
            w = np.exp(s - m)
            acc = (w @ cv[b, h, :n]) / w.sum()         # latent accumulation
            o[b, hq] = bv[h] @ acc                     # lift through B_V^T
            lse[b, hq] = m + math.log(w.sum())
    return o, lse


@pytest.mark.parametrize("orthonormal", [True, False])
def test_latent_equals_reconstructed(orthonormal):
    q, bk, ck, bv, cv = _case(1, orthonormal=orthonormal)
    n = 33
    scale = 1 / math.sqrt(q.shape[-1])
    o, lse = O.decode(q, bk, ck, bv, cv, n)
    o2, lse2 = _latent_decode(q, bk, ck, bv, cv, n, scale)
    assert np.max(np.abs(o - o2)) <= 1e-12 * max(1.0, np.max(np.abs(o)))
    assert np.max(np.abs(lse - lse2)) <= 1e-12 * max(1.0, np.max(np.abs(lse)))


# ----------------------------------------------------------------------------
# I2: identity (and coordinate) bases reduce to dense attention
# ----------------------------------------------------------------------------

def test_identity_basis_is_dense_attention():
    rng = np.random.default_rng(2)
    B, Hq, Hkv, d, N = 2, 8, 2, 16, 29
    K = rng.standard_normal((B, Hkv, N, d))
    V = rng.standard_normal((B, Hkv, N, d))
    q = rng.standard_normal((B, Hq, d))
    eye = np.stack([np.eye(d)] * Hkv)
    o, lse = O.decode(q, eye, K, eye, V, N)
    ref = _sdpa(q, K, V)
    assert np.max(np.abs(o - ref)) <= 1e-13 * max(1, np.abs(ref).max())
    ref_lse = _sdpa_lse(q, K, Hq // Hkv, 1 / math.sqrt(d))
    assert np.max(np.abs(lse - ref_lse)) <= 1e-12


def test_coordinate_basis_scale_is_head_dim():
    """B = first r columns of I: K_hat is C zero-padded to d; scale stays 1/sqrt(d)."""
    rng = np.random.default_rng(3)
    B, Hq, Hkv, d, r, N = 1, 4, 1, 32, 8, 20
    ck = rng.standard_normal((B, Hkv, N, r)) * 3
    cv = rng.standard_normal((B, Hkv, N, r))
    q = rng.standard_normal((B, Hq, d))
    basis = np.stack([np.eye(d)[:, :r]] * Hkv)
    o, _ = O.decode(q, basis, ck, basis, cv, N)
    K = np.zeros((B, Hkv, N, d)); K[..., :r] = ck
    V = np.zeros((B, Hkv, N, d)); V[..., :r] = cv
    ref = _sdpa(q, K, V)
    assert np.max(np.abs(o - ref)) <= 1e-13 * max(1, np.abs(ref).max())


def test_square_rotation_basis_round_trips_keys():
    """r = d, B a random rotation, C = K B exactly: K_hat = K, so dense attention on K."""
    rng = np.random.default_rng(4)
    B, Hq, Hkv, d, N = 1, 6, 3, 12, 17
    K = rng.standard_normal((B, N, Hkv, d))
    V = rng.standard_normal((B, N, Hkv, d))
    bk = np.stack([_rand_orthonormal(rng, d, d) for _ in range(Hkv)])
    bv = np.stack([_rand_orthonormal(rng, d, d) for _ in range(Hkv)])
    ck = O.compress(K, bk)
    cv = O.compress(V, bv)
    q = rng.standard_normal((B, Hq, d))
    o, _ = O.decode(q, bk, ck, bv, cv, N)
    ref = _sdpa(q, K.transpose(0, 2, 1, 3), V.transpose(0, 2, 1, 3))
    assert np.max(np.abs(o - ref)) <= 1e-12


# ----------------------------------------------------------------------------
# I3: the SVD basis is Frobenius-optimal (KV-CoRE: optimal low-rank approximation)
# ----------------------------------------------------------------------------

def _recon_error(x, basis):
    c = O.compress(x[None, :, None, :], basis[None])[0, 0]
    return np.sum((x - O.reconstruct(c, basis)) ** 2)


def test_svd_basis_is_frobenius_optimal():
    rng = np.random.default_rng(5)
    T, d, r = 200, 10, 3
    x = rng.standard_normal((T, d)) * (0.7 ** np.arange(d))[None, :] @ _rand_orthonormal(rng, d, d).T
    _, sv, vt = np.linalg.svd(x, full_matrices=False)
    b_svd = vt[:r].T
    err = _recon_error(x, b_svd)
    assert abs(err - np.sum(sv[r:] ** 2)) <= 1e-10 * np.sum(sv ** 2)
    for _ in range(2000):
        assert _recon_error(x, _rand_orthonormal(rng, d, r)) >= err * (1 - 1e-12)
    # small rotations of the optimum do not improve it
    for eps in (1e-3, 1e-2, 1e-1):
        a = rng.standard_normal((d, d)) * eps
        rot, _ = np.linalg.qr(np.eye(d) + (a - a.T))
        assert _recon_error(x, rot @ b_svd) >= err * (1 - 1e-12)


def test_brute_force_rank1_in_3d():
    """d = 3, r = 1: a hemisphere grid of unit vectors never beats the SVD residual."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((50, 3)) * np.array([2.0, 1.0, 0.3])
    sv = np.linalg.svd(x, compute_uv=False)
    best = math.inf
    for th in np.linspace(0, math.pi / 2, 91):
        for ph in np.linspace(0, 2 * math.pi, 361):
            u = np.array([[math.sin(th) * math.cos(ph)], [math.sin(th) * math.sin(ph)], [math.cos(th)]])
            best = min(best, _recon_error(x, u))
    assert best >= sv[1] ** 2 + sv[2] ** 2 - 1e-9
    assert best <= (sv[1] ** 2 + sv[2] ** 2) * 1.01


# ----------------------------------------------------------------------------
# I4/I5: the NOVA-KV summary's softmax and output-error bounds
# ----------------------------------------------------------------------------

def test_softmax_half_lipschitz_and_output_bound():
    rng = np.random.default_rng(7)
    d, r, N = 32, 8, 300
    fr = _rand_orthonormal(rng, d, d)
    spec = 0.8 ** np.arange(d)
    K = (rng.standard_normal((N, d)) * spec) @ fr.T
    V = (rng.standard_normal((N, d)) * spec) @ fr.T
    b = fr[:, :r]
    Kh = O.reconstruct(K @ b, b)
    Vh = O.reconstruct(V @ b, b)
    for _ in range(20):
        q = rng.standard_normal(d) * 3
        o, _, p, s = O.softmax_attention(q, K, V, 1 / math.sqrt(d))
        oh, _, ph, sh = O.softmax_attention(q, Kh, Vh, 1 / math.sqrt(d))
        assert np.linalg.norm(p - ph) <= 0.5 * np.linalg.norm(s - sh) + 1e-15
        bound = np.linalg.norm(p - ph) * np.linalg.norm(V, 2) + np.linalg.norm(ph @ (V - Vh))
        assert np.linalg.norm(o - oh) <= bound + 1e-12


# ----------------------------------------------------------------------------
# I6: special cases of the softmax definition
# ----------------------------------------------------------------------------

def test_special_cases():
    q, bk, ck, bv, cv = _case(8)
    d = q.shape[-1]
    g = q.shape[1] // bk.shape[0]
    sc = 1 / math.sqrt(d)
    # one token: o = v_hat_0, lse = s_0
    o, lse = O.decode(q, bk, ck, bv, cv, 1)
    for b in range(q.shape[0]):
        for hq in range(q.shape[1]):
            h = hq // g
            assert np.allclose(o[b, hq], cv[b, h, 0] @ bv[h].T, atol=1e-13)
            assert abs(lse[b, hq] - (ck[b, h, 0] @ bk[h].T) @ q[b, hq] * sc) <= 1e-12
    # zero query: uniform weights
    n = 21
    o, lse = O.decode(np.zeros_like(q), bk, ck, bv, cv, n)
    for b in range(q.shape[0]):
        for hq in range(q.shape[1]):
            h = hq // g
            assert np.allclose(o[b, hq], (cv[b, h, :n] @ bv[h].T).mean(0), atol=1e-13)
            assert abs(lse[b, hq] - math.log(n)) <= 1e-13
    # token permutation does not change anything
    perm = np.random.default_rng(0).permutation(n)
    o1, l1 = O.decode(q, bk, ck[:, :, :n], bv, cv[:, :, :n], n)
    o2, l2 = O.decode(q, bk, ck[:, :, perm], bv, cv[:, :, perm], n)
    assert np.max(np.abs(o1 - o2)) <= 1e-13 and np.max(np.abs(l1 - l2)) <= 1e-12
    # every token twice: same output, lse + ln 2
    o3, l3 = O.decode(q, bk, np.concatenate([ck[:, :, :n]] * 2, 2), bv,
                      np.concatenate([cv[:, :, :n]] * 2, 2), 2 * n)
    assert np.max(np.abs(o1 - o3)) <= 1e-13 and np.max(np.abs(l3 - l1 - math.log(2))) <= 1e-12


def test_least_squares_normal_equations():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((40, 3, 24))[None]
    basis = np.stack([_rand_orthonormal(rng, 24, 7) for _ in range(3)])
    c = O.compress(x, basis)
    for h in range(3):
        resid = x[0, :, h].T - basis[h] @ c[0, h].T
        assert np.max(np.abs(basis[h].T @ resid)) <= 1e-12


# ----------------------------------------------------------------------------
# storage rounding against torch's bfloat16 conversion
# ----------------------------------------------------------------------------

def test_round_storage_f32_matches_the_c_conversion():
    """round_storage(x, "f32") against Python's struct packing, which converts
    a double to an IEEE single through the C cast (round to nearest even):
    random values over a wide exponent range, and doubles exactly halfway
    between float32 neighbours (both parities of the lower neighbour)."""
    import struct
    rng = np.random.default_rng(12)
    x = rng.standard_normal(3000) * np.exp(rng.uniform(-30, 30, 3000))
    lo = rng.standard_normal(500).astype(np.float32)
    hi = np.nextafter(lo, np.float32(np.inf), dtype=np.float32)
    mid = (lo.astype(np.float64) + hi.astype(np.float64)) / 2.0     # exact in float64
    vals = np.concatenate([x, mid, [0.0, -0.0, 1.0, -3.5, 2.0 ** -126, 3.0e38]])
    ref = np.array([struct.unpack("<f", struct.pack("<f", float(v)))[0] for v in vals])
    got = O.round_storage(vals, "f32")
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))
    # the halfway cases went to the neighbour with an even last bit
    bits = got[len(x):len(x) + len(mid)].astype(np.float32).view(np.uint32)
    assert np.all((bits & 1) == 0)


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(10)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    # exact halfway cases between bf16 neighbours, both parities
    base = rng.standard_normal(1000).astype(np.float32)
    u = base.view(np.uint32) & np.uint32(0xFFFF0000)
    ties = (u | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, np.float32([0.0, -0.0, 1.0, -3.5])])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(x.astype(np.float64)), ref)


# ----------------------------------------------------------------------------
# hybrid selection and hybrid decode
# ----------------------------------------------------------------------------

def test_hybrid_flags_closed_form():
    """x = c B^T + alpha w, w a unit vector orthogonal to B: e = alpha / sqrt(|c|^2 + alpha^2)."""
    rng = np.random.default_rng(11)
    d, r, T, tau = 64, 16, 400, 0.5
    fr = _rand_orthonormal(rng, d, d)
    b = fr[:, :r]
    c = rng.standard_normal((T, r))
    w = rng.standard_normal((T, d - r)) @ fr[:, r:].T
    w /= np.linalg.norm(w, axis=1, keepdims=True)
    target = rng.uniform(0, 0.99, T)
    target = target[np.abs(target - tau) > 0.05]
    c = c[: len(target)]
    w = w[: len(target)]
    nc = np.linalg.norm(c, axis=1)
    alpha = target * nc / np.sqrt(1 - target ** 2)
    x = c @ b.T + alpha[:, None] * w
    for dtype in ("f32", "bf16"):
        flags = O.hybrid_flags(x, b, tau, dtype)
        assert np.array_equal(flags, target > tau)
    assert np.allclose(O.relative_residual(x, b), target, atol=1e-12)
    # zero tokens are never selected, even at tau = 0
    z = np.zeros((3, d))
    assert not O.hybrid_flags(z, b, 0.0, "bf16").any()
    # tau = +inf selects nothing
    assert not O.hybrid_flags(x, b, math.inf, "bf16").any()


def test_hybrid_flags_use_the_stored_coefficients():
    """The residual is taken against the reconstruction from the coefficients
    the cache stores.  A token exactly in the span whose coefficient is not
    representable in the storage dtype has residual |c - round(c)| / |x|:
    here x = (1 + 2^-8) e_0 against B = e_0, stored in bfloat16 as 1 (the tie
    goes to even), so its relative residual is 2^-8 / (1 + 2^-8) ~ 0.0039 and
    it is selected at tau = 0.002, although x B B^T = x.  Stored in float32
    the coefficient is exact, and nothing is selected."""
    d = 4
    b = np.zeros((d, 1))
    b[0, 0] = 1.0
    x = np.zeros((2, d))
    x[0, 0] = 1.0 + 2.0 ** -8     # halfway between bfloat16 neighbours 1 and 1 + 2^-7
    x[1, 0] = 1.0                 # representable: residual 0
    assert np.array_equal(O.hybrid_flags(x, b, 0.002, "bf16"), [True, False])
    assert not O.hybrid_flags(x, b, 0.005, "bf16").any()
    assert not O.hybrid_flags(x, b, 0.002, "f32").any()
    assert np.allclose(O.relative_residual(x, b), 0.0)


def test_hybrid_compaction_order_golden():
    """Hand-written selection example (tests/golden/hybrid_compaction_small.txt)."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "hybrid_compaction_small.txt")
    spec = {}
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split("=")
            spec[k.strip()] = [int(t) for t in v.split()] if v.strip() else []
    d, r = 8, 2
    basis = np.zeros((1, d, r)); basis[0, 0, 0] = basis[0, 1, 1] = 1.0
    T = spec["n_tokens"][0]
    pos = spec["pos"][0]
    x = np.zeros((1, T, 1, d))
    x[0, :, 0, 0] = 1.0                                # in span: residual 0
    for t in spec["off_span_keys"]:
        x[0, t, 0, 5] = 4.0                            # residual 4/sqrt(17) > 0.5
    v = np.zeros_like(x)
    v[0, :, 0, 1] = 2.0
    for t in spec["off_span_values"]:
        v[0, t, 0, 7] = 0.5                            # residual 0.5/sqrt(4.25) < 0.5
    for t in spec["off_span_values_big"]:
        v[0, t, 0, 7] = 3.0                            # residual 3/sqrt(13) > 0.5
    res = O.compress_hybrid(x, v, basis, basis, 0.5, "bf16", pos=pos)
    assert list(np.nonzero(res["flags"][(0, 0)])[0]) == spec["expect_flagged"]
    assert list(res["side_idx"][(0, 0)]) == spec["expect_side_idx"]
    assert res["ck"][(0, 0)].shape[0] == spec["expect_n_lr"][0]
    assert np.array_equal(res["k_side"][(0, 0)], x[0, spec["expect_flagged"], 0])


def test_hybrid_tau_inf_is_plain_low_rank_and_tau0_is_dense():
    w = synth.scaled(synth.HYBRID_128K, n_ctx=(512,), n_kv_heads=2, n_q_heads=8)
    inj = synth.injected_set(w, 0, 0, 512)
    k = np.stack([synth.hybrid_tokens(w, 0, "k", 0, h, 512, inj).exact for h in range(2)], 1)[None]
    v = np.stack([synth.hybrid_tokens(w, 0, "v", 0, h, 512, inj).exact for h in range(2)], 1)[None]
    bk = synth.basis(w, 0, "k").exact
    bv = synth.basis(w, 0, "v").exact
    q = synth.query(w, 0).exact
    rows = [(0, hq) for hq in range(8)]
    # tau = inf: every token low rank -> plain low-rank decode
    res = O.compress_hybrid(k, v, bk, bv, math.inf, "bf16")
    ck = {key: O.round_bf16(c) for key, c in res["ck"].items()}
    cv = {key: O.round_bf16(c) for key, c in res["cv"].items()}
    hy = O.decode_hybrid_rows(q, bk, bv, ck, cv, res["k_side"], res["v_side"], rows)
    ckf = np.stack([ck[(0, h)] for h in range(2)])[None]
    cvf = np.stack([cv[(0, h)] for h in range(2)])[None]
    o, lse = O.decode(q, bk, ckf, bv, cvf, 512)
    for (b, hq), (oh, lh) in hy.items():
        assert np.max(np.abs(oh - o[b, hq])) <= 1e-13 and abs(lh - lse[b, hq]) <= 1e-12
    # tau = 0: every token with a nonzero residual is full rank -> dense attention on K, V
    res = O.compress_hybrid(k, v, bk, bv, 0.0, "bf16")
    assert all(f.all() for f in res["flags"].values())
    hy = O.decode_hybrid_rows(q, bk, bv, res["ck"], res["cv"], res["k_side"], res["v_side"], rows)
    ref = _sdpa(q, k[0].transpose(1, 0, 2)[None], v[0].transpose(1, 0, 2)[None])
    for (b, hq), (oh, _) in hy.items():
        assert np.max(np.abs(oh - ref[b, hq])) <= 1e-12


def test_hybrid_workload_margin_and_selection():
    """On the hybrid workload's data every token is far from the threshold and
    the selected set is exactly the injected set; the hybrid output is much
    closer to dense attention than the plain low-rank output."""
    n = 4096
    w = synth.scaled(synth.HYBRID_128K, n_ctx=(n,), n_kv_heads=2, n_q_heads=8)
    inj = synth.injected_set(w, 0, 0, n)
    assert len(inj) == round(0.05 * n)
    bk = synth.basis(w, 0, "k").exact
    bv = synth.basis(w, 0, "v").exact
    for h in range(2):
        for which, bb in (("k", bk), ("v", bv)):
            x = synth.hybrid_tokens(w, 0, which, 0, h, n, inj).exact
            e = O.relative_residual(x, bb[h])
            assert not np.any((e >= 0.25) & (e <= 0.75))
            flags = O.hybrid_flags(x, bb[h], 0.5, "bf16")
            assert np.array_equal(np.nonzero(flags)[0], inj)
            # The selection is defined in float64 on the stored coefficients;
            # a kernel may decide it in float32.  The two agree on every token
            # when err^2 / |x|^2 stays far from tau^2 compared with float32's
            # relative error on a d-term sum of squares (about d 2^-24 = 8e-6
            # at d = 128, plus the reconstruction's own float32 error, of the
            # same order relative to |x|^2): here the gap is at least 0.1.
            c = O.round_storage(x @ bb[h], "bf16")
            res = x - c @ bb[h].T
            e2 = np.sum(res * res, axis=1) / np.sum(x * x, axis=1)
            assert np.min(np.abs(e2 - 0.25)) >= 0.1


# ----------------------------------------------------------------------------
# mutation tests: plausible mistakes planted in the oracle must fail a pin
# ----------------------------------------------------------------------------

_DECODE_PINS = (test_identity_basis_is_dense_attention, test_coordinate_basis_scale_is_head_dim,
                test_square_rotation_basis_round_trips_keys, test_special_cases)


def _some_pin_fails(pins=_DECODE_PINS):
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError):   # a wrong value, or operands that no longer fit
            return True
    return False


def _mutant_decode(gqa=lambda hq, g, hkv: hq // g, scale_of=lambda d, r: 1 / math.sqrt(d)):
    """A copy of the oracle's decode with a replaceable GQA map and scale rule."""
    def decode(q, basis_k, coeff_k, basis_v, coeff_v, n_ctx, scale=None):
        B, Hq, d = q.shape
        Hkv = basis_k.shape[0]
        g = Hq // Hkv
        o = np.zeros((B, Hq, d))
        lse = np.zeros((B, Hq))
        for b in range(B):
            for hq in range(Hq):
                h = gqa(hq, g, Hkv)
                K = O.reconstruct(coeff_k[b, h, :n_ctx], basis_k[h])
                V = O.reconstruct(coeff_v[b, h, :n_ctx], basis_v[h])
                sc = scale_of(d, basis_k.shape[2]) if scale is None else scale
                o[b, hq], lse[b, hq], _, _ = O.softmax_attention(q[b, hq], K, V, sc)
        return o, lse
    return decode


def test_unmutated_oracle_passes_pins():
    assert not _some_pin_fails()


@pytest.mark.parametrize("mutant", ["transposed_basis", "dropped_last_token", "scale_one_over_d",
                                    "scale_from_rank", "gqa_modulo", "no_normalisation",
                                    "sign_flip", "lse_without_max"])
def test_planted_mistake_is_caught(monkeypatch, mutant):
    orig_sa = O.softmax_attention
    if mutant == "transposed_basis":
        monkeypatch.setattr(O, "reconstruct", lambda c, b: np.asarray(c) @ np.asarray(b)[: np.shape(c)[1]])
    elif mutant == "dropped_last_token":
        monkeypatch.setattr(O, "softmax_attention", lambda q, K, V, s: orig_sa(q, K[:-1], V[:-1], s)
                            if len(K) > 1 else orig_sa(q, K, V, s))
    elif mutant == "scale_one_over_d":
        monkeypatch.setattr(O, "default_scale", lambda d: 1.0 / d)
        monkeypatch.setattr(O, "decode", _mutant_decode(scale_of=lambda d, r: 1.0 / d))
    elif mutant == "scale_from_rank":
        monkeypatch.setattr(O, "decode", _mutant_decode(scale_of=lambda d, r: 1 / math.sqrt(r)))
    elif mutant == "gqa_modulo":
        monkeypatch.setattr(O, "decode", _mutant_decode(gqa=lambda hq, g, hkv: hq % hkv))
    else:
        def sa(q, K, V, scale):
            s = (np.asarray(K) @ q) * scale
            m = s.max()
            if mutant == "no_normalisation":
                w = np.exp(s - m)
                return w @ V, m + math.log(w.sum()), w, s
            if mutant == "sign_flip":
                w = np.exp(m - s)
                return (w / w.sum()) @ V, m + math.log(w.sum()), w / w.sum(), s
            w = np.exp(s - m)  # lse_without_max
            return (w / w.sum()) @ V, math.log(w.sum()), w / w.sum(), s
        monkeypatch.setattr(O, "softmax_attention", sa)
    assert _some_pin_fails()


@pytest.mark.parametrize("mutant", ["and_instead_of_or", "descending_side_list", "non_strict"])
def test_planted_selection_mistake_is_caught(monkeypatch, mutant):
    orig = O.compress_hybrid
    if mutant == "and_instead_of_or":
        def ch(k, v, bk, bv, tau, dtype, pos=0):
            res = orig(k, v, bk, bv, tau, dtype, pos)
            for key in res["flags"]:
                fk = O.hybrid_flags(np.asarray(k)[key[0], :, key[1]], bk[key[1]], tau, dtype)
                fv = O.hybrid_flags(np.asarray(v)[key[0], :, key[1]], bv[key[1]], tau, dtype)
                res["flags"][key] = fk & fv
            return res
        monkeypatch.setattr(O, "compress_hybrid", ch)
    elif mutant == "descending_side_list":
        def ch(*a, **kw):
            res = orig(*a, **kw)
            for key in res["side_idx"]:
                res["side_idx"][key] = res["side_idx"][key][::-1]
            return res
        monkeypatch.setattr(O, "compress_hybrid", ch)
    else:
        orig_flags = O.hybrid_flags
        # ">=" instead of ">" is visible at tau = 0 on zero tokens
        monkeypatch.setattr(O, "hybrid_flags", lambda x, b, tau, dt: orig_flags(x, b, tau, dt) |
                            (np.linalg.norm(np.asarray(x), axis=1) == 0))
    with pytest.raises(AssertionError):
        if mutant == "non_strict":
            test_hybrid_flags_closed_form()
        else:
            test_hybrid_compaction_order_golden()


def test_row_sampled_decoders_match_the_full_decoder():
    """decode_rows (sampled rows) and decode_hybrid_rows with an empty side list
    equal the pinned full decode."""
    q, bk, ck, bv, cv = _case(12)
    n = 30
    o, lse = O.decode(q, bk, ck, bv, cv, n)
    g = q.shape[1] // bk.shape[0]
    rows = [(b, hq) for b in range(q.shape[0]) for hq in range(q.shape[1])]
    ckd = {(b, h): ck[b, h] for b in range(ck.shape[0]) for h in range(ck.shape[1])}
    cvd = {(b, h): cv[b, h] for b in range(cv.shape[0]) for h in range(cv.shape[1])}
    r1 = O.decode_rows(q, bk, ckd, bv, cvd, n, rows)
    cks = {key: v[:n] for key, v in ckd.items()}
    cvs = {key: v[:n] for key, v in cvd.items()}
    empty = {key: np.zeros((0, q.shape[2])) for key in ckd}
    r2 = O.decode_hybrid_rows(q, bk, bv, cks, cvs, empty, empty, rows)
    for (b, hq) in rows:
        for r in (r1, r2):
            assert np.max(np.abs(r[(b, hq)][0] - o[b, hq])) <= 1e-14
            assert abs(r[(b, hq)][1] - lse[b, hq]) <= 1e-13


def test_latent_decode_matches_sdpa_and_absorbs_the_bases():
    """decode_latent is torch's dense attention on the coefficient rows (with
    the scale passed explicitly), and lifting its output through B_V gives
    the pinned decode over reconstructed keys and values with q' = q B_K, for
    non-orthonormal bases too (absorbed projections change nothing)."""
    rng = np.random.default_rng(21)
    B, Hq, Hkv, d, rk, rv, n = 2, 8, 2, 16, 6, 10, 37
    q = rng.standard_normal((B, Hq, d))
    bk = rng.standard_normal((Hkv, d, rk)) / 3
    bv = rng.standard_normal((Hkv, d, rv)) / 3
    ck = rng.standard_normal((B, Hkv, n + 5, rk))
    cv = rng.standard_normal((B, Hkv, n + 5, rv))
    g = Hq // Hkv
    q_lat = np.stack([np.stack([q[b, hq] @ bk[hq // g] for hq in range(Hq)]) for b in range(B)])
    scale = 1 / math.sqrt(d)
    o_lat, lse_lat = O.decode_latent(q_lat, ck, cv, n, scale)
    assert np.max(np.abs(o_lat - _sdpa(q_lat, ck[:, :, :n], cv[:, :, :n], scale=scale))) <= 1e-13
    assert np.max(np.abs(lse_lat - _sdpa_lse(q_lat, ck[:, :, :n], g, scale))) <= 1e-12
    o, lse = O.decode(q, bk, ck, bv, cv, n)
    lifted = np.stack([np.stack([o_lat[b, hq] @ bv[hq // g].T for hq in range(Hq)]) for b in range(B)])
    assert np.max(np.abs(lifted - o)) <= 1e-12 * np.max(np.abs(o))
    assert np.max(np.abs(lse - lse_lat)) <= 1e-12
