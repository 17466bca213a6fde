"""The seeded input generator: determinism, structure and rounding."""
import hashlib

import numpy as np
import torch

import lrkv_synth as synth


def _sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_deterministic_and_sliceable():
    w = synth.LLAMA_LAYER
    a = synth.direct_coeffs(w, 0, "k", 0, 3, 128)
    b = synth.direct_coeffs(w, 0, "k", 0, 3, 128)
    assert _sha(a.store) == _sha(b.store)
    c = synth.direct_coeffs(w, 0, "k", 0, 4, 128)
    assert _sha(a.store) != _sha(c.store)
    # a prefix of a longer draw is the shorter draw (rows are drawn in order)
    d = synth.direct_coeffs(w, 0, "k", 0, 3, 256)
    assert np.array_equal(d.store[:128], a.store)
    full = synth.stack_heads(w, lambda b, h: synth.direct_coeffs(w, 0, "v", b, h, 64))
    assert full.shape == (1, 8, 64, 80)
    assert np.array_equal(full.store[0, 5], synth.direct_coeffs(w, 0, "v", 0, 5, 64).store)


def test_bases_are_orthonormal_frames():
    w = synth.LLAMA_LAYER
    for h in range(w.n_kv_heads):
        f = synth.frame(w, 0, h, "k")
        assert np.allclose(f.T @ f, np.eye(w.head_dim), atol=1e-12)
    b = synth.basis(w, 0, "v")
    assert b.shape == (8, 128, 80)
    g = np.einsum("hdr,hds->hrs", b.exact, b.exact)
    # rounded to bf16, the columns stay orthonormal to about 2^-8
    assert np.max(np.abs(g - np.eye(80)[None])) < 2 ** -6


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    bits = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    assert np.array_equal(synth.bf16_bits_to_f64(bits),
                          torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_spectrum_and_full_tokens():
    w = synth.scaled(synth.LLAMA_STEP, dtype="f32")
    x = synth.full_tokens(w, 0, "k", 0, 0, 20000, synth.PART_PREFILL).exact
    f = synth.frame(w, 0, 0, "k")
    z = x @ f
    std = z.std(0)
    assert np.allclose(std, 0.95 ** np.arange(128), rtol=0.05)


def test_value_octet_layout_round_trip():
    c = np.arange(2 * 3 * 16 * 5).reshape(2, 3, 16, 5)
    t = synth.to_value_octets(c)
    assert t.shape == (2, 3, 2, 5, 8)
    assert t[1, 2, 1, 4, 3] == c[1, 2, 8 + 3, 4]
    assert np.array_equal(synth.from_value_octets(t), c)


def test_hybrid_injection_structure():
    n = 2048
    w = synth.scaled(synth.HYBRID_128K, n_ctx=(n,))
    inj = synth.injected_set(w, 0, 0, n)
    assert len(inj) == round(0.05 * n) and np.all(np.diff(inj) > 0)
    x = synth.hybrid_tokens(w, 0, "k", 0, 0, n, inj).exact
    q = synth.frame(w, 0, 0, "k")[:, :64]
    off = x - (x @ q) @ q.T
    norms = np.linalg.norm(x, axis=1)
    base = np.setdiff1d(np.arange(n), inj)
    # injected tokens carry an off-span part of 3x the median base norm (before rounding)
    m = np.median(norms[base])
    assert np.allclose(np.linalg.norm(off[inj], axis=1) / m, 3.0, rtol=0.05)
    assert np.max(np.linalg.norm(off[base], axis=1) / norms[base]) < 0.01


def test_key_transform_pairs_are_biorthogonal_and_not_orthonormal():
    w = synth.LLAMA_LAYER
    rk = w.ranks(0)[0]
    enc, dec = synth.key_transform(w, 0, "k")
    assert enc.shape == dec.shape == (8, 128, rk)
    for h in range(w.n_kv_heads):
        root, root_inv = synth.query_moment_root(w, 0, h)
        assert np.allclose(root @ root_inv, np.eye(128), atol=1e-12)
        assert np.allclose(root, root.T, atol=1e-13) and np.linalg.eigvalsh(root).min() > 0.49
        # dec^T enc = I up to the bf16 rounding of both
        assert np.max(np.abs(dec.exact[h].T @ enc.exact[h] - np.eye(rk))) < 2 ** -5
        # the encoder is far from orthonormal, and the decoder spans F_r
        assert np.max(np.abs(enc.exact[h].T @ enc.exact[h] - np.eye(rk))) > 0.5
        fr = synth.frame(w, 0, h, "k")[:, :rk]
        qd = np.linalg.qr(dec.exact[h])[0]
        assert np.max(np.abs(fr - qd @ (qd.T @ fr))) < 2 ** -6
    q = synth.query_aware_query(w, 0)
    assert q.shape == (1, 32, 128)
    q2 = synth.query_aware_query(w, 0)
    assert _sha(q.store) == _sha(q2.store)
