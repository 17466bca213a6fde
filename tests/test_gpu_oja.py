"""GPU parity for the Oja subspace update of the bases (lrkv_oja_update).

The oracle's oja_update_heads (float64, pinned in test_oracle_oja.py) runs
on the same bfloat16 tokens and the same float32 starting basis.  Gate: the
kernel evaluates S1 = X^T Y and B S2 = B Y^T Y in float32 (with the float32
operands split into high and low bfloat16 parts on the matrix cores) and
subtracts them, so its error is a small multiple of float32 rounding of
those two terms, not of their difference:
  |B_gpu - B_ref| <= 1e-4 * eta * max(|S1|, |B S2|) + 2^-23 |B_ref|.
The bfloat16 copy must be the kernel's float32 result rounded to nearest even,
bit for bit.
"""
import numpy as np
import pytest
import torch

import lrkv_synth as synth
from oracle import lrkv_oracle as O
from tests.gpu_helpers import DEV, bits, check_decode, to_dev, to_f64

pytestmark = pytest.mark.gpu

lrkv = pytest.importorskip("decode_attention_lrkv_amd")


def _tokens(w, layer, which, T, part=synth.PART_PREFILL):
    return synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(w, layer, which, b, h, T, part)))


def _check(x_exact, b0, b_gpu, bf_gpu, eta, what):
    ref = O.oja_update_heads(b0, x_exact, eta)
    worst = 0.0
    for h in range(b0.shape[0]):
        X = x_exact[:, :, h, :].reshape(-1, x_exact.shape[-1])
        Y = X @ b0[h]
        scale = eta * max(np.abs(X.T @ Y).max(), np.abs(b0[h] @ (Y.T @ Y)).max())
        err = np.abs(b_gpu[h] - ref[h])
        tol = 1e-4 * scale + 2.0 ** -23 * np.abs(ref[h])
        assert np.all(err <= tol), f"{what}: head {h} error {err.max():.3e} over the gate (scale {scale:.3e})"
        worst = max(worst, float((err / (1e-4 * scale)).max()))
    # the step is not lost in rounding: the basis moved by far more than the error
    assert np.abs(ref - b0).max() > 100 * np.abs(b_gpu - ref).max() or eta == 0.0, what
    # the bfloat16 copy is the float32 result rounded to nearest even
    np.testing.assert_array_equal(bf_gpu, synth.f32_to_bf16_bits(b_gpu.astype(np.float32)), err_msg=what)
    return worst


def _run(x, b0, eta, workspace=None):
    basis = torch.from_numpy(b0.astype(np.float32)).to(DEV)
    bf = lrkv.oja_update(to_dev(x, "bf16"), basis, eta, workspace=workspace)
    torch.cuda.synchronize()
    return to_f64(basis), bits(bf)


@pytest.mark.parametrize("d,r,B,T,H", [(64, 16, 2, 100, 2), (64, 24, 1, 333, 3), (128, 56, 2, 96, 8),
                                       (128, 72, 1, 1, 2), (128, 128, 1, 130, 1), (128, 8, 3, 64, 4),
                                       (128, 32, 2, 77, 3), (64, 48, 1, 200, 2), (128, 112, 1, 250, 2),
                                       (64, 16, 2, 3, 2), (128, 128, 1, 64, 1), (128, 8, 3, 20, 4),
                                       (64, 48, 16, 1, 3), (128, 112, 16, 4, 8), (128, 112, 13, 5, 2),
                                       (64, 64, 8, 8, 1), (128, 40, 3, 3000, 8), (64, 32, 5, 2001, 8)])
def test_oja_update_small(d, r, B, T, H):
    """Ragged token counts (a last step with 1..63 tokens, or one token), ranks
    that pad to whole 16-column blocks, both head dims; one and two
    coefficient blocks put four and two waves on each block.  Chunks of at
    most 64 tokens per head (here 1 to 64, a decode step's 16 among them) take
    the single-launch path; 65 tokens (13 x 5) and more the Gram path, whose
    runs of 128-token steps end ragged (9000 and 10005 tokens over 32 runs
    per head: three steps per run, the last one partial)."""
    w = synth.scaled(synth.LLAMA_LAYER, batch=B, n_kv_heads=H, head_dim=d, ranks_even=(r, r), ranks_odd=(r, r))
    x = _tokens(w, 0, "k", T)
    b0 = synth.basis(w, 0, "k").exact
    eta = 1e-3
    b_gpu, bf_gpu = _run(x, b0, eta)
    worst = _check(x.exact, b0, b_gpu, bf_gpu, eta, f"d {d} r {r} B {B} T {T} H {H}")
    print(f"[oja] d {d} r {r} tokens {B * T}: worst error {worst:.3f} of the gate", flush=True)


@pytest.mark.parametrize("layer", [0, 1])
def test_oja_update_prefill_chunk_full_size(layer):
    """The benchmark's prefill chunk: batch 16 x 4096 tokens x 8 kv heads, the
    key and the value basis of an even and an odd layer (ranks 32/96, 48/112)."""
    w = synth.BATCHED_32K
    rk, rv = w.ranks(layer)
    eta = 2e-6
    for which, r in (("k", rk), ("v", rv)):
        x = _tokens(w, layer, which, w.prefill)
        b0 = synth.basis(w, layer, which).exact
        b_gpu, bf_gpu = _run(x, b0, eta)
        worst = _check(x.exact, b0, b_gpu, bf_gpu, eta, f"layer {layer} {which} r {r}")
        print(f"[oja] layer {layer} {which} r {r}: worst error {worst:.3f} of the gate", flush=True)


def test_oja_zero_step_and_empty_chunk_leave_the_basis():
    w = synth.scaled(synth.LLAMA_LAYER, batch=2, n_kv_heads=2, ranks_even=(32, 32))
    x = _tokens(w, 0, "k", 50)
    b0 = synth.basis(w, 0, "k").exact
    b_gpu, bf_gpu = _run(x, b0, 0.0)
    np.testing.assert_array_equal(b_gpu, b0)
    np.testing.assert_array_equal(bf_gpu, synth.f32_to_bf16_bits(b0.astype(np.float32)))
    basis = torch.from_numpy(b0.astype(np.float32)).to(DEV)
    empty = torch.zeros((2, 0, 2, 128), dtype=torch.bfloat16, device=DEV)
    lrkv.oja_update(empty, basis, 1e-3)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_f64(basis), b0)


def test_oja_tokens_in_the_span_barely_move_the_basis():
    """Tokens c B^T (rounded to bfloat16, so almost in the span): the step is
    within the gate of the oracle's, and tiny against the terms it cancels."""
    w = synth.scaled(synth.LLAMA_LAYER, batch=1, n_kv_heads=2, ranks_even=(48, 48))
    b0 = synth.basis(w, 0, "k").exact
    rng = np.random.default_rng(11)
    c = rng.standard_normal((1, 300, 2, 48))
    x_exact = np.einsum("bthr,hdr->bthd", c, b0)
    x_store = synth.f32_to_bf16_bits(x_exact.astype(np.float32))
    x = synth.Stored(x_store, synth.bf16_bits_to_f64(x_store))
    eta = 1e-3
    basis = torch.from_numpy(b0.astype(np.float32)).to(DEV)
    bf = lrkv.oja_update(to_dev(x, "bf16"), basis, eta)
    torch.cuda.synchronize()
    b_gpu = to_f64(basis)
    ref = O.oja_update_heads(b0, x.exact, eta)
    for h in range(2):
        X = x.exact[:, :, h, :].reshape(-1, 128)
        Y = X @ b0[h]
        scale = eta * np.abs(X.T @ Y).max()
        assert np.abs(b_gpu[h] - ref[h]).max() <= 1e-4 * scale + 2.0 ** -23
        assert np.abs(ref[h] - b0[h]).max() < 1e-2 * scale   # the step is small against the terms
    np.testing.assert_array_equal(bits(bf), synth.f32_to_bf16_bits(b_gpu.astype(np.float32)))


def test_oja_repeated_steps_track_the_principal_subspace():
    """Forty steps on tokens with a planted covariance bring a random
    orthonormal basis onto the top eigenvectors (numpy), as in the oracle."""
    d, r, H = 64, 8, 1
    rng = np.random.default_rng(12)
    U = np.linalg.qr(rng.standard_normal((d, d)))[0]
    lam = np.concatenate([np.linspace(6.0, 4.0, r), np.full(d - r, 0.5)])
    X = (rng.standard_normal((40 * 512, d)) * np.sqrt(lam)[None, :]) @ U.T
    x_store = synth.f32_to_bf16_bits(X.astype(np.float32)).reshape(40, 1, 512, H, d)
    b = np.linalg.qr(rng.standard_normal((d, r)))[0][None].astype(np.float32)
    basis = torch.from_numpy(b).to(DEV)
    ref = b.astype(np.float64)
    for it in range(40):
        xs = synth.Stored(x_store[it], synth.bf16_bits_to_f64(x_store[it]))
        lrkv.oja_update(to_dev(xs, "bf16"), basis, 1e-4)
        ref = O.oja_update_heads(ref, xs.exact, 1e-4)
    torch.cuda.synchronize()
    b_gpu = to_f64(basis)[0]
    top = U[:, :r]
    s = np.linalg.svd(top.T @ np.linalg.qr(b_gpu)[0], compute_uv=False)
    assert np.sqrt(max(0.0, 1.0 - s.min() ** 2)) < 0.1
    assert np.abs(b_gpu - ref[0]).max() < 1e-4 * np.abs(ref[0]).max()


def test_oja_graph_replays_equal_eager_steps():
    """A captured update replayed four times (with unrelated eager work
    between replays) gives, bit for bit, the bases of four eager updates."""
    w = synth.scaled(synth.LLAMA_LAYER, batch=2, n_kv_heads=2, ranks_even=(96, 96))
    x = to_dev(_tokens(w, 0, "k", 300), "bf16")
    b0 = torch.from_numpy(synth.basis(w, 0, "k").exact.astype(np.float32)).to(DEV)
    ws = torch.zeros(lrkv.oja_workspace_bytes(2, 2, 128, 96, 300), dtype=torch.uint8, device=DEV)
    eager = b0.clone()
    eager_bf = []
    for _ in range(4):
        eager_bf.append(lrkv.oja_update(x, eager, 1e-3, workspace=ws).clone())
    torch.cuda.synchronize()
    basis = b0.clone()
    bf = torch.empty_like(eager_bf[0])
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        lrkv.oja_update(x, basis.clone(), 1e-3, basis_bf16=bf, workspace=ws)   # warm up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        lrkv.oja_update(x, basis, 1e-3, basis_bf16=bf, workspace=ws)
    basis.copy_(b0)
    torch.cuda.synchronize()
    for i in range(4):
        bf.zero_()
        _ = (x.float() * 2).sum()                       # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bf.view(torch.int16), eager_bf[i].view(torch.int16)), f"replay {i}"
    assert torch.equal(basis, eager)


@pytest.mark.parametrize("eta", [2e-3, 8e-3])
def test_decode_step_after_an_update_at_decode_shape(eta):
    """The update in decoding ("OjaKV" README, Method Summary, OjaKV: the
    subspace is updated during decoding too), at the decode step's shape:
    batch 16, one token per sequence, 8 kv heads, ranks 48 / 112.  Both bases
    are updated from the step's token, then the decode step compresses that
    token with the updated bases and attends all N rows through them; rows
    already in the cache keep the coefficients of the starting bases (they are
    not re-projected).  GPU and oracle each run the whole sequence from the
    same tokens and starting bases.  The drift those old rows cause (the
    output through the updated bases against the output through the starting
    bases, in units of the output's RMS) is printed."""
    w = synth.scaled(synth.BATCHED_32K, n_ctx=(2048,))
    layer, N = 1, 2048
    B, Hq, H, d = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    ck = synth.stack_heads(w, lambda b, h: synth.direct_coeffs(w, layer, "k", b, h, N - 1))
    cv = synth.stack_heads(w, lambda b, h: synth.direct_coeffs(w, layer, "v", b, h, N - 1))
    xk = _tokens(w, layer, "k", 1, synth.PART_APPEND)
    xv = _tokens(w, layer, "v", 1, synth.PART_APPEND)
    q = synth.query(w, layer)
    bk0, bv0 = synth.basis(w, layer, "k").exact, synth.basis(w, layer, "v").exact
    # GPU: update both float32 bases from the token, then one decode step through the bfloat16 copies
    bk32 = torch.from_numpy(bk0.astype(np.float32)).to(DEV)
    bv32 = torch.from_numpy(bv0.astype(np.float32)).to(DEV)
    kn, vn = to_dev(xk, "bf16"), to_dev(xv, "bf16")
    bkb = lrkv.oja_update(kn, bk32, eta)
    bvb = lrkv.oja_update(vn, bv32, eta)
    ckd = to_dev(np.concatenate([ck.store, np.zeros((B, H, 1, ck.store.shape[-1]), np.uint16)], 2), "bf16")
    cvd = to_dev(synth.to_value_octets(np.concatenate([cv.store, np.zeros((B, H, 1, cv.store.shape[-1]),
                                                                            np.uint16)], 2)), "bf16")
    o, lse = lrkv.decode_step(to_dev(q, "bf16"), kn.view(B, H, d), vn.view(B, H, d), bkb, ckd, bvb, cvd, N)
    torch.cuda.synchronize()
    # oracle: the same sequence in float64 (bases rounded to bfloat16 where the cache and decode take them)
    bk1 = O.round_storage(O.oja_update_heads(bk0, xk.exact, eta), "bf16")
    bv1 = O.round_storage(O.oja_update_heads(bv0, xv.exact, eta), "bf16")
    assert np.any(bk1 != bk0) and np.any(bv1 != bv0)   # the step moved both bfloat16 bases

    def run(bk, bv):
        ak = O.round_storage(O.compress(xk.exact, bk), "bf16")
        av = O.round_storage(O.compress(xv.exact, bv), "bf16")
        return O.decode(q.exact, bk, np.concatenate([ck.exact, ak], 2), bv, np.concatenate([cv.exact, av], 2), N)

    o_ref, lse_ref = run(bk1, bv1)
    check_decode(to_f64(o), to_f64(lse), o_ref, lse_ref, "bf16", f"decode after an update, eta {eta}")
    o_start, _ = run(bk0, bv0)
    drift = np.max(np.abs(o_ref - o_start), -1) / np.sqrt(np.mean(o_ref ** 2, -1))
    print(f"[oja decode] eta {eta}: drift of the output through the updated bases, max {drift.max():.3e}, "
          f"median {np.median(drift):.3e} of the row RMS", flush=True)
