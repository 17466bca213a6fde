"""GPU parity for a non-orthogonal key transform: the key cache is written
with an encoder E and read with its decoder D (D^T E = I), the form of the
attention-aware key transform in the NOVA-KV summary (Methodology, Key
Transform Derivation, Theorem 1 and Proposition 1).  Values keep an
orthonormal basis (same summary, Value Transform, Corollary 1).

The oracle compresses with E and reconstructs with D explicitly; the GPU
compresses with E (lrkv_compress, or the decode step's enc_k) and folds the
query through D.  Gates as for the orthonormal path.
"""
import numpy as np
import pytest
import torch

import lrkv_synth as synth
from oracle import lrkv_oracle as O
from tests.gpu_helpers import (DEV, bits, check_decode, round_store, to_dev, to_f64)
from tests.test_gpu_parity_small import check_compress

pytestmark = pytest.mark.gpu

lrkv = pytest.importorskip("decode_attention_lrkv_amd")

LAYER_BF16 = synth.scaled(synth.LLAMA_LAYER, n_ctx=(1000,))
STEP_BATCHED = synth.scaled(synth.BATCHED_32K, n_ctx=(4096,))


def _full(w, layer, which, n, part):
    return synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(w, layer, which, b, h, n, part)))


def _cache(rows_k, rows_v, dtype, cap):
    B, H, n, rk = rows_k.shape
    ck = np.zeros((B, H, cap, rk))
    cv = np.zeros((B, H, cap, rows_v.shape[-1]))
    ck[:, :, :n] = rows_k
    cv[:, :, :n] = rows_v
    return to_dev(round_store(ck, dtype), dtype), to_dev(synth.to_value_octets(round_store(cv, dtype)), dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_transform_compress_then_decode(dtype):
    """(i) compress with the encoder, (ii) decode with the decoder on the
    oracle's rows, (iii) both on the GPU, against the oracle end to end."""
    w = LAYER_BF16 if dtype == "bf16" else synth.TINY_F32
    layer, N = 0, w.n_ctx[0]
    B, H, d = w.batch, w.n_kv_heads, w.head_dim
    rk, rv = w.ranks(layer)
    enc, dec = synth.key_transform(w, layer, "k")
    bv = synth.basis(w, layer, "v")
    q = synth.query_aware_query(w, layer)
    K = _full(w, layer, "k", N, synth.PART_PREFILL)
    V = _full(w, layer, "v", N, synth.PART_PREFILL)
    ck_exact, cv_exact = O.compress(K.exact, enc.exact), O.compress(V.exact, bv.exact)
    ck_st, cv_st = O.round_storage(ck_exact, dtype), O.round_storage(cv_exact, dtype)
    o_ref, lse_ref = O.decode(q.exact, dec.exact, ck_st, bv.exact, cv_st, N)
    # the decoder matters: reading the rows back through the encoder is far off
    o_wrong, _ = O.decode(q.exact, enc.exact, ck_st, bv.exact, cv_st, N)
    assert np.max(np.abs(o_wrong - o_ref)) > 0.2 * np.sqrt(np.mean(o_ref ** 2))

    cap = (N + 7) // 8 * 8
    qd, encd, decd, bvd = (to_dev(x, dtype) for x in (q, enc, dec, bv))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    ck_dev = torch.zeros((B, H, cap, rk), dtype=tdt, device=DEV)
    cv_dev = torch.zeros(lrkv.value_cache_shape(B, H, cap, rv), dtype=tdt, device=DEV)
    lrkv.compress(to_dev(K, dtype), encd, ck_dev, 0, values=False)
    lrkv.compress(to_dev(V, dtype), bvd, cv_dev, 0, values=True)
    torch.cuda.synchronize()
    check_compress(to_f64(ck_dev)[:, :, :N], ck_exact, K.exact, enc.exact, dtype, "transform K")
    check_compress(synth.from_value_octets(to_f64(cv_dev))[:, :, :N], cv_exact, V.exact, bv.exact, dtype,
                   "transform V")
    ck2, cv2 = _cache(ck_st, cv_st, dtype, cap)
    o, lse = lrkv.decode_attn(qd, decd, ck2, bvd, cv2, N)
    check_decode(to_f64(o), to_f64(lse), o_ref, lse_ref, dtype, "transform decode")
    o3, lse3 = lrkv.decode_attn(qd, decd, ck_dev, bvd, cv_dev, N)
    check_decode(to_f64(o3), to_f64(lse3), o_ref, lse_ref, dtype, "transform end to end")


@pytest.mark.parametrize("case", ["bf16-1", "bf16-33", "bf16-2048", "bf16-b16-4096", "f32-200"])
def test_transform_decode_step(case):
    """The decode step with a key encoder: the appended key row is round(k E),
    the value row round(v B_V), the drawn rows stay, and the output is the
    oracle's decode through D over all N tokens.  b16-4096 has more
    workgroups than one round holds, so the last attention workgroup appends;
    the others append from a workgroup of their own."""
    kind, *rest = case.split("-")
    dtype = kind
    if dtype == "f32":
        w, layer, N = synth.TINY_F32, 0, int(rest[0])
    elif rest[0] == "b16":
        w, layer, N = STEP_BATCHED, 1, int(rest[1])
    else:
        w, layer, N = synth.LLAMA_STEP, 1, int(rest[0])
    B, H, d = w.batch, w.n_kv_heads, w.head_dim
    rk, rv = w.ranks(layer)
    enc, dec = synth.key_transform(w, layer, "k")
    bv = synth.basis(w, layer, "v")
    q = synth.query_aware_query(w, layer)
    xk = _full(w, layer, "k", 1, synth.PART_APPEND)
    xv = _full(w, layer, "v", 1, synth.PART_APPEND)
    ak, av = O.compress(xk.exact, enc.exact), O.compress(xv.exact, bv.exact)
    rows_k = np.zeros((B, H, N, rk))
    rows_v = np.zeros((B, H, N, rv))
    if N > 1:
        rows_k[:, :, :N - 1] = synth.stack_heads(w, lambda b, h: synth.direct_coeffs(w, layer, "k", b, h, N - 1)).exact
        rows_v[:, :, :N - 1] = synth.stack_heads(w, lambda b, h: synth.direct_coeffs(w, layer, "v", b, h, N - 1)).exact
    ck_all = rows_k.copy(); ck_all[:, :, N - 1:] = O.round_storage(ak, dtype)
    cv_all = rows_v.copy(); cv_all[:, :, N - 1:] = O.round_storage(av, dtype)
    o_ref, lse_ref = O.decode(q.exact, dec.exact, ck_all, bv.exact, cv_all, N)

    cap = max(8, (N + 7) // 8 * 8)
    ckd, cvd = _cache(rows_k, rows_v, dtype, cap)
    before = bits(ckd)
    qd, encd, decd, bvd = (to_dev(x, dtype) for x in (q, enc, dec, bv))
    kn, vn = to_dev(xk, dtype), to_dev(xv, dtype)
    o, lse = lrkv.decode_step(qd, kn, vn, decd, ckd, bvd, cvd, N, enc_k=encd)
    torch.cuda.synchronize()
    check_compress(to_f64(ckd)[:, :, N - 1:N], ak, xk.exact, enc.exact, dtype, f"{case} append K")
    check_compress(synth.from_value_octets(to_f64(cvd))[:, :, N - 1:N], av, xv.exact, bv.exact, dtype,
                   f"{case} append V")
    after = bits(ckd)
    assert np.array_equal(after[:, :, :N - 1], before[:, :, :N - 1])
    assert np.array_equal(after[:, :, N:], before[:, :, N:])
    check_decode(to_f64(o), to_f64(lse), o_ref, lse_ref, dtype, f"transform step {case}")


def test_transform_step_without_encoder_is_the_plain_step():
    """enc_k = basis_k agrees with enc_k = None: the encoder path and the
    staged-basis path round the same sums (added in other orders) to the same
    key row up to one bfloat16 step, write the same value row, and give
    outputs within the gate of each other."""
    w, layer, N = synth.LLAMA_STEP, 0, 700
    B, H = w.batch, w.n_kv_heads
    rk, rv = w.ranks(layer)
    rows_k = np.zeros((B, H, N, rk)); rows_k[:, :, :N - 1] = synth.stack_heads(
        w, lambda b, h: synth.direct_coeffs(w, layer, "k", b, h, N - 1)).exact
    rows_v = np.zeros((B, H, N, rv)); rows_v[:, :, :N - 1] = synth.stack_heads(
        w, lambda b, h: synth.direct_coeffs(w, layer, "v", b, h, N - 1)).exact
    xk = to_dev(_full(w, layer, "k", 1, synth.PART_APPEND), "bf16")
    xv = to_dev(_full(w, layer, "v", 1, synth.PART_APPEND), "bf16")
    qd, bkd, bvd = (to_dev(x, "bf16") for x in (synth.query(w, layer), synth.basis(w, layer, "k"),
                                                synth.basis(w, layer, "v")))
    ck1, cv1 = _cache(rows_k, rows_v, "bf16", (N + 7) // 8 * 8)
    ck2, cv2 = ck1.clone(), cv1.clone()
    o1, l1 = lrkv.decode_step(qd, xk, xv, bkd, ck1, bvd, cv1, N)
    o2, l2 = lrkv.decode_step(qd, xk, xv, bkd, ck2, bvd, cv2, N, enc_k=bkd)
    torch.cuda.synchronize()
    # the two paths sum the same products in different orders: rows may differ
    # by one rounding step, outputs stay within the gate of each other
    r1, r2 = to_f64(ck1)[:, :, N - 1], to_f64(ck2)[:, :, N - 1]
    assert np.all(np.abs(r1 - r2) <= 2.0 ** -7 * np.maximum(np.abs(r1), 1e-30) + 1e-30)
    assert np.array_equal(bits(cv1), bits(cv2))
    check_decode(to_f64(o2), to_f64(l2), to_f64(o1), to_f64(l1), "bf16", "enc_k = basis_k")
