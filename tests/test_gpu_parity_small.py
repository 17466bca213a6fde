"""GPU parity on the small workloads: the HIP path against the CPU oracle.

Three comparisons per workload, all gated:
 (i)   compress on the GPU vs the oracle's exact coefficients;
 (ii)  decode on the GPU vs the oracle on identical cache contents (the
       cache is filled from the generator or from the oracle's own rounded
       compress, never from the GPU);
 (iii) end to end: GPU compress then GPU decode vs the oracle's compress and
       decode of the same full vectors.
"""
import math

import numpy as np
import pytest
import torch

import lrkv_synth as synth
from oracle import lrkv_oracle as O
from tests.gpu_helpers import (DEV, bf16_ulp, bits, check_decode, round_store, to_dev, to_f64)

pytestmark = pytest.mark.gpu

lrkv = pytest.importorskip("decode_attention_lrkv_amd")


def check_compress(c_gpu: np.ndarray, c_exact: np.ndarray, x: np.ndarray, basis: np.ndarray,
                   dtype: str, what: str):
    """Compress gate.

    float32: normwise per (b, h) <= 1e-5.
    bfloat16: |c_gpu - c_exact| <= ulp_bf16(c_exact) + delta elementwise, with
    delta = d * 2^-24 * sum_i |x_i B_ic| bounding the float32 accumulation error
    (so a rounding decision that float32 accumulation may flip costs one ulp).
    c_gpu, c_exact [B, Hkv, T, r]; x [B, T, Hkv, d]; basis [Hkv, d, r].
    """
    if dtype == "f32":
        num = np.sqrt(np.sum((c_gpu - c_exact) ** 2, axis=(2, 3)))
        den = np.sqrt(np.sum(c_exact ** 2, axis=(2, 3)))
        assert np.all(num <= 1e-5 * den), f"{what}: compress error {np.max(num / den):.3e}"
        return
    d = x.shape[-1]
    mag = np.einsum("bthd,hdr->bhtr", np.abs(x), np.abs(basis))
    tol = bf16_ulp(c_exact) + d * 2.0 ** -24 * mag
    err = np.abs(c_gpu - c_exact)
    assert np.all(err <= tol), f"{what}: compress error {np.max(err / tol):.3f} of tolerance"


def _cache_from_rows(ck_rows, cv_rows, dtype, cap):
    """Row-layout float64 coefficient rows [B, Hkv, n, r] -> device caches of capacity cap."""
    B, H, n, rk = ck_rows.shape
    rv = cv_rows.shape[-1]
    ck = np.zeros((B, H, cap, rk), dtype=np.float64)
    cv = np.zeros((B, H, cap, rv), dtype=np.float64)
    ck[:, :, :n] = ck_rows
    cv[:, :, :n] = cv_rows
    ck_dev = to_dev(round_store(ck, dtype), dtype)
    cv_dev = to_dev(synth.to_value_octets(round_store(cv, dtype)), dtype)
    return ck_dev, cv_dev


def test_tiny_f32_pipeline():
    w = synth.TINY_F32
    N = w.n_ctx[0]
    K = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(w, 0, "k", b, h, N, synth.PART_PREFILL)))
    V = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(w, 0, "v", b, h, N, synth.PART_PREFILL)))
    bk, bv, q = synth.basis(w, 0, "k"), synth.basis(w, 0, "v"), synth.query(w, 0)
    ck_exact = O.compress(K.exact, bk.exact)
    cv_exact = O.compress(V.exact, bv.exact)
    ck_st = O.round_storage(ck_exact, "f32")
    cv_st = O.round_storage(cv_exact, "f32")
    o_ref, lse_ref = O.decode(q.exact, bk.exact, ck_st, bv.exact, cv_st, N)

    qd, bkd, bvd = to_dev(q, "f32"), to_dev(bk, "f32"), to_dev(bv, "f32")
    cap = N
    ck_dev = torch.empty((1, 1, cap, 16), dtype=torch.float32, device=DEV)
    cv_dev = torch.empty(lrkv.value_cache_shape(1, 1, cap, 16), dtype=torch.float32, device=DEV)
    lrkv.compress(to_dev(K, "f32"), bkd, ck_dev, 0, values=False)
    lrkv.compress(to_dev(V, "f32"), bvd, cv_dev, 0, values=True)
    torch.cuda.synchronize()
    check_compress(to_f64(ck_dev), ck_exact, K.exact, bk.exact, "f32", "tiny K")
    check_compress(synth.from_value_octets(to_f64(cv_dev)), cv_exact, V.exact, bv.exact, "f32", "tiny V")

    ck2, cv2 = _cache_from_rows(ck_st, cv_st, "f32", cap)
    o, lse = lrkv.decode_attn(qd, bkd, ck2, bvd, cv2, N)
    check_decode(to_f64(o), to_f64(lse), o_ref, lse_ref, "f32", "tiny decode")
    o3, lse3 = lrkv.decode_attn(qd, bkd, ck_dev, bvd, cv_dev, N)
    check_decode(to_f64(o3), to_f64(lse3), o_ref, lse_ref, "f32", "tiny end-to-end")


def _direct_rows(w, layer, which, n, batch=None):
    return synth.stack_heads(w, lambda b, h: synth.direct_coeffs(w, layer, which, b, h, n), batch=batch)


def test_llama_layer_decode():
    w = synth.LLAMA_LAYER
    N = w.n_ctx[0]
    ck, cv = _direct_rows(w, 0, "k", N), _direct_rows(w, 0, "v", N)
    bk, bv, q = synth.basis(w, 0, "k"), synth.basis(w, 0, "v"), synth.query(w, 0)
    o_ref, lse_ref = O.decode(q.exact, bk.exact, ck.exact, bv.exact, cv.exact, N)
    ck_dev = to_dev(ck, "bf16")
    cv_dev = to_dev(synth.to_value_octets(cv.store), "bf16")
    o, lse = lrkv.decode_attn(to_dev(q, "bf16"), to_dev(bk, "bf16"), ck_dev, to_dev(bv, "bf16"), cv_dev, N)
    check_decode(to_f64(o), to_f64(lse), o_ref, lse_ref, "bf16", "llama layer")


@pytest.mark.parametrize("N", synth.LLAMA_STEP.n_ctx)
@pytest.mark.parametrize("layer", [0, 1, 31])
def test_llama_step_layer_with_append(N, layer):
    w = synth.LLAMA_STEP
    B, H, d = w.batch, w.n_kv_heads, w.head_dim
    rk, rv = w.ranks(layer)
    ck, cv = _direct_rows(w, layer, "k", N - 1), _direct_rows(w, layer, "v", N - 1)
    xk = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(w, layer, "k", b, h, 1, synth.PART_APPEND)))
    xv = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(w, layer, "v", b, h, 1, synth.PART_APPEND)))
    bk, bv, q = synth.basis(w, layer, "k"), synth.basis(w, layer, "v"), synth.query(w, layer)
    # oracle: compress the appended token, store it, decode over N tokens
    ak = O.compress(xk.exact, bk.exact)
    av = O.compress(xv.exact, bv.exact)
    ck_all = np.concatenate([ck.exact, O.round_storage(ak, "bf16")], axis=2)
    cv_all = np.concatenate([cv.exact, O.round_storage(av, "bf16")], axis=2)
    o_ref, lse_ref = O.decode(q.exact, bk.exact, ck_all, bv.exact, cv_all, N)

    cap = N
    qd, bkd, bvd = to_dev(q, "bf16"), to_dev(bk, "bf16"), to_dev(bv, "bf16")
    # (ii) decode on the oracle's cache contents
    ck2, cv2 = _cache_from_rows(ck_all, cv_all, "bf16", cap)
    o, lse = lrkv.decode_attn(qd, bkd, ck2, bvd, cv2, N)
    check_decode(to_f64(o), to_f64(lse), o_ref, lse_ref, "bf16", f"step N={N} layer={layer}")
    # (i) + (iii): the GPU appends the token into a cache holding the drawn rows
    rows_k = np.zeros((B, H, N, rk)); rows_k[:, :, :N - 1] = ck.exact
    rows_v = np.zeros((B, H, N, rv)); rows_v[:, :, :N - 1] = cv.exact
    ck3, cv3 = _cache_from_rows(rows_k, rows_v, "bf16", cap)
    lrkv.compress(to_dev(xk, "bf16"), bkd, ck3, N - 1, values=False)
    lrkv.compress(to_dev(xv, "bf16"), bvd, cv3, N - 1, values=True)
    o3, lse3 = lrkv.decode_attn(qd, bkd, ck3, bvd, cv3, N)
    torch.cuda.synchronize()
    check_compress(to_f64(ck3)[:, :, N - 1:N], ak, xk.exact, bk.exact, "bf16", "append K")
    check_compress(synth.from_value_octets(to_f64(cv3))[:, :, N - 1:N], av, xv.exact, bv.exact, "bf16", "append V")
    # the drawn rows are untouched
    assert np.array_equal(bits(ck3)[:, :, :N - 1], ck.store)
    check_decode(to_f64(o3), to_f64(lse3), o_ref, lse_ref, "bf16", f"step e2e N={N} layer={layer}")


@pytest.mark.parametrize("N", [1, 2, 33, 256, 2048, 8192])
@pytest.mark.parametrize("layer", [0, 31])
def test_decode_step_appends_and_attends(N, layer):
    """lrkv_decode_step at the 32-layer-step shapes: the appended rows meet the
    compress gate, the drawn rows are untouched, and the output is the
    oracle's decode over all N tokens (the new one included)."""
    w = synth.LLAMA_STEP
    B, H, d = w.batch, w.n_kv_heads, w.head_dim
    rk, rv = w.ranks(layer)
    xk = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(w, layer, "k", b, h, 1, synth.PART_APPEND)))
    xv = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(w, layer, "v", b, h, 1, synth.PART_APPEND)))
    bk, bv, q = synth.basis(w, layer, "k"), synth.basis(w, layer, "v"), synth.query(w, layer)
    ak = O.compress(xk.exact, bk.exact)
    av = O.compress(xv.exact, bv.exact)
    rows_k = np.zeros((B, H, N, rk))
    rows_v = np.zeros((B, H, N, rv))
    if N > 1:
        rows_k[:, :, :N - 1] = _direct_rows(w, layer, "k", N - 1).exact
        rows_v[:, :, :N - 1] = _direct_rows(w, layer, "v", N - 1).exact
    ck_all = rows_k.copy(); ck_all[:, :, N - 1:] = O.round_storage(ak, "bf16")
    cv_all = rows_v.copy(); cv_all[:, :, N - 1:] = O.round_storage(av, "bf16")
    o_ref, lse_ref = O.decode(q.exact, bk.exact, ck_all, bv.exact, cv_all, N)
    cap = max(8, (N + 7) // 8 * 8)
    ckd, cvd = _cache_from_rows(rows_k, rows_v, "bf16", cap)
    before_k = bits(ckd)
    qd, bkd, bvd = to_dev(q, "bf16"), to_dev(bk, "bf16"), to_dev(bv, "bf16")
    kn, vn = to_dev(xk, "bf16"), to_dev(xv, "bf16")
    o, lse = lrkv.decode_step(qd, kn, vn, bkd, ckd, bvd, cvd, N)
    torch.cuda.synchronize()
    check_compress(to_f64(ckd)[:, :, N - 1:N], ak, xk.exact, bk.exact, "bf16", "step append K")
    check_compress(synth.from_value_octets(to_f64(cvd))[:, :, N - 1:N], av, xv.exact, bv.exact, "bf16",
                   "step append V")
    after_k = bits(ckd)
    assert np.array_equal(after_k[:, :, :N - 1], before_k[:, :, :N - 1])
    assert np.array_equal(after_k[:, :, N:], before_k[:, :, N:])
    check_decode(to_f64(o), to_f64(lse), o_ref, lse_ref, "bf16", f"decode step N={N} layer={layer}")


@pytest.mark.parametrize("h_kv,N", [(8, 3000), (2, 1000), (1, 3000)])
def test_decode_step_two_phase_equals_one_call(h_kv, N):
    """lrkv_decode_step_partial + _merge give the bits of lrkv_decode_step,
    also on a workspace whose bytes all start at 0xFF (float NaN): the
    appended token's empty partial slot, whose output words the kernels never
    write, must weigh nothing in the merge whatever those words hold.  With
    one or two kv heads at batch 1 the one call is a launch small enough to
    merge its own partials (its last workgroup per kv head, device-scope
    stores and loads), against the two-phase merge launch."""
    w = synth.scaled(synth.LLAMA_STEP, n_kv_heads=h_kv, n_q_heads=4 * h_kv)
    layer = 1
    B, H, d = w.batch, w.n_kv_heads, w.head_dim
    rk, rv = w.ranks(layer)
    rows_k = np.zeros((B, H, N, rk)); rows_k[:, :, :N - 1] = _direct_rows(w, layer, "k", N - 1).exact
    rows_v = np.zeros((B, H, N, rv)); rows_v[:, :, :N - 1] = _direct_rows(w, layer, "v", N - 1).exact
    xk = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(w, layer, "k", b, h, 1, synth.PART_APPEND)))
    xv = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(w, layer, "v", b, h, 1, synth.PART_APPEND)))
    qd, bkd, bvd = (to_dev(x, "bf16") for x in (synth.query(w, layer), synth.basis(w, layer, "k"), synth.basis(w, layer, "v")))
    kn, vn = to_dev(xk, "bf16"), to_dev(xv, "bf16")
    ck1, cv1 = _cache_from_rows(rows_k, rows_v, "bf16", N)
    ck2, cv2 = ck1.clone(), cv1.clone()
    o1, l1 = lrkv.decode_step(qd, kn, vn, bkd, ck1, bvd, cv1, N)
    ws = torch.full((lrkv.decode_step_workspace_bytes(B, w.n_q_heads, H, d, rk, rv, N, N),), 0xFF,
                    dtype=torch.uint8, device=DEV)
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    lrkv.decode_step_partial(qd, kn, vn, bkd, ck2, bvd, cv2, N, ws)
    lrkv.decode_step_merge(o2, l2, N, ws, H, rk, rv, N)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    assert torch.equal(ck1.view(torch.int16), ck2.view(torch.int16))
    assert torch.equal(cv1.view(torch.int16), cv2.view(torch.int16))
    # one-call steps in a row on one zeroed workspace (appending the same token to
    # the same row again): the same bits each time, and the arrival counters
    # at the workspace's start are back at zero after each call
    wz = torch.zeros_like(ws)
    for _ in range(2):
        o3, l3 = lrkv.decode_step(qd, kn, vn, bkd, ck1, bvd, cv1, N, workspace=wz)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o3.view(torch.int16)) and torch.equal(l1, l3)
        assert not torch.any(wz[:4 * B * H]).item()


def test_decode_step_float32():
    """float32 caches take the compress kernel and the plain decode."""
    w = synth.TINY_F32
    rk, rv = w.ranks(0)
    N = 100
    rows_k = _direct_rows(w, 0, "k", N - 1).exact
    rows_v = _direct_rows(w, 0, "v", N - 1).exact
    xk = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(w, 0, "k", b, h, 1, synth.PART_APPEND)))
    xv = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(w, 0, "v", b, h, 1, synth.PART_APPEND)))
    bk, bv, q = synth.basis(w, 0, "k"), synth.basis(w, 0, "v"), synth.query(w, 0)
    ak, av = O.compress(xk.exact, bk.exact), O.compress(xv.exact, bv.exact)
    ck_all = np.concatenate([rows_k, O.round_storage(ak, "f32")], axis=2)
    cv_all = np.concatenate([rows_v, O.round_storage(av, "f32")], axis=2)
    o_ref, lse_ref = O.decode(q.exact, bk.exact, ck_all, bv.exact, cv_all, N)
    ckd, cvd = _cache_from_rows(rows_k, rows_v, "f32", 104)
    o, lse = lrkv.decode_step(to_dev(q, "f32"), to_dev(xk, "f32"), to_dev(xv, "f32"), to_dev(bk, "f32"), ckd,
                              to_dev(bv, "f32"), cvd, N)
    check_decode(to_f64(o), to_f64(lse), o_ref, lse_ref, "f32", "decode step f32")


def test_prefill_compress_tiles_and_ragged_tail():
    """A prefill chunk that spans several 64-token tiles, starts at an odd row and ends ragged."""
    w = synth.BATCHED_32K
    layer, T, pos, cap = 1, 333, 77, 512
    B = 2
    xk = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(w, layer, "k", b, h, T, synth.PART_PREFILL), batch=B))
    xv = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(w, layer, "v", b, h, T, synth.PART_PREFILL), batch=B))
    bk, bv = synth.basis(w, layer, "k"), synth.basis(w, layer, "v")
    rk, rv = w.ranks(layer)
    ck = torch.zeros((B, 8, cap, rk), dtype=torch.bfloat16, device=DEV)
    cv = torch.zeros(lrkv.value_cache_shape(B, 8, cap, rv), dtype=torch.bfloat16, device=DEV)
    lrkv.compress(to_dev(xk, "bf16"), to_dev(bk, "bf16"), ck, pos, values=False)
    lrkv.compress(to_dev(xv, "bf16"), to_dev(bv, "bf16"), cv, pos, values=True)
    torch.cuda.synchronize()
    gk = to_f64(ck)
    gv = synth.from_value_octets(to_f64(cv))
    check_compress(gk[:, :, pos:pos + T], O.compress(xk.exact, bk.exact), xk.exact, bk.exact, "bf16", "prefill K")
    check_compress(gv[:, :, pos:pos + T], O.compress(xv.exact, bv.exact), xv.exact, bv.exact, "bf16", "prefill V")
    # rows outside [pos, pos + T) stay zero
    assert not gk[:, :, :pos].any() and not gk[:, :, pos + T:].any()
    assert not gv[:, :, :pos].any() and not gv[:, :, pos + T:].any()


@pytest.mark.parametrize("T,pos", [(1, 255), (2, 8), (3, 61), (4, 100), (100, 13)])
def test_compress_kv_both_caches(T, pos):
    """The two-cache entry point: a few tokens in one launch, longer chunks per cache."""
    w = synth.LLAMA_STEP
    layer, cap, B = 0, 264, 2
    rk, rv = w.ranks(layer)
    xk = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(w, layer, "k", b, h, T, synth.PART_PREFILL), batch=B))
    xv = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(w, layer, "v", b, h, T, synth.PART_PREFILL), batch=B))
    bk, bv = synth.basis(w, layer, "k"), synth.basis(w, layer, "v")
    ck = torch.zeros((B, 8, cap, rk), dtype=torch.bfloat16, device=DEV)
    cv = torch.zeros(lrkv.value_cache_shape(B, 8, cap, rv), dtype=torch.bfloat16, device=DEV)
    lrkv.compress_kv(to_dev(xk, "bf16"), to_dev(xv, "bf16"), to_dev(bk, "bf16"), to_dev(bv, "bf16"), ck, cv, pos)
    torch.cuda.synchronize()
    gk = to_f64(ck)
    gv = synth.from_value_octets(to_f64(cv))
    check_compress(gk[:, :, pos:pos + T], O.compress(xk.exact, bk.exact), xk.exact, bk.exact, "bf16", "kv K")
    check_compress(gv[:, :, pos:pos + T], O.compress(xv.exact, bv.exact), xv.exact, bv.exact, "bf16", "kv V")
    assert not gk[:, :, :pos].any() and not gk[:, :, pos + T:].any()
    assert not gv[:, :, :pos].any() and not gv[:, :, pos + T:].any()
