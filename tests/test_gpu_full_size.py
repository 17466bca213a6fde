"""Parity at the benchmark's full size, in the benchmark's launch configuration.

Also the two variants the benchmark times on the same caches: the latent
decode (absorbed projections) and the decode step with a separate key
encoder.

The batched 32K workload (batch 16, 32 query / 8 kv heads, d 128, context
32768, ranks (32, 96) on even and (48, 112) on odd layers): one layer of each
parity goes through exactly what a bench step runs (lrkv_compress_kv of the
4096-token prefill chunk, then lrkv_decode_step_partial + _merge with the
appended token), and every output row (all 16 x 32 (batch, q head) rows) is
checked against the oracle, computed one (batch, kv head) unit at a time on
the cache the oracle builds itself.  Every unit's cache is also compared row
by row: the drawn rows untouched, the prefill rows and the appended row
within the compress gate.
"""
import math

import numpy as np
import pytest
import torch

import lrkv_synth as synth
from oracle import lrkv_oracle as O
from tests.gpu_helpers import DEV, bits, check_decode, to_dev, to_f64
from tests.test_gpu_parity_small import check_compress

pytestmark = pytest.mark.gpu

lrkv = pytest.importorskip("decode_attention_lrkv_amd")

W = synth.BATCHED_32K


@pytest.mark.parametrize("layer", [0, 1])
def test_bench_layer_step_full_size(layer):
    B, Hq, H, d = W.batch, W.n_q_heads, W.n_kv_heads, W.head_dim
    N, P = W.n_ctx[0], W.prefill
    p0 = N - 1 - P
    rk, rv = W.ranks(layer)
    g = W.group
    print(f"[full-size] layer {layer}: B {B}, N {N}, ranks {rk}/{rv}, prefill rows [{p0}, {N - 1})", flush=True)

    ck_rows = synth.stack_heads(W, lambda b, h: synth.direct_coeffs(W, layer, "k", b, h, p0, exact=False))
    cv_rows = synth.stack_heads(W, lambda b, h: synth.direct_coeffs(W, layer, "v", b, h, p0, exact=False))
    xk = synth.tokens_major(synth.stack_heads(W, lambda b, h: synth.full_tokens(W, layer, "k", b, h, P,
                                                                               synth.PART_PREFILL)))
    xv = synth.tokens_major(synth.stack_heads(W, lambda b, h: synth.full_tokens(W, layer, "v", b, h, P,
                                                                               synth.PART_PREFILL)))
    ak = synth.tokens_major(synth.stack_heads(W, lambda b, h: synth.full_tokens(W, layer, "k", b, h, 1,
                                                                               synth.PART_APPEND)))
    av = synth.tokens_major(synth.stack_heads(W, lambda b, h: synth.full_tokens(W, layer, "v", b, h, 1,
                                                                               synth.PART_APPEND)))
    bk, bv, q = synth.basis(W, layer, "k"), synth.basis(W, layer, "v"), synth.query(W, layer)

    kc = np.zeros((B, H, N, rk), np.uint16)
    vc = np.zeros((B, H, N, rv), np.uint16)
    kc[:, :, :p0] = ck_rows.store
    vc[:, :, :p0] = cv_rows.store
    ckd, cvd = to_dev(kc, "bf16"), to_dev(synth.to_value_octets(vc), "bf16")
    del vc
    bkd, bvd, qd = to_dev(bk, "bf16"), to_dev(bv, "bf16"), to_dev(q, "bf16")
    # the bench's launch sequence: prefill compress, then the two phases of the decode step
    lrkv.compress_kv(to_dev(xk, "bf16"), to_dev(xv, "bf16"), bkd, bvd, ckd, cvd, p0)
    ws = torch.zeros(lrkv.decode_step_workspace_bytes(B, Hq, H, d, rk, rv, N, N), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    lrkv.decode_step_partial(qd, to_dev(ak, "bf16"), to_dev(av, "bf16"), bkd, ckd, bvd, cvd, N, ws)
    lrkv.decode_step_merge(out, lse, N, ws, H, rk, rv, N)
    torch.cuda.synchronize()
    ck_gpu = bits(ckd)
    cv_gpu = synth.from_value_octets(bits(cvd))
    o_gpu, lse_gpu = to_f64(out), to_f64(lse)
    # the two variants the bench times on these caches: the latent decode of
    # absorbed projections over all N rows, and the decode step with a
    # separate (non-orthogonal) key encoder, whose decoder folds the query
    q_lat = synth.latent_query(W, layer)
    o_lat, lse_lat = lrkv.decode_attn_latent(to_dev(q_lat, "bf16"), ckd, cvd, N, d)
    enc, dec = synth.key_transform(W, layer, "k")
    ck_t, cv_t = ckd.clone(), cvd.clone()
    out_t = torch.empty_like(out)
    lse_t = torch.empty_like(lse)
    lrkv.decode_step(qd, to_dev(ak, "bf16"), to_dev(av, "bf16"), to_dev(dec, "bf16"), ck_t, bvd, cv_t, N,
                     out=out_t, lse=lse_t, workspace=ws, enc_k=to_dev(enc, "bf16"))
    torch.cuda.synchronize()
    o_lat, lse_lat, o_t, lse_t = to_f64(o_lat), to_f64(lse_lat), to_f64(out_t), to_f64(lse_t)
    ck_t_bits = bits(ck_t)
    del ckd, cvd, ws, ck_t, cv_t

    # oracle, one (batch, kv head) unit at a time, on the cache it builds
    # itself: drawn rows, its own rounded compress of the prefill chunk and of
    # the new token; all g query heads of the unit, for the plain step, the
    # latent decode and the key-encoder step
    o_ref = np.zeros((B, Hq, d))
    lse_ref = np.zeros((B, Hq))
    lat_ref = np.zeros(o_lat.shape)
    lat_lse = np.zeros((B, Hq))
    t_ref = np.zeros((B, Hq, d))
    t_lse = np.zeros((B, Hq))
    for b in range(B):
        for h in range(H):
            pk = O.round_storage(O.compress(xk.exact[b:b + 1, :, h:h + 1], bk.exact[h:h + 1]), "bf16")[0, 0]
            pv = O.round_storage(O.compress(xv.exact[b:b + 1, :, h:h + 1], bv.exact[h:h + 1]), "bf16")[0, 0]
            nk = O.round_storage(O.compress(ak.exact[b:b + 1, :, h:h + 1], bk.exact[h:h + 1]), "bf16")[0, 0]
            nv = O.round_storage(O.compress(av.exact[b:b + 1, :, h:h + 1], bv.exact[h:h + 1]), "bf16")[0, 0]
            drawn_k = synth.bf16_bits_to_f64(ck_rows.store[b, h])     # the generator's rows, as drawn
            drawn_v = synth.bf16_bits_to_f64(cv_rows.store[b, h])
            ck_u = np.concatenate([drawn_k, pk, nk])
            cv_u = np.concatenate([drawn_v, pv, nv])
            # the cache rows of this unit on the GPU
            assert np.array_equal(ck_gpu[b, h, :p0], kc[b, h, :p0]), f"drawn key rows changed at {(b, h)}"
            assert np.array_equal(cv_gpu[b, h, :p0], cv_rows.store[b, h]), f"drawn value rows changed at {(b, h)}"
            gk = synth.bf16_bits_to_f64(ck_gpu[b, h, p0:])[None, None]
            gv = synth.bf16_bits_to_f64(cv_gpu[b, h, p0:])[None, None]
            xk_u = np.concatenate([xk.exact[b:b + 1, :, h:h + 1], ak.exact[b:b + 1, :, h:h + 1]], axis=1)
            xv_u = np.concatenate([xv.exact[b:b + 1, :, h:h + 1], av.exact[b:b + 1, :, h:h + 1]], axis=1)
            check_compress(gk, O.compress(xk_u, bk.exact[h:h + 1]), xk_u, bk.exact[h:h + 1], "bf16",
                           f"K rows {(b, h)}")
            check_compress(gv, O.compress(xv_u, bv.exact[h:h + 1]), xv_u, bv.exact[h:h + 1], "bf16",
                           f"V rows {(b, h)}")
            rows = [(b, h * g + j) for j in range(g)]
            ref = O.decode_rows(q.exact, bk.exact, {(b, h): ck_u}, bv.exact, {(b, h): cv_u}, N, rows)
            # latent decode on the same cache rows
            o_l, l_l = O.decode_latent(q_lat.exact[b:b + 1, h * g:(h + 1) * g], ck_u[None, None], cv_u[None, None],
                                       N, 1 / math.sqrt(d))
            # key-encoder step: rows [0, N - 1) as before, the new row round(k E), read through D
            ek = O.compress(ak.exact[b:b + 1, :, h:h + 1], enc.exact[h:h + 1])
            check_compress(synth.bf16_bits_to_f64(ck_t_bits[b, h, N - 1:N])[None, None], ek,
                           ak.exact[b:b + 1, :, h:h + 1], enc.exact[h:h + 1], "bf16", f"encoder row {(b, h)}")
            ck_t_u = np.concatenate([ck_u[:N - 1], O.round_storage(ek, "bf16")[0, 0]])
            ref_t = O.decode_rows(q.exact, dec.exact, {(b, h): ck_t_u}, bv.exact, {(b, h): cv_u}, N, rows)
            for j, (bb, hq) in enumerate(rows):
                o_ref[bb, hq], lse_ref[bb, hq] = ref[(bb, hq)]
                t_ref[bb, hq], t_lse[bb, hq] = ref_t[(bb, hq)]
                lat_ref[bb, hq], lat_lse[bb, hq] = o_l[0, j], l_l[0, j]
    worst = check_decode(o_gpu, lse_gpu, o_ref, lse_ref, "bf16", f"full-size layer {layer}")
    print(f"[full-size] layer {layer}: worst row error over all {B * Hq} rows {worst:.3e} (gate 2e-2)", flush=True)
    assert math.isfinite(worst)
    w_lat = check_decode(o_lat, lse_lat, lat_ref, lat_lse, "bf16", f"full-size latent layer {layer}",
                         storage_rounding=True)
    w_t = check_decode(o_t, lse_t, t_ref, t_lse, "bf16", f"full-size key-encoder step layer {layer}")
    print(f"[full-size] layer {layer}: latent {w_lat:.3e}, key-encoder step {w_t:.3e}", flush=True)
