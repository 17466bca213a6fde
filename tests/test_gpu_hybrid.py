"""GPU parity of the hybrid (OjaKV-style) cache: selection, compaction and union decode.

Selection is compared bit for bit (flags, counts, side-list indices, side
rows); coefficients within the compress gate; decode within the bfloat16
decode gate, on the oracle's cache contents and end to end.
"""
import math

import numpy as np
import pytest
import torch

import lrkv_synth as synth
from oracle import lrkv_oracle as O
from tests.gpu_helpers import DEV, bits, check_decode, round_store, to_dev, to_f64
from tests.test_gpu_parity_small import check_compress

pytestmark = pytest.mark.gpu
lrkv = pytest.importorskip("decode_attention_lrkv_amd")

TAU = 0.5


def _round8(x):
    return (x + 7) // 8 * 8


def _inputs(n):
    w = synth.scaled(synth.HYBRID_128K, n_ctx=(n,))
    inj = synth.injected_set(w, 0, 0, n)
    k = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.hybrid_tokens(w, 0, "k", b, h, n, inj)))
    v = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.hybrid_tokens(w, 0, "v", b, h, n, inj)))
    return w, inj, k, v, synth.basis(w, 0, "k"), synth.basis(w, 0, "v"), synth.query(w, 0)


def _new_cache(w, cap, side_cap):
    return lrkv.HybridCache(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, *w.ranks(0), cap, side_cap, DEV)


def _snapshot(c):
    torch.cuda.synchronize()
    return {name: bits(getattr(c, name)) for name in
            ("coeff_k", "coeff_v", "k_side", "v_side", "side_idx", "n_lr", "n_side", "overflow")}


def _valid_parts(snap, b, h):
    n_lr, n_side = int(snap["n_lr"][b, h]), int(snap["n_side"][b, h])
    return dict(
        ck=snap["coeff_k"][b, h, :n_lr],
        cv=synth.from_value_octets(snap["coeff_v"][b, h])[:n_lr],
        ks=snap["k_side"][b, h, :n_side],
        vs=synth.from_value_octets(snap["v_side"][b, h])[:n_side],
        idx=snap["side_idx"][b, h, :n_side])


# 150000 tokens are 9375 sub-tiles: the counter scan runs two rounds of 8192
@pytest.mark.parametrize("n", [8192, 131072, 150000])
def test_hybrid_selection_compaction_and_decode(n):
    w, inj, k, v, bk, bv, q = _inputs(n)
    H, d = w.n_kv_heads, w.head_dim
    cap = _round8(n)
    side_cap = _round8(int(math.ceil(0.06 * n)))
    ref = O.compress_hybrid(k.exact, v.exact, bk.exact, bv.exact, TAU, "bf16")

    # --- one call
    c1 = _new_cache(w, cap, side_cap)
    flags = torch.zeros((1, H, n), dtype=torch.uint8, device=DEV)
    kd, vd, bkd, bvd = to_dev(k, "bf16"), to_dev(v, "bf16"), to_dev(bk, "bf16"), to_dev(bv, "bf16")
    lrkv.compress_hybrid(c1, kd, vd, bkd, bvd, TAU, 0, flags=flags)
    s1 = _snapshot(c1)
    fl = flags.cpu().numpy()
    assert s1["overflow"][0] == 0
    for h in range(H):
        f_ref = ref["flags"][(0, h)]
        assert np.array_equal(fl[0, h].astype(bool), f_ref), f"flags differ at head {h}"
        assert np.array_equal(np.nonzero(f_ref)[0], inj)      # the injected tokens, exactly
        part = _valid_parts(s1, 0, h)
        assert s1["n_side"][0, h] == f_ref.sum() and s1["n_lr"][0, h] == n - f_ref.sum()
        assert np.array_equal(part["idx"], ref["side_idx"][(0, h)])
        side = np.nonzero(f_ref)[0]
        lr = np.nonzero(~f_ref)[0]
        assert np.array_equal(part["ks"], k.store[0, side, h])      # bit-identical copies
        assert np.array_equal(part["vs"], v.store[0, side, h])
        ck_gpu = synth.bf16_bits_to_f64(part["ck"])[None, None]
        cv_gpu = synth.bf16_bits_to_f64(part["cv"])[None, None]
        check_compress(ck_gpu, ref["ck"][(0, h)][None, None], k.exact[:, lr, h:h + 1], bk.exact[h:h + 1],
                       "bf16", f"hybrid K h={h}")
        check_compress(cv_gpu, ref["cv"][(0, h)][None, None], v.exact[:, lr, h:h + 1], bv.exact[h:h + 1],
                       "bf16", f"hybrid V h={h}")

    # --- the same tokens in 4096-token chunks give identical caches
    c2 = _new_cache(w, cap, side_cap)
    for p in range(0, n, 4096):
        e = min(n, p + 4096)
        lrkv.compress_hybrid(c2, kd[:, p:e].contiguous(), vd[:, p:e].contiguous(), bkd, bvd, TAU, p)
    s2 = _snapshot(c2)
    for h in range(H):
        a, b_ = _valid_parts(s1, 0, h), _valid_parts(s2, 0, h)
        for key in a:
            assert np.array_equal(a[key], b_[key]), f"chunked compress differs in {key} at head {h}"

    # --- decode: every (batch, q head) row against the oracle's union attention
    rows = [(0, hq) for hq in range(w.n_q_heads)]
    ck_st = {key: O.round_storage(c, "bf16") for key, c in ref["ck"].items()}
    cv_st = {key: O.round_storage(c, "bf16") for key, c in ref["cv"].items()}
    o_ref = O.decode_hybrid_rows(q.exact, bk.exact, bv.exact, ck_st, cv_st, ref["k_side"], ref["v_side"], rows)
    o_ref_arr = np.stack([o_ref[r][0] for r in rows])
    lse_ref = np.array([o_ref[r][1] for r in rows])
    qd = to_dev(q, "bf16")
    # (iii) end to end on the GPU-built cache
    o, lse = lrkv.decode_attn_hybrid(qd, bkd, bvd, c1)
    og, lg = to_f64(o), to_f64(lse)
    check_decode(np.stack([og[r] for r in rows]), np.array([lg[r] for r in rows]), o_ref_arr, lse_ref,
                 "bf16", f"hybrid e2e n={n}")
    # (ii) on the oracle's cache contents
    c3 = _new_cache(w, cap, side_cap)
    ckb = np.zeros((1, H, cap, w.ranks(0)[0]), np.uint16)
    cvb = np.zeros((1, H, cap, w.ranks(0)[1]), np.uint16)
    ksb = np.zeros((1, H, side_cap, d), np.uint16)
    vsb = np.zeros((1, H, side_cap, d), np.uint16)
    for h in range(H):
        nl = len(ck_st[(0, h)])
        ckb[0, h, :nl] = round_store(ck_st[(0, h)], "bf16")
        cvb[0, h, :nl] = round_store(cv_st[(0, h)], "bf16")
        ns = len(ref["k_side"][(0, h)])
        ksb[0, h, :ns] = round_store(ref["k_side"][(0, h)], "bf16")
        vsb[0, h, :ns] = round_store(ref["v_side"][(0, h)], "bf16")
    c3.coeff_k.copy_(to_dev(ckb, "bf16"))
    c3.coeff_v.copy_(to_dev(synth.to_value_octets(cvb), "bf16"))
    c3.k_side.copy_(to_dev(ksb, "bf16"))
    c3.v_side.copy_(to_dev(synth.to_value_octets(vsb), "bf16"))
    c3.n_lr.copy_(torch.tensor([[len(ck_st[(0, h)]) for h in range(H)]], dtype=torch.int32))
    c3.n_side.copy_(torch.tensor([[len(ref["k_side"][(0, h)]) for h in range(H)]], dtype=torch.int32))
    o, lse = lrkv.decode_attn_hybrid(qd, bkd, bvd, c3)
    og, lg = to_f64(o), to_f64(lse)
    check_decode(np.stack([og[r] for r in rows]), np.array([lg[r] for r in rows]), o_ref_arr, lse_ref,
                 "bf16", f"hybrid on oracle cache n={n}")


def test_hybrid_side_list_overflow():
    n = 2048
    w, inj, k, v, bk, bv, q = _inputs(n)
    c = _new_cache(w, n, 16)
    lrkv.compress_hybrid(c, to_dev(k, "bf16"), to_dev(v, "bf16"), to_dev(bk, "bf16"), to_dev(bv, "bf16"), TAU, 0)
    s = _snapshot(c)
    assert s["overflow"][0] == 1
    ref = O.compress_hybrid(k.exact, v.exact, bk.exact, bv.exact, TAU, "bf16")
    for h in range(w.n_kv_heads):
        assert s["n_side"][0, h] == 16
        # the first 16 selected tokens, in order, are the ones kept
        assert np.array_equal(s["side_idx"][0, h, :16], ref["side_idx"][(0, h)][:16])
        assert s["n_lr"][0, h] == n - ref["flags"][(0, h)].sum()


def test_hybrid_empty_cache_gives_zero_and_minus_inf():
    w = synth.scaled(synth.HYBRID_128K, n_ctx=(64,))
    c = _new_cache(w, 64, 8)
    q = to_dev(synth.query(w, 0), "bf16")
    o, lse = lrkv.decode_attn_hybrid(q, to_dev(synth.basis(w, 0, "k"), "bf16"), to_dev(synth.basis(w, 0, "v"), "bf16"), c)
    assert torch.all(o == 0).item()
    assert torch.all(torch.isneginf(lse)).item()


def test_hybrid_tau_inf_matches_plain_decode():
    """tau = +inf keeps every token low rank: the hybrid decode equals the plain decode."""
    n = 1000
    w, inj, k, v, bk, bv, q = _inputs(n)
    c = _new_cache(w, 1000, 8)
    kd, vd, bkd, bvd, qd = (to_dev(x, "bf16") for x in (k, v, bk, bv, q))
    lrkv.compress_hybrid(c, kd, vd, bkd, bvd, math.inf, 0)
    torch.cuda.synchronize()
    assert c.n_lr.cpu().eq(n).all() and c.n_side.cpu().eq(0).all()
    o1, l1 = lrkv.decode_attn_hybrid(qd, bkd, bvd, c)
    o2, l2 = lrkv.decode_attn(qd, bkd, c.coeff_k, bvd, c.coeff_v, n)
    assert np.max(np.abs(to_f64(o1) - to_f64(o2))) <= 2 * 2 ** -8 * np.max(np.abs(to_f64(o2)))
    assert np.max(np.abs(to_f64(l1) - to_f64(l2))) <= 1e-4


@pytest.mark.parametrize("batch,hq,hkv,d,rk,rv,n", [
    (2, 8, 2, 64, 16, 40, 3001),       # head_dim 64, unequal ranks, ragged sub-tile
    (1, 8, 2, 128, 56, 72, 5000),      # the step workload's ranks
    (1, 4, 1, 128, 128, 32, 777),      # full-rank keys, narrow values
])
def test_hybrid_other_shapes(batch, hq, hkv, d, rk, rv, n):
    """Selection, compaction and union decode at shapes other than the 128K workload's."""
    w = synth.scaled(synth.HYBRID_128K, batch=batch, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                     ranks_even=(rk, rv), ranks_odd=(rk, rv), n_ctx=(n,))
    inj = synth.injected_set(w, 0, 0, n)
    k = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.hybrid_tokens(w, 0, "k", b, h, n, inj)))
    v = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.hybrid_tokens(w, 0, "v", b, h, n, inj)))
    bk, bv, q = synth.basis(w, 0, "k"), synth.basis(w, 0, "v"), synth.query(w, 0)
    ref = O.compress_hybrid(k.exact, v.exact, bk.exact, bv.exact, TAU, "bf16")
    # the decision is unique: every token's residual is far from the threshold
    for b in range(batch):
        for h in range(hkv):
            for x, bs in ((k.exact[b, :, h], bk.exact[h]), (v.exact[b, :, h], bv.exact[h])):
                e = O.relative_residual(x, bs)
                assert not np.any((e > 0.25) & (e < 0.75))
    cap = _round8(n)
    side_cap = _round8(len(inj) + 8)
    c = lrkv.HybridCache(batch, hq, hkv, d, rk, rv, cap, side_cap, DEV)
    flags = torch.zeros((batch, hkv, n), dtype=torch.uint8, device=DEV)
    kd, vd, bkd, bvd, qd = (to_dev(x, "bf16") for x in (k, v, bk, bv, q))
    lrkv.compress_hybrid(c, kd, vd, bkd, bvd, TAU, 0, flags=flags)
    s = _snapshot(c)
    fl = flags.cpu().numpy()
    assert s["overflow"][0] == 0
    for b in range(batch):
        for h in range(hkv):
            f_ref = ref["flags"][(b, h)]
            assert np.array_equal(fl[b, h].astype(bool), f_ref), f"flags differ at ({b}, {h})"
            part = _valid_parts(s, b, h)
            assert np.array_equal(part["idx"], ref["side_idx"][(b, h)])
            side, lr = np.nonzero(f_ref)[0], np.nonzero(~f_ref)[0]
            assert np.array_equal(part["ks"], k.store[b, side, h])
            assert np.array_equal(part["vs"], v.store[b, side, h])
            check_compress(synth.bf16_bits_to_f64(part["ck"])[None, None], ref["ck"][(b, h)][None, None],
                           k.exact[b:b + 1, lr, h:h + 1], bk.exact[h:h + 1], "bf16", f"K ({b}, {h})")
            check_compress(synth.bf16_bits_to_f64(part["cv"])[None, None], ref["cv"][(b, h)][None, None],
                           v.exact[b:b + 1, lr, h:h + 1], bv.exact[h:h + 1], "bf16", f"V ({b}, {h})")
    rows = [(b, hq_) for b in range(batch) for hq_ in range(hq)]
    ck_st = {key: O.round_storage(x, "bf16") for key, x in ref["ck"].items()}
    cv_st = {key: O.round_storage(x, "bf16") for key, x in ref["cv"].items()}
    o_ref = O.decode_hybrid_rows(q.exact, bk.exact, bv.exact, ck_st, cv_st, ref["k_side"], ref["v_side"], rows)
    o, lse = lrkv.decode_attn_hybrid(qd, bkd, bvd, c)
    og, lg = to_f64(o), to_f64(lse)
    check_decode(np.stack([og[r] for r in rows]), np.array([lg[r] for r in rows]),
                 np.stack([o_ref[r][0] for r in rows]), np.array([o_ref[r][1] for r in rows]),
                 "bf16", f"hybrid shape {(batch, hq, hkv, d, rk, rv, n)}")


def test_hybrid_decode_uneven_counts_per_unit():
    """Each (b, kv head) divides its workgroups between the two lists from its
    own counts on the device: counts that differ per unit, lists that are
    empty on one side or on both, and a side list much shorter than its
    capacity all give the oracle's union softmax."""
    w = synth.scaled(synth.HYBRID_128K, batch=2, n_q_heads=16, n_kv_heads=4, n_ctx=(8192,))
    B, Hq, H, d = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    rk, rv = w.ranks(0)
    cap, side_cap = 8192, 2048
    n_lr = np.array([[0, 8192, 33, 4096], [1, 0, 7001, 100]], np.int32)
    n_side = np.array([[64, 0, 1000, 9], [0, 0, 300, 2048]], np.int32)
    ck = synth.stack_heads(w, lambda b, h: synth.direct_coeffs(w, 0, "k", b, h, cap))
    cv = synth.stack_heads(w, lambda b, h: synth.direct_coeffs(w, 0, "v", b, h, cap))
    ks = synth.stack_heads(w, lambda b, h: synth.full_tokens(w, 0, "k", b, h, side_cap, synth.PART_PREFILL))
    vs = synth.stack_heads(w, lambda b, h: synth.full_tokens(w, 0, "v", b, h, side_cap, synth.PART_PREFILL))
    bk, bv, q = synth.basis(w, 0, "k"), synth.basis(w, 0, "v"), synth.query(w, 0)
    c = lrkv.HybridCache(B, Hq, H, d, rk, rv, cap, side_cap, DEV)
    c.coeff_k.copy_(to_dev(ck, "bf16"))
    c.coeff_v.copy_(to_dev(synth.to_value_octets(cv.store), "bf16").view(c.coeff_v.shape))
    c.k_side.copy_(to_dev(ks, "bf16"))
    c.v_side.copy_(to_dev(synth.to_value_octets(vs.store), "bf16").view(c.v_side.shape))
    c.n_lr.copy_(torch.from_numpy(n_lr))
    c.n_side.copy_(torch.from_numpy(n_side))
    bkd, bvd, qd = (to_dev(x, "bf16") for x in (bk, bv, q))
    o, lse = lrkv.decode_attn_hybrid(qd, bkd, bvd, c)
    og, lg = to_f64(o), to_f64(lse)
    g = Hq // H
    rows = [(b, hq) for b in range(B) for hq in range(Hq) if n_lr[b, hq // g] + n_side[b, hq // g] > 0]
    empty = [(b, hq) for b in range(B) for hq in range(Hq) if n_lr[b, hq // g] + n_side[b, hq // g] == 0]
    keys = [(b, h) for b in range(B) for h in range(H)]
    o_ref = O.decode_hybrid_rows(q.exact, bk.exact, bv.exact,
                                 {k: ck.exact[k][:n_lr[k]] for k in keys}, {k: cv.exact[k][:n_lr[k]] for k in keys},
                                 {k: ks.exact[k][:n_side[k]] for k in keys}, {k: vs.exact[k][:n_side[k]] for k in keys},
                                 rows)
    check_decode(np.stack([og[r] for r in rows]), np.array([lg[r] for r in rows]),
                 np.stack([o_ref[r][0] for r in rows]), np.array([o_ref[r][1] for r in rows]),
                 "bf16", "hybrid uneven counts")
    assert empty and all(np.all(og[r] == 0) and np.isneginf(lg[r]) for r in empty)


def test_hybrid_tau_zero_keeps_every_token_full_rank():
    """tau = 0 flags every token with a residual off the basis span (here all
    of them: full-spectrum tokens leave about 2% of their energy off a rank-64
    span): nothing is low rank and the hybrid decode is dense attention over
    the bfloat16 keys and values."""
    n = 1500
    w = synth.scaled(synth.HYBRID_128K, n_ctx=(n,))
    k = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(w, 0, "k", b, h, n, synth.PART_PREFILL)))
    v = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(w, 0, "v", b, h, n, synth.PART_PREFILL)))
    bk, bv, q = synth.basis(w, 0, "k"), synth.basis(w, 0, "v"), synth.query(w, 0)
    assert min(O.relative_residual(x[0, :, h], b_.exact[h]).min() for x, b_ in ((k.exact, bk), (v.exact, bv))
               for h in range(w.n_kv_heads)) > 0.05
    c = _new_cache(w, n + 4, _round8(n))
    kd, vd, bkd, bvd, qd = (to_dev(x, "bf16") for x in (k, v, bk, bv, q))
    lrkv.compress_hybrid(c, kd, vd, bkd, bvd, 0.0, 0)
    torch.cuda.synchronize()
    assert c.n_lr.cpu().eq(0).all() and c.n_side.cpu().eq(n).all()
    o, lse = lrkv.decode_attn_hybrid(qd, bkd, bvd, c)
    H, g = w.n_kv_heads, w.n_q_heads // w.n_kv_heads
    rows = [(0, hq) for hq in range(w.n_q_heads)]
    empty = np.zeros((0, bk.exact.shape[2]))
    o_ref = O.decode_hybrid_rows(q.exact, bk.exact, bv.exact, {(0, h): empty for h in range(H)},
                                 {(0, h): np.zeros((0, bv.exact.shape[2])) for h in range(H)},
                                 {(0, h): k.exact[0, :, h] for h in range(H)},
                                 {(0, h): v.exact[0, :, h] for h in range(H)}, rows)
    og, lg = to_f64(o), to_f64(lse)
    check_decode(np.stack([og[r] for r in rows]), np.array([lg[r] for r in rows]),
                 np.stack([o_ref[r][0] for r in rows]), np.array([o_ref[r][1] for r in rows]),
                 "bf16", "hybrid tau = 0")


def test_hybrid_decode_shares_one_workspace_and_replays_in_a_graph():
    """Calls on two caches that share one workspace give the bits of calls
    with fresh workspaces, and a captured call replays to the eager bits with
    eager calls on the same workspace between the replays."""
    w, inj, k, v, bk, bv, q = _inputs(3000)
    kd, vd, bkd, bvd, qd = (to_dev(x, "bf16") for x in (k, v, bk, bv, q))
    caches = []
    for n in (3000, 1234):
        c = _new_cache(w, 3000, _round8(len(inj) + 8))
        lrkv.compress_hybrid(c, kd[:, :n].contiguous(), vd[:, :n].contiguous(), bkd, bvd, TAU, 0)
        caches.append(c)
    fresh = [lrkv.decode_attn_hybrid(qd, bkd, bvd, c) for c in caches]
    need = lrkv.decode_workspace_bytes(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, *w.ranks(0), 3000, 0,
                                       caches[0].side_cap)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for rep in range(3):
        for c, (o_ref, l_ref) in zip(caches, fresh):
            o, lse = lrkv.decode_attn_hybrid(qd, bkd, bvd, c, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(lse, l_ref)
            # the in-launch merge's arrival counters (one word per (b, kv head)
            # at the workspace's start) are back at zero after every call
            assert not torch.any(ws[:4 * w.batch * w.n_kv_heads]).item()
    out = torch.empty_like(qd)
    lse = torch.empty((w.batch, w.n_q_heads), dtype=torch.float32, device=DEV)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        lrkv.decode_attn_hybrid(qd, bkd, bvd, caches[0], out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lrkv.decode_attn_hybrid(qd, bkd, bvd, caches[0], out=out, lse=lse, workspace=ws)
    for rep in range(3):
        out.zero_()
        lse.zero_()
        lrkv.decode_attn_hybrid(qd, bkd, bvd, caches[1], workspace=ws)   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), fresh[0][0].view(torch.int16)) and torch.equal(lse, fresh[0][1])
