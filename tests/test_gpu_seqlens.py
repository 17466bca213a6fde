"""Decode with the context lengths on the device (lrkv_decode_attn_seqlens,
lrkv_decode_step_seqlens): one captured HIP graph serves a decode that
advances, every sequence of the batch at its own length.

Checked against the oracle: a graph captured once and replayed while the
lengths advance (each replay appends a new token to every sequence and
attends its rows); sequences of different lengths in one call; lengths the
plan did not expect; lengths outside [1, capacity]; and, for one common
length planned for exactly, the same bits as the host-length entry points.
"""
import numpy as np
import pytest
import torch

import lrkv_synth as synth
from oracle import lrkv_oracle as O
from tests.gpu_helpers import DEV, bits, check_decode, to_dev, to_f64

pytestmark = pytest.mark.gpu
lrkv = pytest.importorskip("decode_attention_lrkv_amd")

NAN_BF16 = np.uint16(0x7FC0)


def _caches(w, layer, lens, cap):
    """Drawn rows [0, lens[b] - 1) of every sequence; NaN from there to cap
    (nothing past a sequence's length may be read)."""
    B, H = w.batch, w.n_kv_heads
    rk, rv = w.ranks(layer)
    ck = np.full((B, H, cap, rk), NAN_BF16, np.uint16)
    cv = np.full((B, H, cap, rv), NAN_BF16, np.uint16)
    exact_k, exact_v = {}, {}
    for b in range(B):
        n = max(lens[b] - 1, 0)
        for h in range(H):
            sk = synth.direct_coeffs(w, layer, "k", b, h, n)
            sv = synth.direct_coeffs(w, layer, "v", b, h, n)
            ck[b, h, :n] = sk.store
            cv[b, h, :n] = sv.store
            exact_k[(b, h)] = sk.exact
            exact_v[(b, h)] = sv.exact
    return ck, cv, exact_k, exact_v


def _tokens(w, layer, which, n):
    """n appended tokens of every (b, h): [B, n, Hkv, d] stored and exact."""
    return synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(w, layer, which, b, h, n,
                                                                                  synth.PART_APPEND)))


def test_graph_replays_an_advancing_decode():
    """Capture [decode_step_seqlens; seq_lens += 1] once; replay it R times
    with new queries and tokens.  Replay i appends token i of every sequence
    at row lens0[b] + i - 1 and attends lens0[b] + i rows; each replay is
    compared with the oracle's decode of the cache it builds itself."""
    w = synth.scaled(synth.LLAMA_STEP, batch=3)
    layer, R = 1, 4
    lens0 = [700, 2041, 33]
    cap = 2048
    B, Hq, H, d = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    rk, rv = w.ranks(layer)
    ck, cv, ek, ev = _caches(w, layer, lens0, cap)
    xk, xv = _tokens(w, layer, "k", R), _tokens(w, layer, "v", R)
    bk, bv = synth.basis(w, layer, "k"), synth.basis(w, layer, "v")
    qs = [synth.query(w, 40 + i) for i in range(R)]
    ckd, cvd = to_dev(ck, "bf16"), to_dev(synth.to_value_octets(cv), "bf16")
    bkd, bvd = to_dev(bk, "bf16"), to_dev(bv, "bf16")
    seq_lens = torch.tensor(lens0, dtype=torch.int32, device=DEV)
    q_buf = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=DEV)
    k_buf = torch.empty((B, H, d), dtype=torch.bfloat16, device=DEV)
    v_buf = torch.empty((B, H, d), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    ws = torch.zeros(lrkv.decode_step_workspace_bytes(B, Hq, H, d, rk, rv, cap, cap), dtype=torch.uint8, device=DEV)
    xk_dev, xv_dev = to_dev(xk, "bf16"), to_dev(xv, "bf16")

    def step():
        lrkv.decode_step_seqlens(q_buf, k_buf, v_buf, bkd, ckd, bvd, cvd, seq_lens, cap, out=out, lse=lse,
                                 workspace=ws)
        seq_lens.add_(1)

    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    # the oracle's appended rows: round(x B) of each token
    ak = O.round_storage(O.compress(xk.exact, bk.exact), "bf16")   # [B, H, R, rk]
    av = O.round_storage(O.compress(xv.exact, bv.exact), "bf16")
    for i in range(R):
        q_buf.copy_(to_dev(qs[i], "bf16"))
        k_buf.copy_(xk_dev[:, i])
        v_buf.copy_(xv_dev[:, i])
        g.replay()
        torch.cuda.synchronize()
        print(f"replay {i}: lengths {[n + i for n in lens0]}", flush=True)
        rows = [(b, hq) for b in range(B) for hq in range(Hq)]
        cks = {(b, h): np.concatenate([ek[(b, h)], ak[b, h, :i + 1]]) for b in range(B) for h in range(H)}
        cvs = {(b, h): np.concatenate([ev[(b, h)], av[b, h, :i + 1]]) for b in range(B) for h in range(H)}
        o_ref = np.zeros((B, Hq, d))
        lse_ref = np.zeros((B, Hq))
        for b in range(B):
            n = lens0[b] + i
            res = O.decode_rows(qs[i].exact, bk.exact, cks, bv.exact, cvs, n, [r for r in rows if r[0] == b])
            for (bb, hq), (o, l) in res.items():
                o_ref[bb, hq], lse_ref[bb, hq] = o, l
        check_decode(to_f64(out), to_f64(lse), o_ref, lse_ref, "bf16", f"advancing graph replay {i}")
    assert seq_lens.tolist() == [n + R for n in lens0]
    # the appended rows are the oracle's (within one bf16 step of the exact
    # coefficients), and nothing past the last appended row was written
    ckg = bits(ckd)
    cvg = synth.from_value_octets(bits(cvd))
    for b in range(B):
        n0 = lens0[b] - 1
        app_k = synth.bf16_bits_to_f64(ckg[b, :, n0:n0 + R])
        app_v = synth.bf16_bits_to_f64(cvg[b, :, n0:n0 + R])
        ex_k = O.compress(xk.exact[b:b + 1], bk.exact)[0]
        ex_v = O.compress(xv.exact[b:b + 1], bv.exact)[0]
        assert np.all(np.abs(app_k - ex_k) <= 2.0 ** -7 * np.abs(ex_k) + 1e-6)
        assert np.all(np.abs(app_v - ex_v) <= 2.0 ** -7 * np.abs(ex_v) + 1e-6)
        assert np.all(ckg[b, :, n0 + R:] == NAN_BF16) and np.all(cvg[b, :, n0 + R:] == NAN_BF16)
        assert np.array_equal(ckg[b, :, :n0], ck[b, :, :n0])


@pytest.mark.parametrize("max_seq_len", [64, 3000, 4096])
def test_per_sequence_lengths_and_any_plan(max_seq_len):
    """Plain decode with four sequences of different lengths in one call, for
    a plan made for far fewer tokens than some sequences hold (64: each
    workgroup takes more chunks), about as many, and the capacity."""
    w = synth.scaled(synth.LLAMA_STEP, batch=4)
    layer = 0
    lens = [1, 257, 3000, 4096]
    cap = 4096
    B, Hq, H = w.batch, w.n_q_heads, w.n_kv_heads
    # rows [0, n) attended: draw n rows (the "appended" row is a drawn row here)
    ck, cv, ek, ev = _caches(w, layer, [n + 1 for n in lens], cap)
    bk, bv, q = synth.basis(w, layer, "k"), synth.basis(w, layer, "v"), synth.query(w, layer)
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o, l = lrkv.decode_attn_seqlens(to_dev(q, "bf16"), to_dev(bk, "bf16"), to_dev(ck, "bf16"), to_dev(bv, "bf16"),
                                    to_dev(synth.to_value_octets(cv), "bf16"), seq_lens, max_seq_len)
    torch.cuda.synchronize()
    o_ref = np.zeros(o.shape)
    lse_ref = np.zeros(l.shape)
    for b in range(B):
        res = O.decode_rows(q.exact, bk.exact, ek, bv.exact, ev, lens[b], [(b, hq) for hq in range(Hq)])
        for (bb, hq), (oo, ll) in res.items():
            o_ref[bb, hq], lse_ref[bb, hq] = oo, ll
    check_decode(to_f64(o), to_f64(l), o_ref, lse_ref, "bf16", f"per-sequence lengths, plan {max_seq_len}")


def test_lengths_outside_the_cache_attend_nothing():
    """A length of 0 or above the capacity gives out = 0 and lse = -inf for
    that sequence and writes no row of its cache; the other sequences are
    decoded as usual."""
    w = synth.scaled(synth.LLAMA_STEP, batch=3)
    layer, cap = 0, 512
    lens = [0, cap + 5, 300]
    B, Hq, H, d = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    ck, cv, ek, ev = _caches(w, layer, [1, 1, 300], cap)
    xk, xv = _tokens(w, layer, "k", 1), _tokens(w, layer, "v", 1)
    bk, bv, q = synth.basis(w, layer, "k"), synth.basis(w, layer, "v"), synth.query(w, layer)
    ckd, cvd = to_dev(ck, "bf16"), to_dev(synth.to_value_octets(cv), "bf16")
    before_k, before_v = bits(ckd), bits(cvd)
    seq_lens = torch.tensor(lens, dtype=torch.int32, device=DEV)
    for max_seq_len in (300, cap):     # one attention workgroup per unit, and several
        ckd.copy_(to_dev(ck, "bf16"))
        cvd.copy_(to_dev(synth.to_value_octets(cv), "bf16"))
        o, l = lrkv.decode_step_seqlens(to_dev(q, "bf16"), to_dev(xk, "bf16")[:, 0].contiguous(),
                                        to_dev(xv, "bf16")[:, 0].contiguous(), to_dev(bk, "bf16"), ckd,
                                        to_dev(bv, "bf16"), cvd, seq_lens, max_seq_len)
        torch.cuda.synchronize()
        og, lg = to_f64(o), to_f64(l)
        assert np.all(og[:2] == 0.0) and np.all(np.isneginf(lg[:2])), f"plan {max_seq_len}"
        after_k, after_v = bits(ckd), bits(cvd)
        assert np.array_equal(after_k[:2], before_k[:2]) and np.array_equal(after_v[:2], before_v[:2])
        ak = O.round_storage(O.compress(xk.exact, bk.exact), "bf16")
        av = O.round_storage(O.compress(xv.exact, bv.exact), "bf16")
        cks = {(2, h): np.concatenate([ek[(2, h)], ak[2, h]]) for h in range(H)}
        cvs = {(2, h): np.concatenate([ev[(2, h)], av[2, h]]) for h in range(H)}
        res = O.decode_rows(q.exact, bk.exact, cks, bv.exact, cvs, 300, [(2, hq) for hq in range(Hq)])
        o_ref = np.stack([res[(2, hq)][0] for hq in range(Hq)])
        lse_ref = np.array([res[(2, hq)][1] for hq in range(Hq)])
        check_decode(og[2], lg[2], o_ref, lse_ref, "bf16", f"valid sequence beside invalid ones, plan {max_seq_len}")


@pytest.mark.parametrize("batch,N", [(16, 4096), (1, 300), (2, 8192)])
def test_planned_length_gives_the_host_length_bits(batch, N):
    """With every sequence at the length the plan is made for, the
    device-length calls launch what the host-length calls launch: the same
    bits (step: outputs, lse and both caches; plain decode: outputs, lse)."""
    w = synth.scaled(synth.BATCHED_32K, batch=batch)
    layer = 1
    B, Hq, H, d = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    cap = (N + 7) // 8 * 8
    ck, cv, _, _ = _caches(w, layer, [N] * B, cap)
    xk, xv = _tokens(w, layer, "k", 1), _tokens(w, layer, "v", 1)
    qd = to_dev(synth.query(w, layer), "bf16")
    bkd, bvd = to_dev(synth.basis(w, layer, "k"), "bf16"), to_dev(synth.basis(w, layer, "v"), "bf16")
    kn, vn = to_dev(xk, "bf16")[:, 0].contiguous(), to_dev(xv, "bf16")[:, 0].contiguous()
    ck1, cv1 = to_dev(ck, "bf16"), to_dev(synth.to_value_octets(cv), "bf16")
    ck2, cv2 = ck1.clone(), cv1.clone()
    seq_lens = torch.full((B,), N, dtype=torch.int32, device=DEV)
    o1, l1 = lrkv.decode_step(qd, kn, vn, bkd, ck1, bvd, cv1, N)
    o2, l2 = lrkv.decode_step_seqlens(qd, kn, vn, bkd, ck2, bvd, cv2, seq_lens, N)
    o3, l3 = lrkv.decode_attn(qd, bkd, ck1, bvd, cv1, N)
    o4, l4 = lrkv.decode_attn_seqlens(qd, bkd, ck1, bvd, cv1, seq_lens, N)
    torch.cuda.synchronize()
    same = lambda a, b: torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert same(o1, o2) and torch.equal(l1, l2)
    assert same(ck1, ck2) and same(cv1, cv2)
    assert same(o3, o4) and torch.equal(l3, l4)
