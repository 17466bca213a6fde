"""GPU edge cases: ragged and tiny contexts, garbage past the context, forced
split counts, rank and group shapes, needles, determinism, graph replay."""
import math
import os

import numpy as np
import pytest
import torch

import lrkv_synth as synth
from oracle import lrkv_oracle as O
from tests.gpu_helpers import DEV, bits, check_decode, round_store, to_dev, to_f64
from tests.test_gpu_parity_small import check_compress

pytestmark = pytest.mark.gpu
lrkv = pytest.importorskip("decode_attention_lrkv_amd")

NAN_BF16 = np.uint16(0x7FC0)


def _case(seed, B=2, Hq=8, Hkv=2, d=128, rk=48, rv=72, n=200, dtype="bf16", cap=None, scale_q=1.0):
    """Random orthonormal bases and coefficient rows; the cache past n holds NaN."""
    rng = np.random.default_rng(seed)
    cap = cap or (n + 7) // 8 * 8 + 8

    def ortho(r):
        qm, rr = np.linalg.qr(rng.standard_normal((d, d)))
        return (qm * np.sign(np.diag(rr)))[:, :r]

    bk = np.stack([ortho(rk) for _ in range(Hkv)])
    bv = np.stack([ortho(rv) for _ in range(Hkv)])
    ck = rng.standard_normal((B, Hkv, n, rk)) * 0.97 ** np.arange(rk)
    cv = rng.standard_normal((B, Hkv, n, rv)) * 0.97 ** np.arange(rv)
    q = rng.standard_normal((B, Hq, d)) * scale_q
    st = lambda x: round_store(x, dtype)
    ex = lambda a: synth.bf16_bits_to_f64(a) if dtype == "bf16" else np.asarray(a, np.float64)
    bk_s, bv_s, q_s = st(bk), st(bv), st(q)
    ckb = np.full((B, Hkv, cap, rk), NAN_BF16 if dtype == "bf16" else np.float32(np.nan),
                  np.uint16 if dtype == "bf16" else np.float32)
    cvb = np.full((B, Hkv, cap, rv), NAN_BF16 if dtype == "bf16" else np.float32(np.nan),
                  np.uint16 if dtype == "bf16" else np.float32)
    ckb[:, :, :n] = st(ck)
    cvb[:, :, :n] = st(cv)
    ref = O.decode(ex(q_s), ex(bk_s), ex(ckb[:, :, :n]), ex(bv_s), ex(cvb[:, :, :n]), n)
    dev = dict(q=to_dev(q_s, dtype), bk=to_dev(bk_s, dtype), bv=to_dev(bv_s, dtype),
               ck=to_dev(ckb, dtype), cv=to_dev(synth.to_value_octets(cvb), dtype))
    return dev, ref, n


def _run(dev, n, **kw):
    return lrkv.decode_attn(dev["q"], dev["bk"], dev["ck"], dev["bv"], dev["cv"], n, **kw)


@pytest.mark.parametrize("n", [1, 2, 7, 8, 9, 31, 32, 33, 63, 64, 65, 100, 257, 1000])
def test_ragged_contexts_ignore_garbage_past_the_end(n):
    dev, (o_ref, lse_ref), n = _case(n, n=n)
    o, lse = _run(dev, n)
    check_decode(to_f64(o), to_f64(lse), o_ref, lse_ref, "bf16", f"n={n}")


@pytest.mark.parametrize("splits", ["1", "2", "3", "7", "64"])
def test_forced_split_counts(splits, monkeypatch):
    dev, (o_ref, lse_ref), n = _case(3, n=3000)
    monkeypatch.setenv("LRKV_SPLITS", splits)
    o, lse = _run(dev, n)
    check_decode(to_f64(o), to_f64(lse), o_ref, lse_ref, "bf16", f"splits={splits}")


@pytest.mark.parametrize("rk,rv", [(8, 8), (16, 24), (24, 40), (40, 56), (64, 64), (56, 72), (96, 112),
                                   (128, 128), (8, 128), (128, 8)])
def test_rank_shapes(rk, rv):
    dev, (o_ref, lse_ref), n = _case(rk * 1000 + rv, rk=rk, rv=rv, n=333)
    o, lse = _run(dev, n)
    check_decode(to_f64(o), to_f64(lse), o_ref, lse_ref, "bf16", f"rk={rk} rv={rv}")


@pytest.mark.parametrize("hq,hkv,d", [(1, 1, 64), (2, 1, 128), (8, 1, 64), (16, 2, 128), (24, 8, 128), (32, 4, 64)])
def test_group_and_head_dim_shapes(hq, hkv, d):
    dev, (o_ref, lse_ref), n = _case(hq * 100 + hkv, Hq=hq, Hkv=hkv, d=d, rk=min(48, d), rv=min(64, d), n=129)
    o, lse = _run(dev, n)
    check_decode(to_f64(o), to_f64(lse), o_ref, lse_ref, "bf16", f"hq={hq} hkv={hkv} d={d}")


@pytest.mark.parametrize("hq,hkv,d,rk,rv,n", [(4, 1, 64, 16, 16, 256), (8, 2, 128, 36, 44, 301),
                                              (2, 2, 64, 64, 4, 33), (16, 2, 128, 128, 128, 70)])
def test_float32_shapes(hq, hkv, d, rk, rv, n):
    dev, (o_ref, lse_ref), n = _case(n, Hq=hq, Hkv=hkv, d=d, rk=rk, rv=rv, n=n, dtype="f32")
    o, lse = _run(dev, n)
    check_decode(to_f64(o), to_f64(lse), o_ref, lse_ref, "f32", f"f32 {hq}/{hkv}/{d}/{rk}/{rv}/{n}")


@pytest.mark.parametrize("where", ["first", "last"])
def test_peaky_queries(where):
    """Queries scaled x8: the softmax is dominated by a few tokens (the first or last one boosted)."""
    dev, _, n = _case(11, n=777, scale_q=8.0)
    # rebuild the oracle reference from the device cache contents we actually sent
    ck = to_f64(dev["ck"])[:, :, :n]
    cv = synth.from_value_octets(to_f64(dev["cv"]))[:, :, :n]
    t = 0 if where == "first" else n - 1
    ck[:, :, t] *= 4
    dev["ck"][:, :, t] = torch.from_numpy(ck[:, :, t]).to(torch.bfloat16).to(DEV)
    ck = to_f64(dev["ck"])[:, :, :n]
    o_ref, lse_ref = O.decode(to_f64(dev["q"]), to_f64(dev["bk"]), ck, to_f64(dev["bv"]), cv, n)
    o, lse = _run(dev, n)
    check_decode(to_f64(o), to_f64(lse), o_ref, lse_ref, "bf16", f"peaky {where}")


def test_bitwise_deterministic():
    dev, _, n = _case(5, n=5000)
    outs = [_run(dev, n) for _ in range(5)]
    torch.cuda.synchronize()
    for o, lse in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(lse, outs[0][1])


def test_graph_replay_matches_eager():
    dev, (o_ref, lse_ref), n = _case(6, n=1500)
    B, Hq, d = dev["q"].shape
    ws = torch.zeros(lrkv.decode_workspace_bytes(B, Hq, dev["bk"].shape[0], d, dev["bk"].shape[2],
                                                 dev["bv"].shape[2], dev["ck"].shape[2], n), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(dev["q"])
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    eager_o, eager_l = _run(dev, n)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        _run(dev, n, out=out, lse=lse, workspace=ws)      # warm up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _run(dev, n, out=out, lse=lse, workspace=ws)
    for i in range(4):
        out.zero_()
        lse.fill_(float("nan"))
        _ = (dev["q"].float() * 2).sum()                   # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager_o.view(torch.int16)), f"replay {i}"
        assert torch.equal(lse, eager_l), f"replay {i}"
    check_decode(to_f64(out), to_f64(lse), o_ref, lse_ref, "bf16", "graph replay")


def test_partial_then_merge_equals_one_call():
    """The two-phase API runs the same two kernels as the one-call decode."""
    dev, (o_ref, lse_ref), n = _case(7, n=2222)
    B, Hq, d = dev["q"].shape
    H, _, rk = dev["bk"].shape
    rv = dev["bv"].shape[2]
    cap = dev["ck"].shape[2]
    ws = torch.zeros(lrkv.decode_workspace_bytes(B, Hq, H, d, rk, rv, cap, n), dtype=torch.uint8, device=DEV)
    o1, l1 = _run(dev, n)
    out = torch.empty_like(dev["q"])
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    lrkv.decode_attn_partial(dev["q"], dev["bk"], dev["ck"], dev["bv"], dev["cv"], n, ws)
    lrkv.decode_attn_merge(out, lse, n, ws, H, rk, rv, cap)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), o1.view(torch.int16)) and torch.equal(lse, l1)
    check_decode(to_f64(out), to_f64(lse), o_ref, lse_ref, "bf16", "two-phase")


def test_workspace_reuse_across_calls():
    """A workspace reused across calls of different context lengths gives the
    same result call after call."""
    dev, (o_ref, lse_ref), n = _case(9, n=4000)
    B, Hq, d = dev["q"].shape
    H, _, rk = dev["bk"].shape
    rv = dev["bv"].shape[2]
    cap = dev["ck"].shape[2]
    ws = torch.zeros(max(lrkv.decode_workspace_bytes(B, Hq, H, d, rk, rv, cap, m) for m in (n, 777, 64)),
                     dtype=torch.uint8, device=DEV)
    first = None
    for i, m in enumerate([n, 777, n, 64, n]):
        o, lse = _run(dev, m, workspace=ws)
        torch.cuda.synchronize()
        if m == n:
            if first is None:
                first = (o.clone(), lse.clone())
                check_decode(to_f64(o), to_f64(lse), o_ref, lse_ref, "bf16", "reused workspace")
            else:
                assert torch.equal(o.view(torch.int16), first[0].view(torch.int16)), f"call {i}"
                assert torch.equal(lse, first[1]), f"call {i}"


def test_explicit_scale():
    dev, _, n = _case(8, n=400)
    q = to_f64(dev["q"])
    ck = to_f64(dev["ck"])[:, :, :n]
    cv = synth.from_value_octets(to_f64(dev["cv"]))[:, :, :n]
    o_ref, lse_ref = O.decode(q, to_f64(dev["bk"]), ck, to_f64(dev["bv"]), cv, n, scale=0.3)
    o, lse = _run(dev, n, scale=0.3)
    check_decode(to_f64(o), to_f64(lse), o_ref, lse_ref, "bf16", "scale 0.3")


@pytest.mark.parametrize("hq,hkv,d,rk,rv,n", [(1, 1, 64, 16, 24, 33), (8, 1, 64, 64, 8, 300),
                                              (8, 2, 128, 128, 128, 300), (16, 2, 128, 8, 40, 70),
                                              (2, 1, 128, 24, 40, 2), (32, 4, 64, 64, 64, 1),
                                              (24, 8, 128, 40, 56, 129), (4, 2, 64, 48, 64, 1000),
                                              (12, 2, 128, 96, 112, 4097)])
@pytest.mark.parametrize("enc", [False, True])
def test_decode_step_shapes(hq, hkv, d, rk, rv, n, enc):
    """lrkv_decode_step over group sizes, head dims and ranks (the append's
    product depends on all three): row n - 1 of both caches meets the compress
    gate, every other row (NaN past the context included) keeps its bits, and
    the output is the oracle's decode over the n rows.  enc passes the key
    basis again as the explicit encoder."""
    B = 2
    rng = np.random.default_rng(hq * 7919 + d * 31 + rk * 7 + rv + n)
    cap = (n + 7) // 8 * 8 + 8

    def ortho(r):
        qm, rr = np.linalg.qr(rng.standard_normal((d, d)))
        return (qm * np.sign(np.diag(rr)))[:, :r]

    bk_s = round_store(np.stack([ortho(rk) for _ in range(hkv)]), "bf16")
    bv_s = round_store(np.stack([ortho(rv) for _ in range(hkv)]), "bf16")
    q_s = round_store(rng.standard_normal((B, hq, d)), "bf16")
    xk_s = round_store(rng.standard_normal((B, 1, hkv, d)), "bf16")
    xv_s = round_store(rng.standard_normal((B, 1, hkv, d)), "bf16")
    ck_s = round_store(rng.standard_normal((B, hkv, n - 1, rk)) * 0.97 ** np.arange(rk), "bf16")
    cv_s = round_store(rng.standard_normal((B, hkv, n - 1, rv)) * 0.97 ** np.arange(rv), "bf16")
    ex = synth.bf16_bits_to_f64
    bk, bv, q, xk, xv = ex(bk_s), ex(bv_s), ex(q_s), ex(xk_s), ex(xv_s)
    ak, av = O.compress(xk, bk), O.compress(xv, bv)
    ck_all = np.concatenate([ex(ck_s), O.round_storage(ak, "bf16")], axis=2)
    cv_all = np.concatenate([ex(cv_s), O.round_storage(av, "bf16")], axis=2)
    o_ref, lse_ref = O.decode(q, bk, ck_all, bv, cv_all, n)

    ckb = np.full((B, hkv, cap, rk), NAN_BF16, np.uint16)
    cvb = np.full((B, hkv, cap, rv), NAN_BF16, np.uint16)
    ckb[:, :, :n - 1] = ck_s
    cvb[:, :, :n - 1] = cv_s
    ckd, cvd = to_dev(ckb, "bf16"), to_dev(synth.to_value_octets(cvb), "bf16")
    bkd = to_dev(bk_s, "bf16")
    o, lse = lrkv.decode_step(to_dev(q_s, "bf16"), to_dev(xk_s, "bf16"), to_dev(xv_s, "bf16"), bkd, ckd,
                              to_dev(bv_s, "bf16"), cvd, n, enc_k=bkd if enc else None)
    torch.cuda.synchronize()
    what = f"step hq={hq} hkv={hkv} d={d} rk={rk} rv={rv} n={n} enc={enc}"
    check_compress(to_f64(ckd)[:, :, n - 1:n], ak, xk, bk, "bf16", what + " K row")
    check_compress(synth.from_value_octets(to_f64(cvd))[:, :, n - 1:n], av, xv, bv, "bf16", what + " V row")
    after_k = bits(ckd)
    after_v = synth.from_value_octets(bits(cvd))
    others = np.ones(cap, bool)
    others[n - 1] = False
    assert np.array_equal(after_k[:, :, others], ckb[:, :, others]), what + ": key rows touched"
    assert np.array_equal(after_v[:, :, others], cvb[:, :, others]), what + ": value rows touched"
    check_decode(to_f64(o), to_f64(lse), o_ref, lse_ref, "bf16", what)
