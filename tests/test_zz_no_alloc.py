"""lrkv_decode_step_noalloc (the library's fixed workspace, no allocation)
against lrkv_decode_step (a caller's workspace) through the C ABI.

Calls in a row on one GPU, each with a smaller input than the one before:
the batched-32K shape at 4096 tokens (attention workgroups plus the merge
launch); batch 1 at 896 and then 640 tokens (at most 64 workgroups on a
256-compute-unit chip, so the last workgroup of each (batch, kv head) merges
in the launch, counting arrivals in the first bytes of the fixed array: the
640-token call also shows that the 896-token call left those counters zero);
and batch 1 at 300 tokens (one workgroup per (batch, kv head), no merge).
Both entry points run the same kernels on the same inputs, so the outputs,
lse and the appended cache rows must agree bit for bit.  A request larger
than the fixed workspace is refused before any device call.
"""
import ctypes

import numpy as np
import pytest
import torch

import lrkv_synth as synth
from tests.gpu_helpers import DEV, to_dev

pytestmark = pytest.mark.gpu

lrkv = pytest.importorskip("decode_attention_lrkv_amd")


def _case(w, layer, N, cap):
    B, H = w.batch, w.n_kv_heads
    rk, rv = w.ranks(layer)
    ck = np.zeros((B, H, cap, rk), np.uint16)
    cv = np.zeros((B, H, cap, rv), np.uint16)
    ck[:, :, :N - 1] = synth.stack_heads(w, lambda b, h: synth.direct_coeffs(w, layer, "k", b, h, N - 1,
                                                                             exact=False)).store
    cv[:, :, :N - 1] = synth.stack_heads(w, lambda b, h: synth.direct_coeffs(w, layer, "v", b, h, N - 1,
                                                                             exact=False)).store
    xk = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(w, layer, "k", b, h, 1,
                                                                                synth.PART_APPEND)))
    xv = synth.tokens_major(synth.stack_heads(w, lambda b, h: synth.full_tokens(w, layer, "v", b, h, 1,
                                                                                synth.PART_APPEND)))
    return dict(q=to_dev(synth.query(w, layer), "bf16"), bk=to_dev(synth.basis(w, layer, "k"), "bf16"),
                bv=to_dev(synth.basis(w, layer, "v"), "bf16"), ck=to_dev(ck, "bf16"),
                cv=to_dev(synth.to_value_octets(cv), "bf16"), kn=to_dev(xk, "bf16"), vn=to_dev(xv, "bf16"))


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


@pytest.mark.parametrize("first_then_smaller", [True])
def test_noalloc_step_equals_the_workspace_step(first_then_smaller):
    cases = [(synth.scaled(synth.BATCHED_32K, n_ctx=(4096,)), 1, 4096, 4096),
             (synth.LLAMA_STEP, 0, 896, 896), (synth.LLAMA_STEP, 1, 640, 640),
             (synth.LLAMA_STEP, 0, 300, 304)]
    for w, layer, N, cap in cases:
        print(f"noalloc case: batch {w.batch}, N {N}, layer {layer}", flush=True)
        c = _case(w, layer, N, cap)
        ck2, cv2 = c["ck"].clone(), c["cv"].clone()
        B, Hq, d = c["q"].shape
        o1, l1 = lrkv.decode_step(c["q"], c["kn"], c["vn"], c["bk"], c["ck"], c["bv"], c["cv"], N)
        o2 = torch.full_like(o1, float("nan"))
        l2 = torch.full_like(l1, float("nan"))
        lrkv.decode_step_noalloc(c["q"], c["kn"], c["vn"], c["bk"], ck2, c["bv"], cv2, N, o2, l2)
        torch.cuda.synchronize()
        assert _same(o1, o2), f"output differs at batch {w.batch}, N {N}"
        assert _same(l1, l2), f"lse differs at batch {w.batch}, N {N}"
        assert _same(c["ck"], ck2) and _same(c["cv"], cv2), "cache rows differ"
        assert torch.isfinite(o2.float()).all()


def test_noalloc_refuses_oversized_requests():
    lib = lrkv.library()
    cap = lrkv.decode_step_noalloc_max_bytes()
    assert cap == 8 << 20
    dims = lrkv._Dims(1024, 64, 8, 128, 32, 64, 256)
    need = lib.lrkv_decode_step_workspace_bytes(ctypes.byref(dims), 200)
    assert need > cap
    p = ctypes.c_void_p(16)
    st = lib.lrkv_decode_step_noalloc(p, p, p, p, p, p, p, None, p, None, ctypes.byref(dims), 200, 0.0, 1, None)
    assert st == 3 and b"fixed" in lib.lrkv_last_error()
