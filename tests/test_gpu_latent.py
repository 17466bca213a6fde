"""GPU parity for decode with absorbed projections: latent queries in, latent
outputs out, no basis read (the NovaKV delta ships modified query and output
projections: "Llama-3.1-NovaKV" model card, introduction).

The oracle attends the coefficient rows as keys and values (decode_latent);
the GPU runs lrkv_decode_attn_latent on the same bits.  Value ranks whose
quarter is not a power of two (72, 112, 20) exercise the merge's masked lanes.
The bfloat16 gate allows each latent element the half ulp its own storage
costs (the elements scale with the coefficient spectrum; see check_decode).
"""
import math

import numpy as np
import pytest
import torch

import lrkv_synth as synth
from oracle import lrkv_oracle as O
from tests.gpu_helpers import DEV, check_decode, round_store, to_dev, to_f64

pytestmark = pytest.mark.gpu

lrkv = pytest.importorskip("decode_attention_lrkv_amd")

F32_ODD_RANKS = synth.scaled(synth.TINY_F32, ranks_even=(12, 20), ranks_odd=(12, 20))
BATCHED = synth.scaled(synth.BATCHED_32K, n_ctx=(4096,))


def _rows(w, layer, which, n):
    return synth.stack_heads(w, lambda b, h: synth.direct_coeffs(w, layer, which, b, h, n))


@pytest.mark.parametrize("case", ["bf16-step-1", "bf16-step-1000", "bf16-step-8192", "bf16-b16-4096",
                                  "f32-tiny-256", "f32-oddranks-203"])
def test_latent_decode(case):
    dtype, kind, n = case.split("-")
    N = int(n)
    w = {"step": synth.LLAMA_STEP, "b16": BATCHED, "tiny": synth.TINY_F32, "oddranks": F32_ODD_RANKS}[kind]
    layer = 1 if dtype == "bf16" else 0
    B, H, d = w.batch, w.n_kv_heads, w.head_dim
    rk, rv = w.ranks(layer)
    ck, cv = _rows(w, layer, "k", N), _rows(w, layer, "v", N)
    q = synth.latent_query(w, layer)
    o_ref, lse_ref = O.decode_latent(q.exact, ck.exact, cv.exact, N, 1 / math.sqrt(d))

    cap = (N + 7) // 8 * 8 + 8          # rows past N hold other values: they must not be read
    kc = np.ones((B, H, cap, rk)) * 3.0
    vc = np.ones((B, H, cap, rv)) * 3.0
    kc[:, :, :N] = ck.exact
    vc[:, :, :N] = cv.exact
    ckd = to_dev(round_store(kc, dtype), dtype)
    cvd = to_dev(synth.to_value_octets(round_store(vc, dtype)), dtype)
    o, lse = lrkv.decode_attn_latent(to_dev(q, dtype), ckd, cvd, N, d)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (B, w.n_q_heads, rv)
    check_decode(to_f64(o), to_f64(lse), o_ref, lse_ref, dtype, f"latent {case}", storage_rounding=True)

