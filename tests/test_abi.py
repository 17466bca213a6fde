"""The C-ABI library: it loads without a GPU, exports what the header declares,
and rejects invalid calls with a status before launching anything."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lrkv.h")


def _lib():
    lrkv = pytest.importorskip("decode_attention_lrkv_amd")
    if not os.path.exists(lrkv.LIB_PATH):
        pytest.skip("liblrkv.so not built")
    return lrkv, lrkv.library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lrkv_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("lrkv_compress", "lrkv_decode_attn", "lrkv_compress_hybrid", "lrkv_decode_attn_hybrid",
              "lrkv_decode_workspace_bytes", "lrkv_status_string", "lrkv_last_error",
              "lrkv_decode_attn_partial", "lrkv_decode_attn_merge", "lrkv_compress_hybrid_workspace_bytes",
              "lrkv_decode_step", "lrkv_decode_step_workspace_bytes", "lrkv_decode_step_partial",
              "lrkv_decode_step_merge", "lrkv_decode_attn_latent", "lrkv_oja_update",
              "lrkv_oja_workspace_bytes", "lrkv_decode_attn_seqlens", "lrkv_decode_step_seqlens",
              "lrkv_decode_step_noalloc", "lrkv_decode_step_noalloc_max_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lrkv, lib = _lib()
    out = subprocess.run(["nm", "-D", "--defined-only", lrkv.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(lrkv_\w+)", out))
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    for n in _declared():
        assert getattr(lib, n) is not None


def test_header_compiles_as_c():
    """The header is plain C (a C caller needs no C++ or torch)."""
    src = '#include "lrkv.h"\nint main(void) { lrkv_dims d = {0}; (void)d; return (int)LRKV_OK; }\n'
    r = subprocess.run(["gcc", "-x", "c", "-std=c99", "-fsyntax-only", "-D__HIP_PLATFORM_AMD__",
                        f"-I{os.path.dirname(HEADER)}", "-I/opt/rocm/include", "-"],
                       input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_status_strings():
    _, lib = _lib()
    assert lib.lrkv_status_string(0) == b"ok"
    assert lib.lrkv_status_string(3) == b"workspace too small"
    assert lib.lrkv_status_string(99) == b"unknown status"


P = ctypes.c_void_p(16)          # a non-null, 16-byte aligned address that is never dereferenced
MIS = ctypes.c_void_p(18)        # misaligned


def _dims(lrkv, **kw):
    base = dict(batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128, rank_k=32, rank_v=64, capacity=256)
    base.update(kw)
    return lrkv._Dims(*[base[k] for k in ("batch", "n_q_heads", "n_kv_heads", "head_dim", "rank_k",
                                            "rank_v", "capacity")])


def _decode(lib, lrkv, dims, n_ctx=100, q=P, ws=P, ws_bytes=1 << 30, dtype=1, scale=0.0):
    return lib.lrkv_decode_attn(q, P, P, P, P, P, None, ctypes.byref(dims), n_ctx, scale, dtype, ws,
                                ws_bytes, None)


@pytest.mark.parametrize("dims_kw,n_ctx,status,needle", [
    (dict(head_dim=96), 100, 2, "head_dim"),
    (dict(rank_k=36), 100, 2, "rank_k"),            # not a multiple of 8 for bf16
    (dict(rank_v=0), 100, 2, "rank_v"),
    (dict(rank_v=136), 100, 2, "rank_v"),
    (dict(n_q_heads=9), 100, 1, "multiple"),
    (dict(n_q_heads=32, n_kv_heads=2), 100, 2, "8 query heads"),
    (dict(capacity=100), 100, 1, "capacity"),
    (dict(batch=0), 100, 1, "batch"),
    (dict(), 0, 1, "n_ctx"),
    (dict(), 257, 1, "n_ctx"),
])
def test_decode_rejects_invalid_dims(dims_kw, n_ctx, status, needle):
    lrkv, lib = _lib()
    st = _decode(lib, lrkv, _dims(lrkv, **dims_kw), n_ctx=n_ctx)
    assert st == status
    assert needle in lib.lrkv_last_error().decode()


def test_decode_rejects_bad_pointers_and_workspace():
    lrkv, lib = _lib()
    d = _dims(lrkv)
    assert _decode(lib, lrkv, d, q=None) == 1 and b"NULL" in lib.lrkv_last_error()
    assert _decode(lib, lrkv, d, q=MIS) == 1 and b"aligned" in lib.lrkv_last_error()
    assert _decode(lib, lrkv, d, ws_bytes=16) == 3
    assert _decode(lib, lrkv, d, dtype=7) == 1
    assert _decode(lib, lrkv, d, scale=float("inf")) == 1
    # fp32 accepts ranks that are multiples of 4 but not of 8
    assert _decode(lib, lrkv, _dims(lrkv, rank_k=36), dtype=0, ws_bytes=16) == 3


def test_compress_validation():
    lrkv, lib = _lib()
    c = lib.lrkv_compress
    # x, basis, coeff, kind, B, Hkv, d, r, T, pos, cap, dtype, stream
    assert c(P, P, P, 0, 1, 2, 128, 32, 10, 250, 256, 1, None) == 1      # rows past capacity
    assert c(P, P, P, 2, 1, 2, 128, 32, 10, 0, 256, 1, None) == 1        # unknown cache kind
    assert c(P, P, P, 0, 1, 2, 80, 32, 10, 0, 256, 1, None) == 2         # head_dim
    assert c(None, P, P, 0, 1, 2, 128, 32, 10, 0, 256, 1, None) == 1     # null x
    assert c(P, P, MIS, 1, 1, 2, 128, 32, 10, 0, 256, 1, None) == 1      # misaligned coeff
    assert c(P, P, P, 1, 1, 2, 128, 32, 0, 0, 256, 1, None) == 0         # no tokens: nothing to do
    assert c(P, P, P, 1, 1, 2, 128, 32, 10, 0, 252, 1, None) == 1        # capacity not a multiple of 8


def test_hybrid_validation():
    lrkv, lib = _lib()
    d = _dims(lrkv)
    f = lib.lrkv_compress_hybrid
    args = lambda tau=0.5, side_cap=64, dtype=1, n_lr=P: (P, P, P, P, tau, P, P, n_lr, P, P, P, P, None, P,
                                                           ctypes.byref(d), 100, 0, side_cap, dtype, P,
                                                           1 << 30, None)
    assert f(*args(tau=-1.0)) == 1
    assert f(*args(tau=float("nan"))) == 1
    assert f(*args(side_cap=60)) == 1
    assert f(*args(dtype=0)) == 2
    assert f(*args(n_lr=None)) == 1
    g = lib.lrkv_decode_attn_hybrid
    assert g(P, P, P, P, P, P, P, P, P, 0, P, None, ctypes.byref(d), 0.0, 1, P, 1 << 30, None) == 1


def test_workspace_queries():
    lrkv, lib = _lib()
    d = _dims(lrkv)
    n1 = lib.lrkv_decode_workspace_bytes(ctypes.byref(d), 256, 0)
    assert n1 > 0 and n1 % 256 == 0
    assert lib.lrkv_decode_workspace_bytes(ctypes.byref(d), 0, 0) == 0
    assert lib.lrkv_decode_workspace_bytes(ctypes.byref(_dims(lrkv, head_dim=96)), 256, 0) == 0
    assert lib.lrkv_decode_workspace_bytes(ctypes.byref(d), 256, 64) > n1
    assert lib.lrkv_compress_hybrid_workspace_bytes(ctypes.byref(d), 1000) > 0


def test_decode_step_validation():
    lrkv, lib = _lib()
    d = _dims(lrkv)
    f = lib.lrkv_decode_step
    # q, k_new, v_new, basis_k, coeff_k, basis_v, coeff_v, enc_k, out, lse, dims, n_ctx, scale, dtype, ws, bytes, stream
    args = lambda enc=None, k_new=P, n_ctx=100, ws_bytes=1 << 30: (P, k_new, P, P, P, P, P, enc, P, None,
                                                                    ctypes.byref(d), n_ctx, 0.0, 1, P, ws_bytes,
                                                                    None)
    assert f(*args(enc=MIS)) == 1 and b"enc_k" in lib.lrkv_last_error()
    assert f(*args(k_new=None)) == 1 and b"NULL" in lib.lrkv_last_error()
    assert f(*args(n_ctx=0)) == 1
    assert f(*args(enc=P, ws_bytes=16)) == 3
    g = lib.lrkv_decode_step_partial
    assert g(P, P, P, P, P, P, P, MIS, ctypes.byref(d), 100, 0.0, 1, P, 1 << 30, None) == 1


def test_seqlens_validation():
    """The device-length calls check the plan bound, the lengths pointer,
    the dtype and the workspace before any launch."""
    lrkv, lib = _lib()
    d = _dims(lrkv)
    need = lib.lrkv_decode_workspace_bytes(ctypes.byref(d), 256, 0)
    f = lib.lrkv_decode_attn_seqlens
    # q, basis_k, coeff_k, basis_v, coeff_v, out, lse, dims, seq_lens, max_seq_len, scale, dtype, ws, bytes, stream
    args = lambda lens=P, mx=256, dtype=1, ws_bytes=need, scale=0.0: (P, P, P, P, P, P, None, ctypes.byref(d),
                                                                      lens, mx, scale, dtype, P, ws_bytes, None)
    assert f(*args(lens=None)) == 1 and b"seq_lens" in lib.lrkv_last_error()
    assert f(*args(lens=ctypes.c_void_p(18))) == 1 and b"seq_lens" in lib.lrkv_last_error()
    assert f(*args(mx=0)) == 1 and f(*args(mx=257)) == 1
    assert f(*args(dtype=0)) == 2
    assert f(*args(ws_bytes=need - 256)) == 3
    assert f(*args(scale=float("nan"))) == 1
    g = lib.lrkv_decode_step_seqlens
    need_s = lib.lrkv_decode_step_workspace_bytes(ctypes.byref(d), 256)
    # q, k_new, v_new, basis_k, coeff_k, basis_v, coeff_v, enc_k, out, lse, dims, seq_lens, max_seq_len,
    # scale, dtype, ws, bytes, stream
    sargs = lambda lens=P, mx=256, dtype=1, ws_bytes=need_s, k_new=P: (P, k_new, P, P, P, P, P, None, P, None,
                                                                       ctypes.byref(d), lens, mx, 0.0, dtype, P,
                                                                       ws_bytes, None)
    assert g(*sargs(lens=None)) == 1
    assert g(*sargs(k_new=None)) == 1
    assert g(*sargs(mx=300)) == 1
    assert g(*sargs(dtype=0)) == 2
    assert g(*sargs(ws_bytes=16)) == 3


def test_noalloc_refuses_oversized_requests_before_any_device_call():
    """The fixed-workspace step refuses dims whose workspace exceeds the
    library's array, with a message, and without touching a device (this
    runs without a GPU)."""
    lrkv, lib = _lib()
    cap = lib.lrkv_decode_step_noalloc_max_bytes()
    assert cap == 8 << 20
    big = _dims(lrkv, batch=1024, n_q_heads=64, n_kv_heads=8)
    assert lib.lrkv_decode_step_workspace_bytes(ctypes.byref(big), 200) > cap
    f = lib.lrkv_decode_step_noalloc
    # q, k_new, v_new, basis_k, coeff_k, basis_v, coeff_v, enc_k, out, lse, dims, n_ctx, scale, dtype, stream
    assert f(P, P, P, P, P, P, P, None, P, None, ctypes.byref(big), 200, 0.0, 1, None) == 3
    assert b"fixed" in lib.lrkv_last_error()
    assert f(P, P, P, P, P, P, P, None, P, None, None, 200, 0.0, 1, None) == 1
    assert f(P, P, P, P, P, P, P, None, P, None, ctypes.byref(_dims(lrkv)), 0, 0.0, 1, None) == 1


def test_latent_decode_validation():
    lrkv, lib = _lib()
    f = lib.lrkv_decode_attn_latent
    d = _dims(lrkv)
    # q_lat, coeff_k, coeff_v, out_lat, lse, dims, n_ctx, scale, dtype, ws, bytes, stream
    assert f(None, P, P, P, None, ctypes.byref(d), 100, 0.0, 1, P, 1 << 30, None) == 1
    assert f(P, P, P, MIS, None, ctypes.byref(d), 100, 0.0, 1, P, 1 << 30, None) == 1
    assert f(P, P, P, P, None, ctypes.byref(d), 300, 0.0, 1, P, 1 << 30, None) == 1
    assert f(P, P, P, P, None, ctypes.byref(d), 100, 0.0, 1, P, 16, None) == 3
    assert f(P, P, P, P, None, ctypes.byref(_dims(lrkv, rank_v=12)), 100, 0.0, 1, P, 1 << 30, None) == 2


def test_oja_update_validation():
    lrkv, lib = _lib()
    f = lib.lrkv_oja_update
    need = lib.lrkv_oja_workspace_bytes(2, 8, 128, 48, 100)
    assert need > 0
    assert lib.lrkv_oja_workspace_bytes(2, 8, 128, 48, 100) == need       # deterministic plan
    assert lib.lrkv_oja_workspace_bytes(2, 8, 128, 48, 0) > 0
    # x, basis, basis_bf16, batch, Hkv, d, rank, n_tokens, eta, ws, bytes, stream
    assert f(None, P, None, 2, 8, 128, 48, 100, 1e-3, P, need, None) == 1
    assert f(P, None, None, 2, 8, 128, 48, 100, 1e-3, P, need, None) == 1
    assert f(P, P, MIS, 2, 8, 128, 48, 100, 1e-3, P, need, None) == 1
    assert f(P, P, None, 2, 8, 96, 48, 100, 1e-3, P, need, None) == 2
    assert f(P, P, None, 2, 8, 128, 12, 100, 1e-3, P, need, None) != 0
    assert f(P, P, None, 2, 8, 128, 48, -1, 1e-3, P, need, None) == 1
    assert f(P, P, None, 2, 8, 128, 48, 100, float("nan"), P, need, None) == 1
    assert f(P, P, None, 0, 8, 128, 48, 100, 1e-3, P, need, None) == 1
    assert f(P, P, None, 2, 8, 128, 48, 100, 1e-3, P, need - 4, None) == 3
    assert f(P, P, None, 2, 8, 128, 48, 100, 1e-3, None, need, None) == 1
    assert f(P, P, None, 2, 8, 128, 48, 0, 1e-3, None, 0, None) == 0      # nothing to do, nothing launched
    assert f(None, P, None, 2, 8, 128, 48, 0, 1e-3, None, 0, None) == 0


def test_missing_library_fails_loudly():
    """Without the built library every entry point raises; nothing falls back to another path."""
    code = (
        "import sys, torch\n"
        "import decode_attention_lrkv_amd as lrkv\n"
        "lrkv.LIB_PATH = '/nonexistent/liblrkv.so'\n"
        "for call in (lambda: lrkv.library(),\n"
        "             lambda: lrkv.decode_workspace_bytes(1, 8, 2, 128, 32, 64, 256, 100),\n"
        "             lambda: lrkv.decode_attn_latent(torch.zeros(1, 8, 32), torch.zeros(1, 2, 256, 32),\n"
        "                                             torch.zeros(1, 2, 32, 64, 8), 100, 128),\n"
        "             lambda: lrkv.oja_workspace_bytes(1, 2, 128, 32, 64)):\n"
        "    try:\n"
        "        call()\n"
        "    except lrkv.LrkvError as e:\n"
        "        assert 'missing' in str(e), e\n"
        "    else:\n"
        "        sys.exit('no error')\n"
        "print('ok')\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


def test_build_compiles_every_source():
    """Every kernel and host source in csrc/ goes into the library."""
    from decode_attention_lrkv_amd import build as B
    on_disk = sorted(f for f in os.listdir(B.CSRC) if f.endswith((".hip", ".cpp")))
    assert sorted(B.SOURCES) == on_disk
