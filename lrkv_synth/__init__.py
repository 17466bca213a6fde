"""Seeded synthetic inputs for low-rank KV-cache decode attention.

This module only *draws* inputs: per-kv-head orthonormal frames and bases,
non-orthogonal encoder/decoder pairs (a query-aware key transform's shape),
rank-r coefficient rows, full key/value vectors and queries, each rounded once
to the storage dtype.  It holds no step of the method itself (no projection
onto a basis for compression, no reconstruction, no attention): both the
CPU oracle and the GPU path consume what it returns, and neither shares any
other code.

Shapes follow the Llama-3.1-8B geometry the NovaKV model card compresses
(page "Llama-3.1-NovaKV", the cache table: 32 layers, 8 kv heads of 128 dims);
decaying per-dimension spectra stand in for the singular-value decay of real
key/value caches that the KV-CoRE summary analyses (page "KV-CoRE",
abstract), and keys get lower ranks than values because that summary reports
lower normalized effective rank for keys.  No dataset, prompt or weight is
reproduced: all values are Gaussian draws.

Every array is keyed by ``SeedSequence([0x4C524B56, cfg, layer, b, h, tag, part])``
so any (batch, kv-head) slice can be regenerated on its own, which is how the
parity tests check sampled rows of full-size workloads.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

MAGIC = 0x4C524B56  # "LRKV"

# Draw tags: one independent stream per kind of array.
TAG_FRAME_K = 0      # orthonormal frame whose leading columns are the key basis
TAG_FRAME_V = 1      # same for values
TAG_KEYS = 2         # key coefficients / key vectors
TAG_VALUES = 3       # value coefficients / value vectors
TAG_QUERY = 4        # decode queries
TAG_INJECT_SET = 5   # which tokens get an off-subspace component (hybrid workload)
TAG_INJECT_DIR_K = 6
TAG_INJECT_DIR_V = 9
TAG_QMOMENT = 7      # eigenframe of the synthetic query second moment (query-aware transform)
TAG_QUERY_AWARE = 8  # decode queries drawn with that second moment
TAG_LATENT_QUERY = 10  # queries already in the key latent space (absorbed projections)

# "part" of a sequence a draw belongs to.
PART_DIRECT = 0      # rows drawn directly as coefficients (an already-filled cache)
PART_PREFILL = 1     # full vectors of a prefill chunk that go through compress
PART_APPEND = 2      # the full vectors of the token appended at this decode step


# ----------------------------------------------------------------------------
# storage-dtype rounding (input quantisation only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Inputs here are finite.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = bits.astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


@dataclasses.dataclass
class Stored:
    """An array as the GPU receives it (``store``) and its exact value (``exact``).

    ``store`` is uint16 bfloat16 bit patterns or float32; ``exact`` is the
    float64 image of exactly those bits.
    """
    store: np.ndarray
    exact: np.ndarray

    @property
    def shape(self):
        return self.store.shape


def quantize(x: np.ndarray, dtype: str) -> Stored:
    """Round float64 values once to the storage dtype.

    bf16 goes through float32 first (both steps round to nearest even); the
    result is a deterministic function of the seed, which is all an input needs.
    """
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return Stored(x32, x32.astype(np.float64))
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x32)
        return Stored(bits, bf16_bits_to_f64(bits))
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, ranks, spectrum and context lengths."""
    name: str
    cfg_id: int
    dtype: str                 # storage dtype: "f32" or "bf16"
    layers: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ranks_even: tuple          # (r_K, r_V) on even layers
    ranks_odd: tuple           # (r_K, r_V) on odd layers
    n_ctx: tuple               # context lengths N, counting the appended token
    rho: float                 # per-dimension std decays as rho**i
    prefill: int = 0           # tokens of the last prefill chunk that go through compress
    append: bool = False       # the last token of the context is appended through compress
    full_all: bool = False     # every token is a full vector that goes through compress
    hybrid_frac: float = 0.0   # fraction of tokens with an injected off-subspace component
    inject_scale: float = 3.0  # injected component norm, in units of the median token norm

    def ranks(self, layer: int) -> tuple:
        return self.ranks_even if layer % 2 == 0 else self.ranks_odd

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def n_injected(self, n_ctx: int) -> int:
        return int(round(self.hybrid_frac * n_ctx))


# The five synthetic workloads; shapes and spectra follow the Llama-3.1-8B
# geometry and the context ladder the pages quote (256 .. 131072 tokens).
TINY_F32 = Workload("tiny-f32", 1, "f32", 1, 1, 4, 1, 64, (16, 16), (16, 16), (256,), 0.9,
                    full_all=True)
LLAMA_LAYER = Workload("llama8b-layer-2k", 2, "bf16", 1, 1, 32, 8, 128, (64, 80), (64, 80),
                       (2048,), 0.95)
LLAMA_STEP = Workload("llama8b-32layer-step", 3, "bf16", 32, 1, 32, 8, 128, (56, 72), (56, 72),
                      (256, 2048, 8192), 0.95, append=True)
BATCHED_32K = Workload("llama8b-b16-32k", 4, "bf16", 32, 16, 32, 8, 128, (32, 96), (48, 112),
                       (32768,), 0.97, prefill=4096, append=True)
HYBRID_128K = Workload("llama8b-hybrid-128k", 5, "bf16", 1, 1, 32, 8, 128, (64, 64), (64, 64),
                       (131072,), 0.97, hybrid_frac=0.05)

WORKLOADS = {w.name: w for w in (TINY_F32, LLAMA_LAYER, LLAMA_STEP, BATCHED_32K, HYBRID_128K)}


def scaled(w: Workload, **changes) -> Workload:
    """A smaller copy of a workload (same seeds and spectra, other sizes)."""
    return dataclasses.replace(w, **changes)


# ----------------------------------------------------------------------------
# draws
# ----------------------------------------------------------------------------

def rng(w: Workload, layer: int, b: int, h: int, tag: int, part: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([MAGIC, w.cfg_id, layer, b, h, tag, part])
    return np.random.Generator(np.random.PCG64(ss))


def spectrum(w: Workload, n: int) -> np.ndarray:
    return w.rho ** np.arange(n, dtype=np.float64)


def frame(w: Workload, layer: int, h: int, which: str) -> np.ndarray:
    """Orthonormal d x d frame (float64): QR of a seeded Gaussian, diag(R) > 0."""
    tag = TAG_FRAME_K if which == "k" else TAG_FRAME_V
    g = rng(w, layer, 0, h, tag).standard_normal((w.head_dim, w.head_dim))
    q, r = np.linalg.qr(g)
    return q * np.sign(np.diag(r))[None, :]


def basis(w: Workload, layer: int, which: str) -> Stored:
    """Per-kv-head basis [Hkv, d, r]: the leading r columns of each frame."""
    r = w.ranks(layer)[0 if which == "k" else 1]
    b = np.stack([frame(w, layer, h, which)[:, :r] for h in range(w.n_kv_heads)])
    return quantize(b, w.dtype)


def query(w: Workload, layer: int, batch: Optional[int] = None) -> Stored:
    """Decode queries [B, Hq, d], standard normal."""
    B = w.batch if batch is None else batch
    q = np.stack([rng(w, layer, b, 0, TAG_QUERY).standard_normal((w.n_q_heads, w.head_dim))
                  for b in range(B)])
    return quantize(q, w.dtype)


def latent_query(w: Workload, layer: int, batch: Optional[int] = None) -> Stored:
    """Queries already projected into the key latent space [B, Hq, r_K], standard normal.

    With projections that absorb the key basis, a decode query arrives with
    r_K coordinates; a standard normal query against an orthonormal basis has
    standard normal coordinates, which is what is drawn here.
    """
    B = w.batch if batch is None else batch
    rk = w.ranks(layer)[0]
    q = np.stack([rng(w, layer, b, 0, TAG_LATENT_QUERY).standard_normal((w.n_q_heads, rk)) for b in range(B)])
    return quantize(q, w.dtype)


def direct_coeffs(w: Workload, layer: int, which: str, b: int, h: int, n_rows: int,
                  exact: bool = True) -> Stored:
    """Coefficient rows c ~ N(0, diag(rho^(2i))) for i < r, as an already-filled cache [n, r].

    exact=False skips the float64 image (``Stored.exact`` is None) for bulk inputs.
    """
    r = w.ranks(layer)[0 if which == "k" else 1]
    tag = TAG_KEYS if which == "k" else TAG_VALUES
    z = rng(w, layer, b, h, tag, PART_DIRECT).standard_normal((n_rows, r), dtype=np.float32)
    c = z * spectrum(w, r).astype(np.float32)[None, :]
    if w.dtype == "bf16":
        bits = f32_to_bf16_bits(c)
        return Stored(bits, bf16_bits_to_f64(bits) if exact else None)
    return Stored(c, c.astype(np.float64) if exact else None)


def full_tokens(w: Workload, layer: int, which: str, b: int, h: int, n_tokens: int,
                part: int) -> Stored:
    """Full vectors x = (z * rho^i) Q^T [n, d], Q the kv head's frame, z standard normal."""
    tag = TAG_KEYS if which == "k" else TAG_VALUES
    z = rng(w, layer, b, h, tag, part).standard_normal((n_tokens, w.head_dim))
    x = (z * spectrum(w, w.head_dim)[None, :]) @ frame(w, layer, h, which).T
    return quantize(x, w.dtype)


def stack_heads(w: Workload, fn, batch: Optional[int] = None, threads: int = 8) -> Stored:
    """Call ``fn(b, h) -> Stored`` for every (batch, kv-head) and stack to [B, Hkv, ...]."""
    B = w.batch if batch is None else batch
    keys = [(b, h) for b in range(B) for h in range(w.n_kv_heads)]
    if threads > 1 and len(keys) > 1:
        with ThreadPoolExecutor(threads) as ex:
            parts = list(ex.map(lambda bh: fn(*bh), keys))
    else:
        parts = [fn(b, h) for b, h in keys]
    store = np.stack([p.store for p in parts]).reshape((B, w.n_kv_heads) + parts[0].store.shape)
    if parts[0].exact is None:
        return Stored(store, None)
    exact = np.stack([p.exact for p in parts]).reshape((B, w.n_kv_heads) + parts[0].exact.shape)
    return Stored(store, exact)


def tokens_major(s: Stored) -> Stored:
    """[B, Hkv, T, d] -> [B, T, Hkv, d] (the layout a K/V projection produces)."""
    return Stored(np.ascontiguousarray(s.store.transpose(0, 2, 1, 3)),
                  None if s.exact is None else np.ascontiguousarray(s.exact.transpose(0, 2, 1, 3)))


# ----------------------------------------------------------------------------
# hybrid workload: tokens in the span of the basis, some with an injected
# off-subspace component (the outliers an OjaKV-style cache keeps full rank)
# ----------------------------------------------------------------------------

def injected_set(w: Workload, layer: int, b: int, n_tokens: int) -> np.ndarray:
    """Sorted token indices that carry an injected component (same for all heads, K and V)."""
    f = w.n_injected(n_tokens)
    perm = rng(w, layer, b, 0, TAG_INJECT_SET).permutation(n_tokens)
    return np.sort(perm[:f])


def hybrid_tokens(w: Workload, layer: int, which: str, b: int, h: int, n_tokens: int,
                  inject: np.ndarray) -> Stored:
    """Full vectors [n, d] for the hybrid workload.

    Base tokens are x = c B^T with c drawn like ``direct_coeffs`` and B the
    stored (rounded) basis, so they lie in the basis span up to the final
    rounding.  Tokens in ``inject`` get ``inject_scale * m * w_hat`` added,
    m the median base-token norm of this (b, h, K|V) and w_hat a unit Gaussian
    direction with its component in the span of the exact frame columns removed.
    """
    r = w.ranks(layer)[0 if which == "k" else 1]
    fr = frame(w, layer, h, which)
    bq = quantize(fr[:, :r], w.dtype).exact
    tag = TAG_KEYS if which == "k" else TAG_VALUES
    z = rng(w, layer, b, h, tag, PART_DIRECT).standard_normal((n_tokens, r))
    x = (z * spectrum(w, r)[None, :]) @ bq.T
    if len(inject):
        m = float(np.median(np.linalg.norm(x, axis=1)))
        dtag = TAG_INJECT_DIR_K if which == "k" else TAG_INJECT_DIR_V
        g = rng(w, layer, b, h, dtag).standard_normal((len(inject), w.head_dim))
        q = fr[:, :r]
        g = g - (g @ q) @ q.T
        g /= np.linalg.norm(g, axis=1, keepdims=True)
        x[inject] += w.inject_scale * m * g
    return quantize(x, w.dtype)


# ----------------------------------------------------------------------------
# query-aware (non-orthogonal) key transform: an encoder/decoder pair per kv
# head of the form the NOVA-KV summary derives (Methodology, Key Transform
# Derivation, Theorem 1): R = M_q^(1/2) E with E orthonormal columns,
# coefficients r = k R, keys back as r R^-1
# ----------------------------------------------------------------------------

def query_moment_root(w: Workload, layer: int, h: int, kappa: float = 4.0):
    """A synthetic square root W = M_q^(1/2) of a query second moment and its inverse (float64 [d, d]).

    W = U diag(s) U^T with U a seeded orthonormal frame and s spaced
    geometrically over [kappa^-1/2, kappa^1/2]; W^-1 = U diag(1/s) U^T.
    """
    g = rng(w, layer, 0, h, TAG_QMOMENT).standard_normal((w.head_dim, w.head_dim))
    u, r = np.linalg.qr(g)
    u = u * np.sign(np.diag(r))[None, :]
    s = np.geomspace(kappa ** -0.5, kappa ** 0.5, w.head_dim)
    return (u * s[None, :]) @ u.T, (u / s[None, :]) @ u.T


def key_transform(w: Workload, layer: int, which: str = "k", kappa: float = 4.0):
    """Encoder and decoder [Hkv, d, r] per kv head, each rounded to the storage dtype.

    enc = W E and dec = W^-1 E, W from :func:`query_moment_root`, so that
    dec^T enc = I (before rounding) and enc is not orthonormal.  E is the
    orthonormalised W F_r, F_r the leading r columns of the kv head's frame,
    so the decoder spans the subspace the synthetic tokens concentrate in.
    The pair has the theorem's form; E is not solved for (the decode path
    treats any such pair alike).  Returns (enc, dec) as Stored.
    """
    r = w.ranks(layer)[0 if which == "k" else 1]
    encs, decs = [], []
    for h in range(w.n_kv_heads):
        root, root_inv = query_moment_root(w, layer, h, kappa)
        e, rr = np.linalg.qr(root @ frame(w, layer, h, which)[:, :r])
        e = e * np.sign(np.diag(rr))[None, :]
        encs.append(root @ e)
        decs.append(root_inv @ e)
    return quantize(np.stack(encs), w.dtype), quantize(np.stack(decs), w.dtype)


def query_aware_query(w: Workload, layer: int, kappa: float = 4.0, batch: Optional[int] = None) -> Stored:
    """Decode queries [B, Hq, d] with second moment W^2 (q = z W, z standard
    normal), W the square root of the query head's kv head."""
    B = w.batch if batch is None else batch
    roots = [query_moment_root(w, layer, h, kappa)[0] for h in range(w.n_kv_heads)]
    q = np.stack([rng(w, layer, b, 0, TAG_QUERY_AWARE).standard_normal((w.n_q_heads, w.head_dim))
                  for b in range(B)])
    for hq in range(w.n_q_heads):
        q[:, hq] = q[:, hq] @ roots[hq // w.group]
    return quantize(q, w.dtype)


def to_value_octets(c: np.ndarray) -> np.ndarray:
    """Row layout [..., n, r] -> value-cache layout [..., n/8, r, 8] (n % 8 == 0).

    The value cache keeps each column's 8 consecutive tokens contiguous; this
    helper only permutes axes, for loading drawn coefficients into a cache.
    """
    *lead, n, r = c.shape
    assert n % 8 == 0, n
    return np.ascontiguousarray(c.reshape(*lead, n // 8, 8, r).swapaxes(-1, -2))


def from_value_octets(c: np.ndarray) -> np.ndarray:
    """Inverse of :func:`to_value_octets`: [..., n/8, r, 8] -> [..., n, r]."""
    *lead, n8, r, e = c.shape
    assert e == 8
    return np.ascontiguousarray(c.swapaxes(-1, -2).reshape(*lead, n8 * 8, r))
