"""CPU oracle for decode attention over a low-rank KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only the test suite, the graft entry's smoke check and the benchmark's
``cpu_baseline`` leg use it.  It shares no code with the HIP library (no
helpers, constants or tables) and imports nothing from the package.

Plain, slow, float64 numpy, written from the pages' description of what is
computed:

* A low-rank KV cache stores, per token and kv head, rank-r coefficients of
  the key and of the value against a fixed per-head basis ("Llama-3.1-NovaKV"
  model card, introduction: post-hoc low-rank factorisation of the K and V
  projections; "OjaKV" README, Method Summary, StaticPCA: an offline basis
  that is fixed at inference).  With an orthonormal basis B the coefficients
  of x are c = x B.
* StaticPCA attends by reconstructing keys and values from the coefficients
  on the fly and running standard attention ("OjaKV" README, Method Summary,
  StaticPCA).  That is the definition used here: K_hat = C_K B_K^T,
  V_hat = C_V B_V^T, then textbook softmax attention of one decode query.
* A non-orthogonal transform splits the basis in two: an encoder E for the
  coefficients (c = x E) and a decoder D for the reconstruction
  (x_hat = c D^T), with D^T E = I.  compress takes the encoder and decode the
  decoder; with an orthonormal basis both are B.  The attention-aware key
  transform of the NOVA-KV summary (Methodology, Key Transform Derivation,
  Theorem 1) is such a pair; query_aware_key_transform builds it from
  queries and keys.
* With the bases absorbed into the query and output projections, decode
  takes q' = q B_K and returns the latent output p C_V (decode_latent).
* OjaKV keeps tokens whose reconstruction error is high in full rank and
  compresses the rest ("OjaKV" README, Method Summary, OjaKV).  The hybrid
  functions below select those tokens and attend the union of the
  reconstructed low-rank tokens and the full-rank tokens in one softmax.
* OjaKV also updates the subspace online with Oja's algorithm (same
  section); oja_update is Oja's subspace rule, summed over a call's tokens.

Readings where the pages are silent:
* softmax scale 1/sqrt(head_dim) (the NOVA-KV summary's logit bound divides
  by sqrt(d), d the head dimension);
* grouped-query attention: q head h reads kv head h // (Hq/Hkv);
* no centring, no bias: c = x B, x_hat = c B^T;
* the decode query attends tokens [0, N) of the cache, N counting the
  token appended at this step;
* bfloat16 rounding is round-to-nearest-even;
* hybrid selection: relative residual ||x - round(x B) B^T|| / ||x|| > tau for
  the key or the value (strict), with round(x B) the coefficients the cache
  stores, evaluated in float64 like the rest of this module; tokens of zero
  norm are never selected; low-rank rows and the full-rank side list both keep
  ascending token order;
* Oja update: one basis per kv head, updated from every token of the call
  (all batch rows) against the same B, step size eta given by the caller, no
  re-orthonormalisation, cached coefficients left as stored.
"""
from __future__ import annotations

import math

import numpy as np


# ----------------------------------------------------------------------------
# storage rounding
# ----------------------------------------------------------------------------

def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), as float64.

    Written from the format's definition: 8 significant bits.  With
    x = m 2^e, 0.5 <= |m| < 1, the representable neighbours are multiples of
    2^(e-8); numpy's rint rounds halfway cases to even.  Valid for the normal
    range, which is all the data here uses.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def round_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Value after storing x in the cache's dtype ("f32" or "bf16")."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# compress: coefficients against a per-kv-head basis
# ----------------------------------------------------------------------------

def compress(x: np.ndarray, basis: np.ndarray) -> np.ndarray:
    """Exact coefficients C[b, h, t, :] = X[b, t, h, :] @ B[h].

    x: [B, T, Hkv, d]; basis: [Hkv, d, r].  Returns [B, Hkv, T, r] float64.
    (NovaKV model card: the cache holds low-rank factors of K and V; OjaKV
    README, StaticPCA: a fixed offline basis.)
    """
    x = np.asarray(x, dtype=np.float64)
    basis = np.asarray(basis, dtype=np.float64)
    B, T, H, d = x.shape
    out = np.empty((B, H, T, basis.shape[2]))
    for b in range(B):
        for h in range(H):
            out[b, h] = x[b, :, h, :] @ basis[h]
    return out


def reconstruct(coeff: np.ndarray, basis: np.ndarray) -> np.ndarray:
    """K_hat = C B^T for one kv head: coeff [N, r], basis [d, r] -> [N, d]."""
    return np.asarray(coeff, dtype=np.float64) @ np.asarray(basis, dtype=np.float64).T


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------

def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Textbook attention of one query over N tokens.

    q [d]; K [N, d]; V [N, dv].  Returns (o [dv], lse, p [N], s [N]) with
    s = K q * scale, p = softmax(s), o = p V and lse = log(sum(exp(s))).
    An empty token set gives o = 0 and lse = -inf.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1]), -math.inf, np.zeros(0), np.zeros(0)
    s = (K @ np.asarray(q, dtype=np.float64)) * scale
    m = s.max()
    w = np.exp(s - m)
    L = w.sum()
    p = w / L
    return p @ V, m + math.log(L), p, s


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def decode(q, basis_k, coeff_k, basis_v, coeff_v, n_ctx: int, scale: float = None):
    """Decode attention over a low-rank cache, by explicit reconstruction.

    q [B, Hq, d]; basis_k [Hkv, d, r_K]; coeff_k [B, Hkv, >=n_ctx, r_K];
    basis_v [Hkv, d, r_V]; coeff_v [B, Hkv, >=n_ctx, r_V] (row layout).
    Query head h attends kv head h // (Hq/Hkv) over tokens [0, n_ctx).
    Returns o [B, Hq, d] float64 and lse [B, Hq] (natural log).
    (OjaKV README, StaticPCA: reconstruct keys and values, then standard
    attention.)
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = basis_k.shape[0]
    group = Hq // Hkv
    scale = default_scale(d) if scale is None else scale
    o = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    for b in range(B):
        for h in range(Hkv):
            K = reconstruct(coeff_k[b, h, :n_ctx], basis_k[h])
            V = reconstruct(coeff_v[b, h, :n_ctx], basis_v[h])
            for j in range(group):
                hq = h * group + j
                o[b, hq], lse[b, hq], _, _ = softmax_attention(q[b, hq], K, V, scale)
    return o, lse


def decode_rows(q, basis_k, coeff_k, basis_v, coeff_v, n_ctx: int, rows, scale: float = None):
    """Like :func:`decode` for a few (b, hq) rows; coeff_* hold only what those rows need.

    ``rows`` is a list of (b, hq); coeff_k/coeff_v are dicts keyed by (b, kv_head)
    giving [>=n_ctx, r] arrays.  Returns {(b, hq): (o [d], lse)}.
    """
    q = np.asarray(q, dtype=np.float64)
    Hq, d = q.shape[1], q.shape[2]
    group = Hq // basis_k.shape[0]
    scale = default_scale(d) if scale is None else scale
    out = {}
    for b, hq in rows:
        h = hq // group
        K = reconstruct(coeff_k[(b, h)][:n_ctx], basis_k[h])
        V = reconstruct(coeff_v[(b, h)][:n_ctx], basis_v[h])
        o, lse, _, _ = softmax_attention(q[b, hq], K, V, scale)
        out[(b, hq)] = (o, lse)
    return out


def decode_latent(q_lat, coeff_k, coeff_v, n_ctx: int, scale: float):
    """Decode attention in the latent space, for projections that absorb the bases.

    When the bases are folded into the model's projections offline (the
    NovaKV delta ships modified query and output projections alongside the K
    and V factors: "Llama-3.1-NovaKV" model card, introduction), a query
    arrives already as q' = q B_K and the output leaves as the latent
    o' = p C_V, lifted by the absorbed output projection.  Attention is then
    textbook attention with the coefficient rows as keys and values:
    s_t = q' . C_K[t] * scale, p = softmax(s), o' = p C_V.

    q_lat [B, Hq, r_K]; coeff_k [B, Hkv, >=n_ctx, r_K]; coeff_v [B, Hkv, >=n_ctx, r_V]
    (row layout).  scale is explicit (the head dimension is not visible
    here).  Returns o' [B, Hq, r_V] float64 and lse [B, Hq].
    """
    q_lat = np.asarray(q_lat, dtype=np.float64)
    B, Hq, _ = q_lat.shape
    Hkv = coeff_k.shape[1]
    group = Hq // Hkv
    rv = coeff_v.shape[-1]
    o = np.zeros((B, Hq, rv))
    lse = np.zeros((B, Hq))
    for b in range(B):
        for h in range(Hkv):
            K = np.asarray(coeff_k[b, h, :n_ctx], dtype=np.float64)
            V = np.asarray(coeff_v[b, h, :n_ctx], dtype=np.float64)
            for j in range(group):
                hq = h * group + j
                o[b, hq], lse[b, hq], _, _ = softmax_attention(q_lat[b, hq], K, V, scale)
    return o, lse


# ----------------------------------------------------------------------------
# hybrid (OjaKV-style) cache
# ----------------------------------------------------------------------------

def hybrid_flags(x: np.ndarray, basis: np.ndarray, tau: float, dtype: str) -> np.ndarray:
    """Per-token "reconstruction error is high" decision for one kv head.

    x [T, d] token vectors; basis [d, r].  The token is stored as the rounded
    coefficients round(x B); its reconstruction is round(x B) B^T.  The token
    is selected when ||x - x_hat|| > tau ||x||, evaluated as
    ||x - x_hat||^2 > tau^2 ||x||^2 in float64.  A token of zero norm is never
    selected (0 > 0 is false); tau = +inf selects nothing.  (OjaKV README,
    Method Summary, OjaKV: tokens with high reconstruction error stay full
    rank.)
    """
    x = np.asarray(x, dtype=np.float64)
    b = np.asarray(basis, dtype=np.float64)
    if not math.isfinite(tau):
        return np.zeros(x.shape[0], dtype=bool)
    c_stored = round_storage(x @ b, dtype)
    r = x - c_stored @ b.T
    err2 = np.sum(r * r, axis=1)
    nrm2 = np.sum(x * x, axis=1)
    return err2 > (tau * tau) * nrm2


def relative_residual(x: np.ndarray, basis: np.ndarray) -> np.ndarray:
    """||x - (x B) B^T|| / ||x|| in float64 (no rounding), per token."""
    x = np.asarray(x, dtype=np.float64)
    basis = np.asarray(basis, dtype=np.float64)
    r = x - (x @ basis) @ basis.T
    n = np.linalg.norm(x, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(n > 0, np.linalg.norm(r, axis=1) / n, 0.0)


def compress_hybrid(k, v, basis_k, basis_v, tau: float, dtype: str, pos: int = 0):
    """Split a chunk of tokens into low-rank rows and a full-rank side list.

    k, v: [B, T, Hkv, d]; bases [Hkv, d, r].  A token is kept full rank when
    its key or its value is selected by :func:`hybrid_flags` (the same token
    set for K and V keeps one side list).  Per (b, h), in ascending token
    order: low-rank tokens contribute exact coefficient rows (float64, before
    rounding) and full-rank tokens contribute their K and V rows unchanged
    and their absolute index pos + t.

    Returns a dict of per-(b, h) lists: flags [T] bool, ck, cv (exact
    coefficient rows), k_side, v_side, side_idx.
    """
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, H, d = k.shape
    res = {"flags": {}, "ck": {}, "cv": {}, "k_side": {}, "v_side": {}, "side_idx": {}}
    for b in range(B):
        for h in range(H):
            fk = hybrid_flags(k[b, :, h], basis_k[h], tau, dtype)
            fv = hybrid_flags(v[b, :, h], basis_v[h], tau, dtype)
            flag = fk | fv
            lr = np.nonzero(~flag)[0]
            side = np.nonzero(flag)[0]
            res["flags"][(b, h)] = flag
            res["ck"][(b, h)] = k[b, lr, h] @ np.asarray(basis_k[h], dtype=np.float64)
            res["cv"][(b, h)] = v[b, lr, h] @ np.asarray(basis_v[h], dtype=np.float64)
            res["k_side"][(b, h)] = k[b, side, h].copy()
            res["v_side"][(b, h)] = v[b, side, h].copy()
            res["side_idx"][(b, h)] = (pos + side).astype(np.int64)
    return res


def decode_hybrid_rows(q, basis_k, basis_v, ck, cv, k_side, v_side, rows, scale: float = None):
    """Decode over the union of low-rank and full-rank tokens, one softmax.

    ck/cv: {(b, h): [n_lr, r]} stored coefficient rows; k_side/v_side:
    {(b, h): [n_side, d]}; rows: list of (b, hq).  The low-rank tokens are
    reconstructed (StaticPCA) and stacked with the full-rank tokens, then one
    textbook softmax runs over all of them (OjaKV: both kinds of token stay in
    the same cache).  Returns {(b, hq): (o [d], lse)}.
    """
    q = np.asarray(q, dtype=np.float64)
    Hq, d = q.shape[1], q.shape[2]
    group = Hq // basis_k.shape[0]
    scale = default_scale(d) if scale is None else scale
    out = {}
    for b, hq in rows:
        h = hq // group
        K = np.concatenate([reconstruct(ck[(b, h)], basis_k[h]),
                            np.asarray(k_side[(b, h)], dtype=np.float64).reshape(-1, d)])
        V = np.concatenate([reconstruct(cv[(b, h)], basis_v[h]),
                            np.asarray(v_side[(b, h)], dtype=np.float64).reshape(-1, d)])
        o, lse, _, _ = softmax_attention(q[b, hq], K, V, scale)
        out[(b, hq)] = (o, lse)
    return out


# ----------------------------------------------------------------------------
# query-aware key transform (NOVA-KV summary, Methodology, Key Transform
# Derivation, Theorem 1 and Proposition 1)
# ----------------------------------------------------------------------------

def psd_sqrt(m: np.ndarray, inverse: bool = False) -> np.ndarray:
    """Symmetric square root M^(1/2) (or M^(-1/2)) of a symmetric positive definite matrix.

    From its eigendecomposition M = U diag(mu) U^T: M^(1/2) = U diag(sqrt(mu)) U^T.
    """
    m = np.asarray(m, dtype=np.float64)
    mu, u = np.linalg.eigh(0.5 * (m + m.T))
    if mu.min() <= 0:
        raise ValueError("matrix is not positive definite")
    root = np.sqrt(mu)
    return (u * (1.0 / root if inverse else root)[None, :]) @ u.T


def query_aware_key_transform(queries: np.ndarray, keys: np.ndarray, p: int):
    """The attention-aware key transform of one kv head, truncated to p coefficients.

    queries [Nq, d] (row vectors q), keys [Nk, d] (row vectors k).
    The score error a reconstruction k_hat causes over the queries is
    sum_i (q_i . (k - k_hat))^2 = (k - k_hat) M_q (k - k_hat)^T with
    M_q = Q^T Q (Key Transform Derivation, eq. 5).  Theorem 1: with
    E Lambda E^T the eigendecomposition of M_q^(1/2) S_k M_q^(1/2), S_k the
    centred key scatter sum_j (k_j - mean)^T (k_j - mean), eigenvalues in
    decreasing order, the optimal transform is R_K = M_q^(1/2) E; its first p
    columns give the coefficients r = k R_K[:, :p].  Keys come back as
    k = r R_K^(-1) (Proposition 1); R_K^(-1) = E^T M_q^(-1/2), whose first p
    rows are the decoder for a truncated r: k_hat = r D^T with
    D = M_q^(-1/2) E[:, :p].

    Returns (encoder [d, p], decoder [d, p], eigenvalues [d] decreasing).
    The encoder plays the part of a basis in compress (c = k enc) and the
    decoder the part of a basis in decode (k_hat = c dec^T, fold q' = q dec).
    """
    Q = np.asarray(queries, dtype=np.float64)
    K = np.asarray(keys, dtype=np.float64)
    m_q = Q.T @ Q
    root = psd_sqrt(m_q)
    root_inv = psd_sqrt(m_q, inverse=True)
    kc = K - K.mean(axis=0, keepdims=True)
    s_k = kc.T @ kc
    a = root @ s_k @ root
    lam, e = np.linalg.eigh(0.5 * (a + a.T))
    order = np.argsort(lam)[::-1]
    lam, e = lam[order], e[:, order]
    return root @ e[:, :p], root_inv @ e[:, :p], lam


def score_error(queries: np.ndarray, keys: np.ndarray, keys_hat: np.ndarray) -> float:
    """||Q K^T - Q K_hat^T||_F^2: every query's logit error over every key, summed (eq. 5, left side)."""
    Q = np.asarray(queries, dtype=np.float64)
    diff = Q @ np.asarray(keys, dtype=np.float64).T - Q @ np.asarray(keys_hat, dtype=np.float64).T
    return float(np.sum(diff * diff))


# ----------------------------------------------------------------------------
# online basis update ("OjaKV" README, Method Summary, OjaKV: the low-rank
# subspace is updated with Oja's algorithm during prefill and decoding)
# ----------------------------------------------------------------------------

def oja_update(basis: np.ndarray, x: np.ndarray, eta: float) -> np.ndarray:
    """One step of Oja's subspace rule for the basis of one kv head.

    basis [d, r], x [n, d] (the new tokens' vectors as rows).  Every token t
    projects onto the basis, y_t = x_t B, and pulls the basis towards itself
    along its residual: B <- B + eta * sum_t (x_t - y_t B^T)^T y_t.  The sum
    runs over the tokens of the call against the same B (the batched form of
    the per-token rule), i.e. B + eta (X^T Y - B Y^T Y) with Y = X B.  No
    re-orthonormalisation: for an orthonormal B the step keeps B^T B = I up
    to the second-order term eta^2 (.)^T (.).
    """
    B = np.asarray(basis, dtype=np.float64)
    X = np.asarray(x, dtype=np.float64)
    Y = X @ B
    return B + eta * (X.T @ Y - B @ (Y.T @ Y))


def oja_update_heads(basis: np.ndarray, x: np.ndarray, eta: float) -> np.ndarray:
    """oja_update for every kv head of a chunk: basis [Hkv, d, r], x [B, T, Hkv, d];
    head h is updated from the tokens of every batch row (one basis per kv head)."""
    x = np.asarray(x, dtype=np.float64)
    return np.stack([oja_update(basis[h], x[:, :, h, :].reshape(-1, x.shape[-1]), eta)
                     for h in range(x.shape[2])])
