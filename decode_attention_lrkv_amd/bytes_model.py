"""Algorithmic byte counts: what the method must move through HBM.

Used by the benchmark to turn kernel times into bandwidth.  The counts leave
out what the low-rank path avoids (dense K_hat / V_hat) and the split-K
workspace (reported separately).
"""
from __future__ import annotations


def dense_kv_bytes_per_token(layers: int, n_kv_heads: int, head_dim: int, elem_bytes: int = 2) -> int:
    """Dense K+V cache bytes per token: layers x kv heads x head_dim x 2 (K, V) x element size.

    Llama-3.1-8B in bf16 gives 131072 B (the NovaKV model card's 131.07 KB/token);
    LLaMA-7B (32 kv heads) in fp16 gives 524288 B (the KVQuant catalog record).
    """
    return layers * n_kv_heads * head_dim * 2 * elem_bytes


def lowrank_kv_bytes_per_token(n_kv_heads: int, ranks, elem_bytes: int = 2) -> int:
    """Low-rank cache bytes per token: sum over layers of kv heads x (r_K + r_V) x element size."""
    return sum(n_kv_heads * (rk + rv) * elem_bytes for rk, rv in ranks)


def quantized_bytes_per_token(dense_bytes: int, bits: float, dense_bits: int = 16) -> float:
    """Bytes per token of a cache stored at `bits` average bits per element."""
    return dense_bytes * bits / dense_bits


def decode_bytes(batch, n_q_heads, n_kv_heads, head_dim, rank_k, rank_v, n_ctx, elem_bytes=2,
                 side_tokens=0):
    """One decode layer-step: coefficient rows, bases, query in and output out.

    With a hybrid side list, side_tokens of the n_ctx tokens per (b, kv head)
    are full-rank rows (K and V, d elements each) plus a 4-byte index.
    """
    s = elem_bytes
    lr = n_ctx - side_tokens
    cache = s * batch * n_kv_heads * lr * (rank_k + rank_v)
    side = batch * n_kv_heads * side_tokens * (2 * head_dim * s + 4)
    bases = s * n_kv_heads * head_dim * (rank_k + rank_v)
    io = 2 * s * batch * n_q_heads * head_dim
    return cache + side + bases + io


def split_kernel_bytes(batch, n_q_heads, n_kv_heads, head_dim, rank_k, rank_v, n_ctx, elem_bytes=2):
    """The attention kernel alone: C_K and C_V rows, both bases (B_K folds the
    query, B_V lifts each workgroup's partial) and the queries.  Its float32
    partials (a few KB per workgroup) are workspace traffic, not counted."""
    s = elem_bytes
    return (s * batch * n_kv_heads * n_ctx * (rank_k + rank_v) + s * n_kv_heads * head_dim * (rank_k + rank_v)
            + s * batch * n_q_heads * head_dim)


def step_kernel_bytes(batch, n_q_heads, n_kv_heads, head_dim, rank_k, rank_v, n_ctx, elem_bytes=2):
    """The attention kernel of a decode step: the attention of rows
    [0, n_ctx - 1) (as split_kernel_bytes) plus the appended token, whose key
    and value come in and whose coefficient rows go out."""
    s = elem_bytes
    return (split_kernel_bytes(batch, n_q_heads, n_kv_heads, head_dim, rank_k, rank_v, n_ctx - 1, elem_bytes)
            + s * batch * n_kv_heads * (2 * head_dim + rank_k + rank_v))


def latent_decode_bytes(batch, n_q_heads, n_kv_heads, rank_k, rank_v, n_ctx, elem_bytes=2):
    """Decode with absorbed projections: coefficient rows, r_K-wide queries in
    and r_V-wide outputs out; no basis is read."""
    s = elem_bytes
    return (s * batch * n_kv_heads * n_ctx * (rank_k + rank_v)
            + s * batch * n_q_heads * (rank_k + rank_v))


def compress_bytes(batch, n_tokens, n_kv_heads, head_dim, rank, elem_bytes=2):
    """One compress call: token rows in, basis in, coefficient rows out."""
    s = elem_bytes
    return s * batch * n_tokens * n_kv_heads * (head_dim + rank) + s * n_kv_heads * head_dim * rank


def decode_flops(batch, n_q_heads, n_ctx, rank_k, rank_v):
    """Multiply-adds x 2 of scores and accumulation (fold and lift excluded)."""
    return 2 * batch * n_q_heads * n_ctx * (rank_k + rank_v)


def compress_flops(batch, n_tokens, n_kv_heads, head_dim, rank):
    return 2 * batch * n_tokens * n_kv_heads * head_dim * rank


def oja_bytes(batch, n_tokens, n_kv_heads, head_dim, rank):
    """One Oja update: the chunk's bfloat16 token rows in, the float32 basis in
    and out, its bfloat16 copy out."""
    return (2 * batch * n_tokens * n_kv_heads * head_dim
            + (4 + 4 + 2) * n_kv_heads * head_dim * rank)


def oja_flops(batch, n_tokens, n_kv_heads, head_dim, rank):
    """Multiply-adds x 2 of Y = X B, X^T Y and Y^T Y (the update itself, B S2 and the
    step, is d r (r + 2) per head: negligible)."""
    n = batch * n_tokens * n_kv_heads
    return 2 * n * (2 * head_dim * rank + rank * rank)
