/*
 * lrkv.h -- decode attention over a low-rank KV cache, for AMD Instinct MI355X (gfx950).
 *
 * A low-rank KV cache stores, for every token and kv head, rank-r coefficients
 * of the key and of the value against fixed per-kv-head bases:
 *     C_K = K B_K,   C_V = V B_V,   B_K in R^{d x r_K}, B_V in R^{d x r_V}
 * ("Llama-3.1-NovaKV" model card, introduction: a post-hoc low-rank
 * factorisation of the K and V projections shrinks the cache; "OjaKV" README,
 * Method Summary, StaticPCA: an offline basis, fixed at inference).  A decode
 * step attends one query per q head over the cache without reconstructing K
 * or V: the query is folded into the key latent space, scored against C_K,
 * softmax-weighted, accumulated against C_V and lifted back through B_V^T.
 * The result equals standard attention over K_hat = C_K B_K^T and
 * V_hat = C_V B_V^T, which is how StaticPCA attends (same README section).
 * The hybrid variant keeps tokens whose reconstruction error is high in full
 * rank in a side list and attends both kinds in one softmax ("OjaKV" README,
 * Method Summary, OjaKV).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All pointers to tensors are DEVICE pointers, 16-byte aligned, to dense
 *   row-major arrays in the layouts stated per argument.  The caller
 *   allocates and owns every buffer (inputs, outputs, caches, counters,
 *   workspace); the library allocates no device memory and keeps no state
 *   beyond a per-device compute-unit count, a thread-local error string and
 *   the fixed scratch array of lrkv_decode_step_noalloc (a static device
 *   array of the library, not an allocation).
 * - One storage dtype (lrkv_dtype) for every floating-point tensor of a call;
 *   lse and workspaces are float32.  Arithmetic accumulates in float32;
 *   rounding to bfloat16 is round-to-nearest-even.
 * - Grouped-query attention: q head h reads kv head h / (Hq / Hkv).
 * - Bases and transforms: a cache row is c = x E for an encoder E and is read
 *   back as x_hat = c D^T for a decoder D, both [Hkv, d, r].  With an
 *   orthonormal basis B (StaticPCA) E = D = B and one array serves both.
 *   A non-orthogonal transform passes E where a call encodes (lrkv_compress,
 *   lrkv_compress_kv, the enc_k of a decode step) and D where it decodes
 *   (basis_k folds the query, basis_v lifts the output), with D^T E = I:
 *   the attention-aware key transform of the NOVA-KV summary (Methodology,
 *   Key Transform Derivation, Theorem 1: R_K = M_q^(1/2) E, keys recovered
 *   through R_K^-1) is such a pair.  Its value transform is orthogonal (same
 *   summary, Value Transform, Corollary 1), so the decode step takes a
 *   separate encoder for keys only.  The hybrid cache assumes an orthonormal
 *   basis (its residual test reconstructs with the encoding basis).
 * - Layouts ("B" batch, "Hq"/"Hkv" query/kv heads, "d" head_dim, "cap" cache
 *   capacity in tokens):
 *     keys, row layout:     key coefficient cache [B, Hkv, cap, r_K],
 *                           full-rank key side list [B, Hkv, side_cap, d]
 *     values, octet layout: value coefficient cache [B, Hkv, cap/8, r_V, 8],
 *                           full-rank value side list [B, Hkv, side_cap/8, d, 8]
 *   In the octet layout element (t, c) of a token-by-column matrix lives at
 *   ((t / 8) * ncols + c) * 8 + t % 8: each column's 8 consecutive tokens are
 *   contiguous.  cap and side_cap must be multiples of 8.
 *   Value caches and value side lists are ONLY read and written in the octet
 *   layout: a value array in the row layout [B, Hkv, cap, r_V] is not
 *   accepted, and since a pointer does not carry its layout, passing one
 *   returns LRKV_OK with wrong results.
 * - Every call is asynchronous on `stream` (0 = the null stream), allocates
 *   nothing and synchronizes nothing, so it can be captured in a HIP graph.
 * - Errors: arguments are validated before any HIP call; an invalid call
 *   returns a non-zero lrkv_status, launches nothing and leaves a message in
 *   lrkv_last_error().  A failed launch returns LRKV_ERR_DEVICE.  Faults
 *   during kernel execution surface at the caller's next synchronization.
 *   No C++ exception crosses this interface.
 * - Supported shapes: head_dim in {64, 128}; 1 <= rank <= head_dim; ranks a
 *   multiple of 8 for bfloat16 and of 4 for float32; Hq a multiple of Hkv with
 *   Hq / Hkv <= 8; B, Hkv >= 1.
 */
#ifndef LRKV_H
#define LRKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lrkv_status {
  LRKV_OK = 0,
  LRKV_ERR_INVALID_ARGUMENT = 1,   /* null pointer, misaligned pointer, inconsistent sizes */
  LRKV_ERR_UNSUPPORTED = 2,        /* valid request outside the supported shapes */
  LRKV_ERR_WORKSPACE_TOO_SMALL = 3,
  LRKV_ERR_DEVICE = 4              /* a HIP runtime call failed; see lrkv_last_error() */
} lrkv_status;

typedef enum lrkv_dtype { LRKV_F32 = 0, LRKV_BF16 = 1 } lrkv_dtype;

/* Which cache a compress call writes: keys use the row layout, values the octet layout. */
typedef enum lrkv_cache_kind { LRKV_KEYS = 0, LRKV_VALUES = 1 } lrkv_cache_kind;

typedef struct lrkv_dims {
  int32_t batch;        /* B */
  int32_t n_q_heads;    /* Hq */
  int32_t n_kv_heads;   /* Hkv */
  int32_t head_dim;     /* d */
  int32_t rank_k;       /* r_K */
  int32_t rank_v;       /* r_V */
  int64_t capacity;     /* cap: tokens the coefficient caches hold per (b, kv head) */
} lrkv_dims;

/*
 * Compress / append (the cache write).
 *   coeff[b, h, pos + t, :] = x[b, t, h, :] @ basis[h]      for t in [0, n_tokens)
 * ("Llama-3.1-NovaKV" model card: the cache holds the low-rank factors of K
 * and V; "OjaKV" README, StaticPCA: a fixed offline basis.)  One call writes
 * one cache (K or V) with its own basis and rank.
 *   x      [B, n_tokens, Hkv, d]   the new tokens' full keys or values
 *   basis  [Hkv, d, rank]          the encoder: an orthonormal basis, or the
 *                                  encoding half of a transform (not checked)
 *   coeff  key row layout [B, Hkv, capacity, rank] (kind = LRKV_KEYS) or
 *          value octet layout [B, Hkv, capacity/8, rank, 8] (kind = LRKV_VALUES)
 * Rows outside [pos, pos + n_tokens) are not touched.  n_tokens = 0 is a no-op.
 * Requires pos >= 0 and pos + n_tokens <= capacity.
 */
lrkv_status lrkv_compress(const void* x, const void* basis, void* coeff, lrkv_cache_kind kind,
                          int32_t batch, int32_t n_kv_heads, int32_t head_dim, int32_t rank,
                          int64_t n_tokens, int64_t pos, int64_t capacity, lrkv_dtype dtype,
                          hipStream_t stream);

/*
 * Both caches of a layer in one call: lrkv_compress of the keys (row layout,
 * rank_k) and of the values (octet layout, rank_v), with the shapes of dims
 * (n_q_heads is not used).  Up to 4 tokens (an appended decode token) are
 * compressed in a single launch that reads the bases straight from memory;
 * longer chunks use the matrix-core path of lrkv_compress for each cache.
 *   xk, xv  [B, n_tokens, Hkv, d]
 */
lrkv_status lrkv_compress_kv(const void* xk, const void* xv, const void* basis_k, const void* basis_v,
                             void* coeff_k, void* coeff_v, const lrkv_dims* dims, int64_t n_tokens,
                             int64_t pos, lrkv_dtype dtype, hipStream_t stream);

/*
 * Bytes of workspace lrkv_decode_attn (side_cap = 0) or
 * lrkv_decode_attn_hybrid (side_cap > 0) needs for these dims.  n_ctx is the
 * context length of a plain decode; the hybrid decode plans for
 * dims->capacity and side_cap instead.  Returns 0 for invalid dims.  The
 * split plan depends on the current device's compute-unit count, so query on
 * the device that will run the call.
 * The workspace starts with one 32-bit arrival counter per (b, kv head)
 * (rounded up to 256 bytes) that the calls merging in their own launch use
 * (lrkv_decode_attn_hybrid, and the small bfloat16 launches of
 * lrkv_decode_attn, lrkv_decode_step and their _seqlens forms): these words
 * must be zero before a workspace's first call (allocate the workspace
 * zeroed), and every call of any decode entry point leaves them zero.  The rest is scratch.  Calls that
 * share a workspace must be ordered on one stream (they must not overlap in
 * time; overlapping hybrid calls on one workspace would also share its
 * counters).
 */
size_t lrkv_decode_workspace_bytes(const lrkv_dims* dims, int64_t n_ctx, int64_t side_cap);

/*
 * Decode attention of one query per q head over tokens [0, n_ctx) of a
 * low-rank cache (the token appended at this step included):
 *   q' = q B_K[h] * scale,  s_t = q' . C_K[t],  p = softmax(s),
 *   acc = sum_t p_t C_V[t],  out = acc B_V[h]^T,  lse = log sum_t exp(s_t)
 * which equals softmax(q K_hat^T * scale) V_hat with K_hat = C_K B_K^T and
 * V_hat = C_V B_V^T ("OjaKV" README, StaticPCA: standard attention over
 * keys and values reconstructed from the low-rank cache).  The context is
 * split into chunks attended in parallel (one launch) and the partial
 * results are merged by log-sum-exp (a second launch; for bfloat16 launches
 * of at most a quarter as many workgroups as the GPU has compute units, the
 * last workgroup of each (b, kv head) merges in the same launch instead,
 * using the workspace's arrival counters).  For bfloat16, when one
 * workgroup per (b, kv head) covers the whole context (short contexts),
 * that workgroup normalises and writes out and lse itself: one launch.
 *   q        [B, Hq, d]
 *   basis_k  [Hkv, d, r_K];   coeff_k  key row layout [B, Hkv, capacity, r_K]
 *   basis_v  [Hkv, d, r_V];   coeff_v  value octet layout [B, Hkv, capacity/8, r_V, 8]
 *            (the decoders: the basis itself, or a transform's decoding half)
 *   out      [B, Hq, d] (storage dtype);  lse [B, Hq] float32 natural log, or NULL
 *   scale    softmax scale; 0 selects 1/sqrt(head_dim)
 *   workspace at least lrkv_decode_workspace_bytes(dims, n_ctx, 0) bytes
 * Requires 1 <= n_ctx <= capacity.
 */
lrkv_status lrkv_decode_attn(const void* q, const void* basis_k, const void* coeff_k,
                             const void* basis_v, const void* coeff_v, void* out, float* lse,
                             const lrkv_dims* dims, int64_t n_ctx, float scale, lrkv_dtype dtype,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The two phases of lrkv_decode_attn, callable separately (same arguments,
 * same workspace, same result when called back to back on one stream):
 *   _partial  attends the context in splits; each workgroup of splits merges
 *             its splits and lifts the result through B_V^T, leaving per
 *             (b, q head, workgroup) a running max, a softmax sum and an
 *             unnormalised head_dim-wide output in the workspace;
 *   _merge    combines those by log-sum-exp into out and lse.
 * The split plan is a function of dims, n_ctx and the device, so both phases
 * must see the same values.  Splitting the call lets a caller time the phases
 * or combine partial results computed elsewhere (for example on other GPUs,
 * each holding a range of the context) before the merge.
 */
lrkv_status lrkv_decode_attn_partial(const void* q, const void* basis_k, const void* coeff_k,
                                     const void* basis_v, const void* coeff_v, const lrkv_dims* dims,
                                     int64_t n_ctx, float scale, lrkv_dtype dtype, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);
lrkv_status lrkv_decode_attn_merge(void* out, float* lse, const lrkv_dims* dims, int64_t n_ctx,
                                   lrkv_dtype dtype, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/*
 * Decode attention with the bases absorbed into the model's projections.
 * The NovaKV delta ships modified query and output projections together
 * with the K and V factors ("Llama-3.1-NovaKV" model card, introduction);
 * with W_q B_K and B_V^T W_o formed offline, a query arrives as
 * q' = q B_K and the layer needs only the latent output
 *   s_t = q' . C_K[t] * scale,  p = softmax(s),  out_lat = sum_t p_t C_V[t]
 * (lse as lrkv_decode_attn).  No basis is read; the query fold and the
 * output lift of lrkv_decode_attn are left to the absorbed projections.
 *   q_lat    [B, Hq, r_K] latent queries (storage dtype)
 *   coeff_k  key row layout [B, Hkv, capacity, r_K]
 *   coeff_v  value octet layout [B, Hkv, capacity/8, r_V, 8]
 *   out_lat  [B, Hq, r_V] (storage dtype);  lse [B, Hq] float32, or NULL
 *   scale    softmax scale; 0 selects 1/sqrt(dims->head_dim), the model's
 *            head dimension (dims->head_dim also sets the supported shapes)
 *   workspace at least lrkv_decode_workspace_bytes(dims, n_ctx, 0) bytes
 * Requires 1 <= n_ctx <= capacity.
 */
lrkv_status lrkv_decode_attn_latent(const void* q_lat, const void* coeff_k, const void* coeff_v, void* out_lat,
                                    float* lse, const lrkv_dims* dims, int64_t n_ctx, float scale, lrkv_dtype dtype,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Decode step: append the token of this step, then attend.  Equivalent to
 * lrkv_compress_kv of one token at row n_ctx - 1 followed by
 * lrkv_decode_attn over [0, n_ctx) (the "Llama-3.1-NovaKV" model card,
 * results section, times whole decode steps with the cache written and read
 * inside the step; the cache row is c = round(x E) as in lrkv_compress).
 * For bfloat16 the append runs inside the attention launch: per (b, kv head)
 * one workgroup (an extra one when the grid has room for it, else the last
 * attention workgroup, after its fold) compresses the token, stores its rows
 * and contributes its softmax term, while the others attend rows
 * [0, n_ctx - 1); a second launch merges.  When one attention workgroup per
 * (b, kv head) covers rows [0, n_ctx - 1) (short contexts), it also appends
 * and writes out and lse itself: one launch.  Small bfloat16 launches
 * without a separate key encoder merge in the launch, as lrkv_decode_attn.
 * float32 runs lrkv_compress_kv, then the decode.  The two-phase entry
 * points below always use the partials and the merge launch.
 *   k_new, v_new  [B, Hkv, d] the new token's key and value
 *   basis_k, basis_v  the decoders (fold and lift), as in lrkv_decode_attn
 *   coeff_k, coeff_v  the caches (row n_ctx - 1 is written; rows below are read)
 *   enc_k    [Hkv, d, r_K] encoder of the new key, or NULL when basis_k is an
 *            orthonormal basis that also encodes (the value is encoded by basis_v)
 *   workspace at least lrkv_decode_step_workspace_bytes(dims, n_ctx) bytes,
 *             laid out (arrival counters first, zero before the first call)
 *             as described at lrkv_decode_workspace_bytes
 * Other arguments as lrkv_decode_attn.  Requires 1 <= n_ctx <= capacity.
 */
size_t lrkv_decode_step_workspace_bytes(const lrkv_dims* dims, int64_t n_ctx);
lrkv_status lrkv_decode_step(const void* q, const void* k_new, const void* v_new, const void* basis_k,
                             void* coeff_k, const void* basis_v, void* coeff_v, const void* enc_k, void* out,
                             float* lse, const lrkv_dims* dims, int64_t n_ctx, float scale, lrkv_dtype dtype,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The two phases of lrkv_decode_step (same arguments and workspace, same
 * result back to back on one stream), as for lrkv_decode_attn: _partial
 * appends the token and leaves the partial results in the workspace, _merge
 * combines them into out and lse.
 */
lrkv_status lrkv_decode_step_partial(const void* q, const void* k_new, const void* v_new, const void* basis_k,
                                     void* coeff_k, const void* basis_v, void* coeff_v, const void* enc_k,
                                     const lrkv_dims* dims, int64_t n_ctx, float scale, lrkv_dtype dtype,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);
lrkv_status lrkv_decode_step_merge(void* out, float* lse, const lrkv_dims* dims, int64_t n_ctx, lrkv_dtype dtype,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Decode with the context lengths on the device, so that one captured HIP
 * graph serves a decode that advances ("Llama-3.1-NovaKV" model card, results
 * section: decode runs from a fixed-shape cache through a captured graph; a
 * graph replays its launches with the same arguments, so a length the host
 * passes by value would be frozen into it).  Same computation as
 * lrkv_decode_attn / lrkv_decode_step, with sequence b of the batch taking
 * its own length n = seq_lens[b]:
 *   _attn_seqlens   attends rows [0, n) of sequence b;
 *   _step_seqlens   appends the step's token at row n - 1 of sequence b
 *                   (compress as lrkv_decode_step) and attends rows [0, n).
 * A length outside [1, capacity] gives out = 0 and lse = -inf for that
 * sequence's heads, and the step writes no cache row for it.
 *   seq_lens     [B] int32, device, read only (the caller advances it, for
 *                example with a kernel of its own recorded in the same graph)
 *   max_seq_len  host upper bound the split plan is made for, in
 *                [1, capacity]; any lengths are attended correctly, but
 *                lengths far above it use fewer workgroups than the chip has
 *   workspace    at least lrkv_decode_workspace_bytes(dims, max_seq_len, 0)
 *                (_attn_seqlens) or lrkv_decode_step_workspace_bytes(dims,
 *                max_seq_len) (_step_seqlens) bytes
 * Other arguments as lrkv_decode_attn / lrkv_decode_step.  bfloat16 only.
 */
lrkv_status lrkv_decode_attn_seqlens(const void* q, const void* basis_k, const void* coeff_k,
                                     const void* basis_v, const void* coeff_v, void* out, float* lse,
                                     const lrkv_dims* dims, const int32_t* seq_lens, int64_t max_seq_len,
                                     float scale, lrkv_dtype dtype, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);
lrkv_status lrkv_decode_step_seqlens(const void* q, const void* k_new, const void* v_new, const void* basis_k,
                                     void* coeff_k, const void* basis_v, void* coeff_v, const void* enc_k, void* out,
                                     float* lse, const lrkv_dims* dims, const int32_t* seq_lens, int64_t max_seq_len,
                                     float scale, lrkv_dtype dtype, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/*
 * lrkv_decode_step without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments (minus the workspace),
 * same kernels and same result as lrkv_decode_step.  The workspace is a fixed
 * device array inside this library of lrkv_decode_step_noalloc_max_bytes()
 * bytes (8 MiB) per GPU, held until the process ends; each GPU has its own.
 * The array is zero when the library loads, and every call leaves its
 * arrival counters zero, as lrkv_decode_step requires of a workspace.
 * Calls whose lrkv_decode_step_workspace_bytes(dims, n_ctx) exceeds that size
 * return LRKV_ERR_WORKSPACE_TOO_SMALL before any device call.  The call
 * allocates nothing.  All calls on one GPU share that GPU's array: calls that
 * overlap in time on one GPU (other streams, other threads) race, so order
 * them on one stream.  The first call on a device looks up the array's
 * address there (LRKV_ERR_DEVICE if that fails).
 */
size_t lrkv_decode_step_noalloc_max_bytes(void);
lrkv_status lrkv_decode_step_noalloc(const void* q, const void* k_new, const void* v_new, const void* basis_k,
                                     void* coeff_k, const void* basis_v, void* coeff_v, const void* enc_k, void* out,
                                     float* lse, const lrkv_dims* dims, int64_t n_ctx, float scale, lrkv_dtype dtype,
                                     hipStream_t stream);

/* Bytes of workspace lrkv_compress_hybrid needs for n_tokens new tokens. */
size_t lrkv_compress_hybrid_workspace_bytes(const lrkv_dims* dims, int64_t n_tokens);

/*
 * Hybrid compress ("OjaKV" README, Method Summary, OjaKV: tokens with high
 * reconstruction error are kept in full rank, the rest are compressed).
 * For every new token t of (b, h) with key k and value v:
 *   c = round(x B) (the stored coefficients), x_hat = c B^T,
 *   selected(x) = ||x - x_hat||^2 > tau^2 ||x||^2   (evaluated in float32),
 *   flag_t = selected(k) or selected(v).
 * Unflagged tokens are appended, in ascending t, to the low-rank caches at
 * rows n_lr[b, h], n_lr[b, h] + 1, ...; flagged tokens are appended, in
 * ascending t, to the full-rank side lists at n_side[b, h], ... with
 * side_idx = pos + t.  n_lr and n_side are then advanced.  Selection and
 * placement are deterministic (no dependence on execution order).
 *   k, v      [B, n_tokens, Hkv, d]
 *   tau       >= 0 (+inf keeps every token low rank); tokens of zero norm are never flagged
 *   coeff_k / coeff_v   key row / value octet layout caches (dims->capacity tokens)
 *   n_lr, n_side        [B, Hkv] int32, device, in/out (the caller zeroes them once)
 *   k_side    key row layout [B, Hkv, side_cap, d]; v_side value octet layout
 *             [B, Hkv, side_cap/8, d, 8]; side_idx [B, Hkv, side_cap] int32
 *   flags     [B, Hkv, n_tokens] uint8 (1 = full rank), or NULL
 *   overflow  device int32, set to 1 when a low-rank cache or a side list is
 *             full; the tokens that do not fit are dropped and the counts stop
 *             at the capacities.  The caller zeroes it.
 *   workspace at least lrkv_compress_hybrid_workspace_bytes(dims, n_tokens) bytes
 * Only bfloat16 is supported for the hybrid cache.
 */
lrkv_status lrkv_compress_hybrid(const void* k, const void* v, const void* basis_k,
                                 const void* basis_v, float tau, void* coeff_k, void* coeff_v,
                                 int32_t* n_lr, void* k_side, void* v_side, int32_t* side_idx,
                                 int32_t* n_side, uint8_t* flags, int32_t* overflow,
                                 const lrkv_dims* dims, int64_t n_tokens, int64_t pos,
                                 int64_t side_cap, lrkv_dtype dtype, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * Hybrid decode: one softmax over the n_lr[b, h] low-rank tokens and the
 * n_side[b, h] full-rank side-list tokens of each (b, kv head)
 * ("OjaKV" README, Method Summary, OjaKV):
 *   out = (sum_lr p_t C_V[t] B_V^T + sum_side p_j v_j),  p = softmax over both sets
 * with s_t = q' . C_K[t] for low-rank tokens and s_j = scale q . k_j for side tokens.
 * Counts are read on the device; an empty (b, h) gives out = 0, lse = -inf.
 * Each (b, kv head) gets a fixed number of workgroups, divided between the
 * two lists on the device in proportion to the bytes the counts there
 * describe; the workgroup of each (b, kv head) that finishes last merges
 * the partials in the same launch (one launch per call).  bfloat16 only.
 *   workspace at least lrkv_decode_workspace_bytes(dims, 0, side_cap) bytes,
 *             its arrival counters zero (see lrkv_decode_workspace_bytes);
 *             the call leaves them zero.
 */
lrkv_status lrkv_decode_attn_hybrid(const void* q, const void* basis_k, const void* coeff_k,
                                    const void* basis_v, const void* coeff_v,
                                    const int32_t* n_lr, const void* k_side, const void* v_side,
                                    const int32_t* n_side, int64_t side_cap, void* out,
                                    float* lse, const lrkv_dims* dims, float scale,
                                    lrkv_dtype dtype, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* Bytes of workspace lrkv_oja_update needs. */
size_t lrkv_oja_workspace_bytes(int32_t batch, int32_t n_kv_heads, int32_t head_dim, int32_t rank,
                                int64_t n_tokens);

/*
 * Online basis update by Oja's subspace rule ("OjaKV" README, Method
 * Summary, OjaKV: the low-rank subspace is updated online with Oja's
 * algorithm, in prefill and in decoding).  For every kv head h, with the
 * n_tokens new tokens x_t of every batch row as the rows of X:
 *   Y = X B[h],   B[h] <- B[h] + eta (X^T Y - B[h] Y^T Y)
 * i.e. the per-token rule B <- B + eta (x - y B^T)^T y summed over the
 * chunk's tokens against the same B.  No re-orthonormalisation (the rule
 * keeps B^T B = I to first order in eta); coefficients already in a cache
 * are left as they are.
 *   x           [B, n_tokens, Hkv, d] bfloat16 (a chunk, as for lrkv_compress)
 *   basis       [Hkv, d, rank] float32, read and overwritten: the basis kept
 *               at full precision, since steps of this size vanish in bfloat16
 *   basis_bf16  [Hkv, d, rank] bfloat16, written with the updated basis
 *               rounded to nearest even (the copy the compress and decode
 *               calls take), or NULL
 *   eta         step size (finite)
 *   workspace   at least lrkv_oja_workspace_bytes(...) bytes, 16-byte aligned;
 *               scratch, no initial contents needed
 * head_dim 64 or 128; rank a multiple of 8, at most head_dim.  The result
 * is deterministic (fixed summation order).  n_tokens = 0 leaves the basis
 * as it is (x may then be NULL).  Up to 64 tokens per head: one launch;
 * more: three (the chunk's Gram matrix G = X^T X per run of tokens, then
 * X^T Y = G B, then the step with B Y^T Y = (B B^T) G B).
 */
lrkv_status lrkv_oja_update(const void* x, float* basis, void* basis_bf16, int32_t batch,
                            int32_t n_kv_heads, int32_t head_dim, int32_t rank, int64_t n_tokens,
                            float eta, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static description of a status code. */
const char* lrkv_status_string(lrkv_status status);

/* Detail of the last non-OK status returned on this thread ("" if none). */
const char* lrkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LRKV_H */
