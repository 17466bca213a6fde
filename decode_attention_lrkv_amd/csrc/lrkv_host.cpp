// C-ABI layer of liblrkv: argument validation, split planning, workspace
// layout and kernel launches.  No device memory is allocated here.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "lrkv.h"
#include "lrkv_internal.h"

using namespace lrkv;

namespace {
thread_local std::string g_last_error;
}  // namespace

namespace lrkv {
lrkv_status fail(lrkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}
}  // namespace lrkv

namespace {

lrkv_status device_fail(const char* fn, hipError_t e) {
  return fail(LRKV_ERR_DEVICE, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Compute units of the current device (cached); 256 when no device answers.
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

struct Plan {
  int n_splits = 1;
  int chunks_per_split = 1;
};

// Split a context of n_tokens over (units) independent (batch, kv head) rows so
// that one round of workgroups fills the chip (8 resident waves per compute
// unit at the split kernel's register use; one and a half rounds for many
// units, below), with at least 4 chunks (128
// tokens) per split.  When that still leaves several workgroups per unit but
// few units (batch-1 decodes, bound by each wave's chain of dependent work,
// not by bytes), the splits go down to one chunk each, as long as the launch
// keeps to one workgroup per compute unit (one workgroup of four splits per
// unit kept free for a decode step's appended token): on the batch-1
// 32-layer step at 2048 tokens (64 chunks per unit) 64 splits per unit took
// 423.8 us per graph replay against 487.9 us with 16, and at 8192 tokens
// 124 splits (3 chunks per wave, 184 workgroups) 481.6 against 509.9 us with
// 64, while 128 splits (2 chunks per wave, 264 workgroups, two on some
// compute units) took 577 us.  A context that one workgroup per unit covers
// (at most 16 chunks) keeps that single workgroup, which also writes the
// outputs (no merge): at 256 tokens 342.5 against 397 us with more splits.
// LRKV_SPLITS forces the split count.
Plan plan_splits(int64_t units, int64_t n_tokens, int cus, int max_splits) {
  Plan p;
  const int64_t n_chunks = n_tokens > 0 ? cdiv(n_tokens, kChunk) : 1;
  const int64_t u = units > 0 ? units : 1;
  int64_t s = cdiv((int64_t)cus * 8, u);
  // Many units (a batch of sequences, bandwidth-bound): one and a half
  // rounds, so that the hardware dispatcher hands the last half round to the
  // compute units that finish first (the batched 32K step: 188.8 against
  // 190.4-190.7 us per layer-step, alternating runs on one box; two full
  // rounds 192.3 us).
  // (only where whole workgroups of four splits per unit make it at most one
  // and a half rounds: 768 workgroups at 256 compute units)
  if (2 * u >= cus) {
    const int64_t s15 = cdiv((int64_t)cus * 12, u);
    if (cdiv(s15, 4) * u <= 3 * (int64_t)cus) s = s15;
  }
  s = std::min<int64_t>(s, cdiv(n_chunks, 4));
  if (s > 4) s = std::max<int64_t>(s, std::min<int64_t>(n_chunks, (int64_t)cus * 4 / u - 4));
  if (const char* env = std::getenv("LRKV_SPLITS")) {
    const long v = std::strtol(env, nullptr, 10);
    if (v > 0) s = v;
  }
  s = std::max<int64_t>(1, std::min<int64_t>(s, n_chunks));
  s = std::min<int64_t>(s, max_splits);
  const int64_t cps = cdiv(n_chunks, s);
  p.chunks_per_split = (int)cps;
  p.n_splits = (int)cdiv(n_chunks, cps);
  return p;
}

// Decode workspace: arrival counters [B, Hkv] (uint32, used by the launches
// that merge in the launch: the hybrid decode and small bfloat16 plain and
// step launches; zero at rest), the partials [B, Hq, parts, d]
// and their (max, sum) [B, Hq, parts, 2].  The counters come first in every
// layout, so calls of any kind that share a workspace leave them alone.
struct DecodeLayout {
  Plan lr;             // plain decode: splits of the context
  int parts = 0;       // partials per (b, q head): one per attention workgroup
  size_t cnt = 0, o = 0, ml = 0, total = 0;
};

// append (decode step): one more partial slot, the appended token's, which
// stays empty (max -inf): the appending workgroup adds the token to its own
// partial.  The token is compressed by one more workgroup per (b, kv head)
// when the grid still fits one round of two workgroups per compute unit
// (then it runs beside the attention), else by the last attention workgroup
// before its own chunks.
DecodeLayout decode_layout(const lrkv_dims& d, int64_t n_lr_tokens, int64_t side_cap, bool append = false) {
  DecodeLayout L;
  const int cus = device_cu_count();
  const int64_t units = (int64_t)d.batch * d.n_kv_heads;
  const int64_t rows = (int64_t)d.batch * d.n_q_heads;
  if (side_cap > 0) {
    // hybrid: one workgroup per compute unit (measured faster than two: the
    // streams stay as long as possible and the merge has half the partials),
    // divided between the two lists on the device; at least one per list,
    // and no more than one chunk per wave of the largest possible lists
    const int64_t chunks = cdiv(n_lr_tokens, kChunk) + cdiv(side_cap, kChunk);
    int64_t p = (int64_t)cus / units;
    p = std::min<int64_t>(p, cdiv(chunks, kSplitsPerPart));
    p = std::min<int64_t>(p, kMaxSplits / kSplitsPerPart);
    if (const char* env = std::getenv("LRKV_HYBRID_WGS")) {   // forced workgroups per (b, kv head)
      const long v = std::strtol(env, nullptr, 10);
      if (v > 0) p = std::min<long>(v, kMaxSplits / kSplitsPerPart);
    }
    L.parts = (int)std::max<int64_t>(2, p);
  } else {
    L.lr = plan_splits(units, n_lr_tokens, cus, kMaxSplits);
    L.parts = (int)cdiv(L.lr.n_splits, kSplitsPerPart);
    if (append) {
      const bool own_wg = (int64_t)(L.parts + 1) * units <= 2 * (int64_t)cus;
      L.parts += own_wg ? 2 : 1;   // workgroups (the appending one included) + the token's slot, left empty
    }
  }
  size_t off = 0;
  L.cnt = off;      off = align256(off + sizeof(uint32_t) * units);
  L.o = off;        off = align256(off + sizeof(float) * rows * L.parts * d.head_dim);
  L.ml = off;       off = align256(off + sizeof(float) * rows * L.parts * 2);
  L.total = off;
  return L;
}

lrkv_status check_rank(int32_t r, int32_t hd, lrkv_dtype dt, const char* fn, const char* what) {
  const int mult = dt == LRKV_BF16 ? 8 : 4;
  if (r < 1 || r > hd)
    return fail(LRKV_ERR_UNSUPPORTED, "%s: %s = %d outside [1, head_dim = %d]", fn, what, r, hd);
  if (r % mult)
    return fail(LRKV_ERR_UNSUPPORTED, "%s: %s = %d is not a multiple of %d", fn, what, r, mult);
  return LRKV_OK;
}

lrkv_status check_dims(const lrkv_dims* d, lrkv_dtype dt, const char* fn) {
  if (!d) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: dims is NULL", fn);
  if (dt != LRKV_F32 && dt != LRKV_BF16) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", fn, (int)dt);
  if (d->batch < 1 || d->n_kv_heads < 1 || d->n_q_heads < 1)
    return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: batch, n_q_heads and n_kv_heads must be >= 1", fn);
  if (d->batch > 65535 || d->n_kv_heads > 65535)
    return fail(LRKV_ERR_UNSUPPORTED, "%s: batch and n_kv_heads must be <= 65535", fn);
  if (d->n_q_heads % d->n_kv_heads)
    return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: n_q_heads = %d is not a multiple of n_kv_heads = %d", fn,
                d->n_q_heads, d->n_kv_heads);
  if (d->n_q_heads / d->n_kv_heads > 8)
    return fail(LRKV_ERR_UNSUPPORTED, "%s: more than 8 query heads per kv head", fn);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(LRKV_ERR_UNSUPPORTED, "%s: head_dim = %d (supported: 64, 128)", fn, d->head_dim);
  lrkv_status st = check_rank(d->rank_k, d->head_dim, dt, fn, "rank_k");
  if (st != LRKV_OK) return st;
  st = check_rank(d->rank_v, d->head_dim, dt, fn, "rank_v");
  if (st != LRKV_OK) return st;
  if (d->capacity < 8 || d->capacity % 8)
    return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: capacity = %lld must be a positive multiple of 8", fn,
                (long long)d->capacity);
  // the kernels address one (batch, kv head) of a cache with 31-bit byte offsets
  const int64_t elem = dt == LRKV_BF16 ? 2 : 4;
  const int64_t widest = std::max<int64_t>(d->rank_k, d->rank_v);
  if (d->capacity * widest * elem >= ((int64_t)1 << 31))
    return fail(LRKV_ERR_UNSUPPORTED, "%s: capacity %lld too large (capacity x rank x element size must be < 2^31)",
                fn, (long long)d->capacity);
  return LRKV_OK;
}

#define LRKV_CHECK_PTR(p, fn)                                                              \
  do {                                                                                     \
    if (!(p)) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: %s is NULL", fn, #p);            \
    if (!aligned16(p)) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: %s is not 16-byte aligned", fn, #p); \
  } while (0)

// Gram workgroups per kv head for an Oja update: one per compute unit over
// all heads, no more than there are 128-token steps.  (One per compute unit
// rather than two: every workgroup writes a d x d partial, which the s1
// launch reads back.)
int oja_workgroups(int hkv, int64_t tokens) {
  const int64_t steps = std::max<int64_t>(1, (tokens + kOjaGramStep - 1) / kOjaGramStep);
  const int64_t per_head = std::max<int64_t>(1, (int64_t)device_cu_count() / std::max(1, hkv));
  return (int)std::min<int64_t>(std::min<int64_t>(steps, per_head), 65535);
}

float resolve_scale(float scale, int head_dim) {
  return scale == 0.f ? 1.f / std::sqrt((float)head_dim) : scale;
}

}  // namespace

extern "C" {

const char* lrkv_status_string(lrkv_status s) {
  switch (s) {
    case LRKV_OK: return "ok";
    case LRKV_ERR_INVALID_ARGUMENT: return "invalid argument";
    case LRKV_ERR_UNSUPPORTED: return "unsupported";
    case LRKV_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case LRKV_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* lrkv_last_error(void) { return g_last_error.c_str(); }

lrkv_status lrkv_compress(const void* x, const void* basis, void* coeff, lrkv_cache_kind kind,
                          int32_t batch, int32_t n_kv_heads, int32_t head_dim, int32_t rank,
                          int64_t n_tokens, int64_t pos, int64_t capacity, lrkv_dtype dtype,
                          hipStream_t stream) {
  const char* fn = "lrkv_compress";
  if (dtype != LRKV_F32 && dtype != LRKV_BF16) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: unknown dtype", fn);
  if (kind != LRKV_KEYS && kind != LRKV_VALUES) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: unknown cache kind", fn);
  if (batch < 1 || n_kv_heads < 1) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: batch and n_kv_heads must be >= 1", fn);
  if (batch > 65535 || n_kv_heads > 65535) return fail(LRKV_ERR_UNSUPPORTED, "%s: batch and n_kv_heads must be <= 65535", fn);
  if (head_dim != 64 && head_dim != 128)
    return fail(LRKV_ERR_UNSUPPORTED, "%s: head_dim = %d (supported: 64, 128)", fn, head_dim);
  lrkv_status st = check_rank(rank, head_dim, dtype, fn, "rank");
  if (st != LRKV_OK) return st;
  if (capacity < 8 || capacity % 8)
    return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: capacity = %lld must be a positive multiple of 8", fn, (long long)capacity);
  if (n_tokens < 0 || pos < 0 || pos + n_tokens > capacity)
    return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: rows [%lld, %lld) do not fit capacity %lld", fn, (long long)pos,
                (long long)(pos + n_tokens), (long long)capacity);
  LRKV_CHECK_PTR(x, fn);
  LRKV_CHECK_PTR(basis, fn);
  LRKV_CHECK_PTR(coeff, fn);
  if (n_tokens == 0) return LRKV_OK;
  CompressArgs a{x, basis, coeff, kind == LRKV_VALUES ? 1 : 0, batch, n_kv_heads, head_dim, rank,
                 n_tokens, pos, capacity};
  const hipError_t e = dtype == LRKV_BF16 ? launch_compress_bf16(a, stream) : launch_compress_f32(a, stream);
  return e == hipSuccess ? LRKV_OK : device_fail(fn, e);
}

lrkv_status lrkv_compress_kv(const void* xk, const void* xv, const void* basis_k, const void* basis_v,
                             void* coeff_k, void* coeff_v, const lrkv_dims* dims, int64_t n_tokens,
                             int64_t pos, lrkv_dtype dtype, hipStream_t stream) {
  const char* fn = "lrkv_compress_kv";
  lrkv_status st = check_dims(dims, dtype, fn);
  if (st != LRKV_OK) return st;
  if (n_tokens < 0 || pos < 0 || pos + n_tokens > dims->capacity)
    return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: rows [%lld, %lld) do not fit capacity %lld", fn, (long long)pos,
                (long long)(pos + n_tokens), (long long)dims->capacity);
  LRKV_CHECK_PTR(xk, fn);
  LRKV_CHECK_PTR(xv, fn);
  LRKV_CHECK_PTR(basis_k, fn);
  LRKV_CHECK_PTR(basis_v, fn);
  LRKV_CHECK_PTR(coeff_k, fn);
  LRKV_CHECK_PTR(coeff_v, fn);
  if (n_tokens == 0) return LRKV_OK;
  if (dtype == LRKV_BF16 && n_tokens <= kSmallT) {
    CompressKvArgs a{xk, xv, basis_k, basis_v, coeff_k, coeff_v, dims->batch, dims->n_kv_heads, dims->head_dim,
                     dims->rank_k, dims->rank_v, n_tokens, pos, dims->capacity};
    const hipError_t e = launch_compress_kv_small_bf16(a, stream);
    return e == hipSuccess ? LRKV_OK : device_fail(fn, e);
  }
  CompressArgs ak{xk, basis_k, coeff_k, 0, dims->batch, dims->n_kv_heads, dims->head_dim, dims->rank_k,
                  n_tokens, pos, dims->capacity};
  CompressArgs av{xv, basis_v, coeff_v, 1, dims->batch, dims->n_kv_heads, dims->head_dim, dims->rank_v,
                  n_tokens, pos, dims->capacity};
  if (dtype == LRKV_BF16) {   // both caches in one launch
    const hipError_t e = launch_compress_pair_bf16(ak, av, stream);
    return e == hipSuccess ? LRKV_OK : device_fail(fn, e);
  }
  hipError_t e = launch_compress_f32(ak, stream);
  if (e != hipSuccess) return device_fail(fn, e);
  e = launch_compress_f32(av, stream);
  return e == hipSuccess ? LRKV_OK : device_fail(fn, e);
}

size_t lrkv_decode_workspace_bytes(const lrkv_dims* dims, int64_t n_ctx, int64_t side_cap) {
  if (check_dims(dims, LRKV_F32, "lrkv_decode_workspace_bytes") != LRKV_OK &&
      check_dims(dims, LRKV_BF16, "lrkv_decode_workspace_bytes") != LRKV_OK)
    return 0;
  if (side_cap < 0) return 0;
  const int64_t n = side_cap > 0 ? dims->capacity : n_ctx;
  if (n < 1) return 0;
  return decode_layout(*dims, n, side_cap).total;
}

}  // extern "C"

namespace {

lrkv_status check_decode_common(const lrkv_dims* dims, int64_t n_ctx, lrkv_dtype dtype, void* workspace,
                                size_t workspace_bytes, const char* fn, DecodeLayout* L) {
  lrkv_status st = check_dims(dims, dtype, fn);
  if (st != LRKV_OK) return st;
  if (n_ctx < 1 || n_ctx > dims->capacity)
    return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: n_ctx = %lld outside [1, capacity = %lld]", fn, (long long)n_ctx,
                (long long)dims->capacity);
  LRKV_CHECK_PTR(workspace, fn);
  *L = decode_layout(*dims, n_ctx, 0);
  if (workspace_bytes < L->total)
    return fail(LRKV_ERR_WORKSPACE_TOO_SMALL, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, L->total);
  return LRKV_OK;
}

// seq_lens: per-sequence lengths on the device (the plan L was made for an
// upper bound n_ctx of them), or null: n_ctx is the length of every sequence
lrkv_status decode_partial(const void* q, const void* basis_k, const void* coeff_k, const void* basis_v,
                           const void* coeff_v, const lrkv_dims* dims, int64_t n_ctx, float scale,
                           lrkv_dtype dtype, void* workspace, const DecodeLayout& L, hipStream_t stream,
                           const char* fn, const void* k_new = nullptr, const void* v_new = nullptr,
                           const void* enc_k = nullptr, void* out = nullptr, float* lse = nullptr,
                           const int32_t* seq_lens = nullptr, bool merge_here = false, void* m_out = nullptr,
                           float* m_lse = nullptr) {
  char* ws = static_cast<char*>(workspace);
  SplitArgs sa{};
  sa.q = q; sa.basis_k = basis_k; sa.ck = coeff_k; sa.cv = coeff_v; sa.basis_v = basis_v;
  sa.cap = dims->capacity; sa.rk = dims->rank_k; sa.rv = dims->rank_v; sa.d = dims->head_dim;
  sa.g = dims->n_q_heads / dims->n_kv_heads; sa.hq = dims->n_q_heads; sa.hkv = dims->n_kv_heads;
  sa.batch = dims->batch;
  sa.n_static = n_ctx; sa.n_dev = nullptr;
  sa.chunks_per_split = L.lr.chunks_per_split; sa.n_splits = L.lr.n_splits; sa.n_parts = L.parts;
  sa.qscale = resolve_scale(scale, dims->head_dim) * kLog2eHost;
  sa.part_o = reinterpret_cast<float*>(ws + L.o);
  sa.part_ml = reinterpret_cast<float*>(ws + L.ml);
  if (k_new) {   // decode step: rows [0, n_ctx - 1) attended, row n_ctx - 1 appended by the last workgroup
    sa.n_static = n_ctx - 1;
    sa.k_new = k_new;
    sa.v_new = v_new;
    sa.enc_k = enc_k;
    sa.append_row = n_ctx - 1;
  }
  sa.out = out;   // final outputs (one attention workgroup per unit), or partials
  sa.lse = lse;
  sa.n_ctx_b = seq_lens;
  if (merge_here) {   // the launch merges its own partials (see merge_in_step)
    sa.merge_cnt = reinterpret_cast<uint32_t*>(ws + L.cnt);
    sa.merge_out = m_out;
    sa.merge_lse = m_lse;
  }
  // no basis_k: latent queries (absorbed projections), no fold and no lift
  const hipError_t e = dtype != LRKV_BF16 ? launch_split_f32(sa, stream)
                                          : (basis_k ? launch_split_bf16(sa, stream) : launch_split_bf16_latent(sa, stream));
  return e == hipSuccess ? LRKV_OK : device_fail(fn, e);
}

// width: elements per output row (head_dim, or rank_v for latent outputs)
lrkv_status decode_merge(void* out, float* lse, const lrkv_dims* dims, lrkv_dtype dtype, void* workspace,
                         const DecodeLayout& L, hipStream_t stream, const char* fn, int width = 0) {
  char* ws = static_cast<char*>(workspace);
  MergeArgs ma{};
  ma.part_o = reinterpret_cast<const float*>(ws + L.o);
  ma.part_ml = reinterpret_cast<const float*>(ws + L.ml);
  ma.n_parts = L.parts;
  ma.d = width > 0 ? width : dims->head_dim; ma.g = dims->n_q_heads / dims->n_kv_heads; ma.hq = dims->n_q_heads;
  ma.hkv = dims->n_kv_heads; ma.batch = dims->batch;
  ma.out = out; ma.lse = lse;
  const hipError_t e = launch_merge(ma, dtype == LRKV_BF16, stream);
  return e == hipSuccess ? LRKV_OK : device_fail(fn, e);
}

// Whether a bfloat16 attention launch (with B_K, no separate key encoder)
// merges its partials itself: when it has at most a quarter as many
// workgroups as the chip has compute units (batch-1 decodes of short and
// medium contexts, where the second launch is a large part of a layer's
// time).  Its last workgroup of each unit then merges, and there is no
// merge launch.  Measured on the batch-1 32-layer step (graph replays,
// alternating runs on one box): 40 workgroups (2048 tokens) 487.5 against
// 491.5 us per step (eager 485 against 501), but 136 workgroups (8192
// tokens) 521.4 against 507.7 us, and the batched 32K step (512
// workgroups) 191.4-191.8 against 189.4-189.5 us per layer.  (Those
// workgroup counts are from an earlier split plan: with the plan above, a
// batch-1 step over 8 kv heads merges in its launch from 17 to 28 chunks
// (up to 896 tokens; at most 16 chunks take one workgroup per unit, which
// writes the outputs), and at 2048 tokens takes 136 workgroups and a merge
// launch.)
bool merge_in_step(const lrkv_dims& d, const DecodeLayout& L, lrkv_dtype dt, const void* enc_k, bool append) {
  if (dt != LRKV_BF16 || enc_k) return false;
  const int64_t wgs = (int64_t)d.batch * d.n_kv_heads * (append ? L.parts - 1 : L.parts);
  return 4 * wgs <= device_cu_count();
}

}  // namespace

extern "C" {

lrkv_status lrkv_decode_attn(const void* q, const void* basis_k, const void* coeff_k,
                             const void* basis_v, const void* coeff_v, void* out, float* lse,
                             const lrkv_dims* dims, int64_t n_ctx, float scale, lrkv_dtype dtype,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "lrkv_decode_attn";
  DecodeLayout L;
  lrkv_status st = check_decode_common(dims, n_ctx, dtype, workspace, workspace_bytes, fn, &L);
  if (st != LRKV_OK) return st;
  if (!std::isfinite(scale)) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: scale is not finite", fn);
  LRKV_CHECK_PTR(q, fn);
  LRKV_CHECK_PTR(basis_k, fn);
  LRKV_CHECK_PTR(coeff_k, fn);
  LRKV_CHECK_PTR(basis_v, fn);
  LRKV_CHECK_PTR(coeff_v, fn);
  LRKV_CHECK_PTR(out, fn);
  if (lse && !aligned16(lse)) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: lse is not 16-byte aligned", fn);
  if (dtype == LRKV_BF16 && L.parts == 1)   // one workgroup per unit: it writes the outputs, no merge launch
    return decode_partial(q, basis_k, coeff_k, basis_v, coeff_v, dims, n_ctx, scale, dtype, workspace, L, stream,
                          fn, nullptr, nullptr, nullptr, out, lse);
  if (merge_in_step(*dims, L, dtype, nullptr, false))
    return decode_partial(q, basis_k, coeff_k, basis_v, coeff_v, dims, n_ctx, scale, dtype, workspace, L, stream,
                          fn, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, true, out, lse);
  st = decode_partial(q, basis_k, coeff_k, basis_v, coeff_v, dims, n_ctx, scale, dtype, workspace, L, stream, fn);
  if (st != LRKV_OK) return st;
  return decode_merge(out, lse, dims, dtype, workspace, L, stream, fn);
}

lrkv_status lrkv_decode_attn_partial(const void* q, const void* basis_k, const void* coeff_k,
                                     const void* basis_v, const void* coeff_v, const lrkv_dims* dims,
                                     int64_t n_ctx, float scale, lrkv_dtype dtype, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "lrkv_decode_attn_partial";
  DecodeLayout L;
  lrkv_status st = check_decode_common(dims, n_ctx, dtype, workspace, workspace_bytes, fn, &L);
  if (st != LRKV_OK) return st;
  if (!std::isfinite(scale)) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: scale is not finite", fn);
  LRKV_CHECK_PTR(q, fn);
  LRKV_CHECK_PTR(basis_k, fn);
  LRKV_CHECK_PTR(coeff_k, fn);
  LRKV_CHECK_PTR(basis_v, fn);
  LRKV_CHECK_PTR(coeff_v, fn);
  return decode_partial(q, basis_k, coeff_k, basis_v, coeff_v, dims, n_ctx, scale, dtype, workspace, L, stream, fn);
}

lrkv_status lrkv_decode_attn_merge(void* out, float* lse, const lrkv_dims* dims, int64_t n_ctx,
                                   lrkv_dtype dtype, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  const char* fn = "lrkv_decode_attn_merge";
  DecodeLayout L;
  lrkv_status st = check_decode_common(dims, n_ctx, dtype, workspace, workspace_bytes, fn, &L);
  if (st != LRKV_OK) return st;
  LRKV_CHECK_PTR(out, fn);
  if (lse && !aligned16(lse)) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: lse is not 16-byte aligned", fn);
  return decode_merge(out, lse, dims, dtype, workspace, L, stream, fn);
}

lrkv_status lrkv_decode_attn_latent(const void* q_lat, const void* coeff_k, const void* coeff_v, void* out_lat,
                                    float* lse, const lrkv_dims* dims, int64_t n_ctx, float scale, lrkv_dtype dtype,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "lrkv_decode_attn_latent";
  DecodeLayout L;
  lrkv_status st = check_decode_common(dims, n_ctx, dtype, workspace, workspace_bytes, fn, &L);
  if (st != LRKV_OK) return st;
  if (!std::isfinite(scale)) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: scale is not finite", fn);
  LRKV_CHECK_PTR(q_lat, fn);
  LRKV_CHECK_PTR(coeff_k, fn);
  LRKV_CHECK_PTR(coeff_v, fn);
  LRKV_CHECK_PTR(out_lat, fn);
  if (lse && !aligned16(lse)) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: lse is not 16-byte aligned", fn);
  // the plain decode's workspace holds these partials: rank_v <= head_dim floats each
  st = decode_partial(q_lat, nullptr, coeff_k, nullptr, coeff_v, dims, n_ctx, scale, dtype, workspace, L, stream, fn);
  if (st != LRKV_OK) return st;
  return decode_merge(out_lat, lse, dims, dtype, workspace, L, stream, fn, dims->rank_v);
}

size_t lrkv_decode_step_workspace_bytes(const lrkv_dims* dims, int64_t n_ctx) {
  if (check_dims(dims, LRKV_F32, "lrkv_decode_step_workspace_bytes") != LRKV_OK &&
      check_dims(dims, LRKV_BF16, "lrkv_decode_step_workspace_bytes") != LRKV_OK)
    return 0;
  if (n_ctx < 1) return 0;
  const size_t step = decode_layout(*dims, std::max<int64_t>(n_ctx - 1, 1), 0, true).total;
  return std::max(step, decode_layout(*dims, n_ctx, 0).total);   // float32 runs compress + decode
}

}  // extern "C"

namespace {

lrkv_status check_step(const void* q, const void* k_new, const void* v_new, const void* basis_k,
                       const void* coeff_k, const void* basis_v, const void* coeff_v, const void* enc_k,
                       const lrkv_dims* dims, int64_t n_ctx, float scale, lrkv_dtype dtype, void* workspace,
                       size_t workspace_bytes, const char* fn) {
  lrkv_status st = check_dims(dims, dtype, fn);
  if (st != LRKV_OK) return st;
  if (n_ctx < 1 || n_ctx > dims->capacity)
    return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: n_ctx = %lld outside [1, capacity = %lld]", fn, (long long)n_ctx,
                (long long)dims->capacity);
  if (!std::isfinite(scale)) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: scale is not finite", fn);
  LRKV_CHECK_PTR(q, fn);
  LRKV_CHECK_PTR(k_new, fn);
  LRKV_CHECK_PTR(v_new, fn);
  LRKV_CHECK_PTR(basis_k, fn);
  LRKV_CHECK_PTR(coeff_k, fn);
  LRKV_CHECK_PTR(basis_v, fn);
  LRKV_CHECK_PTR(coeff_v, fn);
  LRKV_CHECK_PTR(workspace, fn);
  if (enc_k && !aligned16(enc_k)) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: enc_k is not 16-byte aligned", fn);
  const size_t need = lrkv_decode_step_workspace_bytes(dims, n_ctx);
  if (workspace_bytes < need)
    return fail(LRKV_ERR_WORKSPACE_TOO_SMALL, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
  return LRKV_OK;
}

// Workspace layout of a decode step: the attention workgroups of rows
// [0, n_ctx - 1) plus the appended token's (empty) slot (bfloat16); float32 runs
// the plain decode over n_ctx rows after the compress kernel.
DecodeLayout step_layout(const lrkv_dims& d, int64_t n_ctx, lrkv_dtype dtype) {
  return dtype == LRKV_BF16 ? decode_layout(d, std::max<int64_t>(n_ctx - 1, 1), 0, true) : decode_layout(d, n_ctx, 0);
}

lrkv_status step_partial(const void* q, const void* k_new, const void* v_new, const void* basis_k, void* coeff_k,
                         const void* basis_v, void* coeff_v, const void* enc_k, const lrkv_dims* dims, int64_t n_ctx, float scale, lrkv_dtype dtype, void* workspace,
                         const DecodeLayout& L, hipStream_t stream, const char* fn) {
  if (dtype != LRKV_BF16) {
    const lrkv_status st = lrkv_compress_kv(k_new, v_new, enc_k ? enc_k : basis_k, basis_v, coeff_k, coeff_v, dims,
                                            1, n_ctx - 1, dtype, stream);
    if (st != LRKV_OK) return st;
    return decode_partial(q, basis_k, coeff_k, basis_v, coeff_v, dims, n_ctx, scale, dtype, workspace, L, stream, fn);
  }
  return decode_partial(q, basis_k, coeff_k, basis_v, coeff_v, dims, n_ctx, scale, dtype, workspace, L, stream, fn,
                        k_new, v_new, enc_k);
}

}  // namespace

extern "C" {

lrkv_status lrkv_decode_step(const void* q, const void* k_new, const void* v_new, const void* basis_k,
                             void* coeff_k, const void* basis_v, void* coeff_v, const void* enc_k, void* out, float* lse, const lrkv_dims* dims, int64_t n_ctx, float scale,
                             lrkv_dtype dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "lrkv_decode_step";
  lrkv_status st = check_step(q, k_new, v_new, basis_k, coeff_k, basis_v, coeff_v, enc_k, dims, n_ctx, scale, dtype,
                              workspace, workspace_bytes, fn);
  if (st != LRKV_OK) return st;
  LRKV_CHECK_PTR(out, fn);
  if (lse && !aligned16(lse)) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: lse is not 16-byte aligned", fn);
  if (dtype == LRKV_BF16) {
    // one attention workgroup per unit: it also appends the token (after its
    // fold) and writes the outputs itself; no merge launch
    DecodeLayout F = decode_layout(*dims, std::max<int64_t>(n_ctx - 1, 1), 0);
    if (F.parts == 1) {
      F.parts = 2;   // the workgroup's slot and the token's (neither is written)
      return decode_partial(q, basis_k, coeff_k, basis_v, coeff_v, dims, n_ctx, scale, dtype, workspace, F, stream,
                            fn, k_new, v_new, enc_k, out, lse);
    }
  }
  const DecodeLayout L = step_layout(*dims, n_ctx, dtype);
  if (merge_in_step(*dims, L, dtype, enc_k, true))
    return decode_partial(q, basis_k, coeff_k, basis_v, coeff_v, dims, n_ctx, scale, dtype, workspace, L, stream,
                          fn, k_new, v_new, nullptr, nullptr, nullptr, nullptr, true, out, lse);
  st = step_partial(q, k_new, v_new, basis_k, coeff_k, basis_v, coeff_v, enc_k, dims, n_ctx, scale, dtype, workspace,
                    L, stream, fn);
  if (st != LRKV_OK) return st;
  return decode_merge(out, lse, dims, dtype, workspace, L, stream, fn);
}

lrkv_status lrkv_decode_step_partial(const void* q, const void* k_new, const void* v_new, const void* basis_k,
                                     void* coeff_k, const void* basis_v, void* coeff_v, const void* enc_k,
                                     const lrkv_dims* dims, int64_t n_ctx, float scale, lrkv_dtype dtype,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "lrkv_decode_step_partial";
  const lrkv_status st = check_step(q, k_new, v_new, basis_k, coeff_k, basis_v, coeff_v, enc_k, dims, n_ctx, scale,
                                    dtype, workspace, workspace_bytes, fn);
  if (st != LRKV_OK) return st;
  return step_partial(q, k_new, v_new, basis_k, coeff_k, basis_v, coeff_v, enc_k, dims, n_ctx, scale, dtype,
                      workspace, step_layout(*dims, n_ctx, dtype), stream, fn);
}

lrkv_status lrkv_decode_step_merge(void* out, float* lse, const lrkv_dims* dims, int64_t n_ctx, lrkv_dtype dtype,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "lrkv_decode_step_merge";
  lrkv_status st = check_dims(dims, dtype, fn);
  if (st != LRKV_OK) return st;
  if (n_ctx < 1 || n_ctx > dims->capacity)
    return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: n_ctx = %lld outside [1, capacity = %lld]", fn, (long long)n_ctx,
                (long long)dims->capacity);
  LRKV_CHECK_PTR(out, fn);
  LRKV_CHECK_PTR(workspace, fn);
  if (lse && !aligned16(lse)) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: lse is not 16-byte aligned", fn);
  const size_t need = lrkv_decode_step_workspace_bytes(dims, n_ctx);
  if (workspace_bytes < need)
    return fail(LRKV_ERR_WORKSPACE_TOO_SMALL, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
  return decode_merge(out, lse, dims, dtype, workspace, step_layout(*dims, n_ctx, dtype), stream, fn);
}

lrkv_status lrkv_decode_attn_seqlens(const void* q, const void* basis_k, const void* coeff_k,
                                     const void* basis_v, const void* coeff_v, void* out, float* lse,
                                     const lrkv_dims* dims, const int32_t* seq_lens, int64_t max_seq_len,
                                     float scale, lrkv_dtype dtype, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  const char* fn = "lrkv_decode_attn_seqlens";
  DecodeLayout L;
  lrkv_status st = check_decode_common(dims, max_seq_len, dtype, workspace, workspace_bytes, fn, &L);
  if (st != LRKV_OK) return st;
  if (dtype != LRKV_BF16) return fail(LRKV_ERR_UNSUPPORTED, "%s: only bfloat16 caches are supported", fn);
  if (!std::isfinite(scale)) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: scale is not finite", fn);
  if (!seq_lens || (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: seq_lens is NULL or not 4-byte aligned", fn);
  LRKV_CHECK_PTR(q, fn);
  LRKV_CHECK_PTR(basis_k, fn);
  LRKV_CHECK_PTR(coeff_k, fn);
  LRKV_CHECK_PTR(basis_v, fn);
  LRKV_CHECK_PTR(coeff_v, fn);
  LRKV_CHECK_PTR(out, fn);
  if (lse && !aligned16(lse)) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: lse is not 16-byte aligned", fn);
  if (L.parts == 1)
    return decode_partial(q, basis_k, coeff_k, basis_v, coeff_v, dims, max_seq_len, scale, dtype, workspace, L,
                          stream, fn, nullptr, nullptr, nullptr, out, lse, seq_lens);
  const bool here = merge_in_step(*dims, L, dtype, nullptr, false);
  st = decode_partial(q, basis_k, coeff_k, basis_v, coeff_v, dims, max_seq_len, scale, dtype, workspace, L, stream,
                      fn, nullptr, nullptr, nullptr, nullptr, nullptr, seq_lens, here, out, lse);
  if (st != LRKV_OK || here) return st;
  return decode_merge(out, lse, dims, dtype, workspace, L, stream, fn);
}

lrkv_status lrkv_decode_step_seqlens(const void* q, const void* k_new, const void* v_new, const void* basis_k,
                                     void* coeff_k, const void* basis_v, void* coeff_v, const void* enc_k, void* out,
                                     float* lse, const lrkv_dims* dims, const int32_t* seq_lens, int64_t max_seq_len,
                                     float scale, lrkv_dtype dtype, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  const char* fn = "lrkv_decode_step_seqlens";
  lrkv_status st = check_step(q, k_new, v_new, basis_k, coeff_k, basis_v, coeff_v, enc_k, dims, max_seq_len, scale,
                              dtype, workspace, workspace_bytes, fn);
  if (st != LRKV_OK) return st;
  if (dtype != LRKV_BF16) return fail(LRKV_ERR_UNSUPPORTED, "%s: only bfloat16 caches are supported", fn);
  if (!seq_lens || (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: seq_lens is NULL or not 4-byte aligned", fn);
  LRKV_CHECK_PTR(out, fn);
  if (lse && !aligned16(lse)) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: lse is not 16-byte aligned", fn);
  DecodeLayout F = decode_layout(*dims, std::max<int64_t>(max_seq_len - 1, 1), 0);
  if (F.parts == 1) {   // one workgroup per unit attends, appends and writes the outputs
    F.parts = 2;
    return decode_partial(q, basis_k, coeff_k, basis_v, coeff_v, dims, max_seq_len, scale, dtype, workspace, F,
                          stream, fn, k_new, v_new, enc_k, out, lse, seq_lens);
  }
  const DecodeLayout L = step_layout(*dims, max_seq_len, dtype);
  const bool here = merge_in_step(*dims, L, dtype, enc_k, true);
  st = decode_partial(q, basis_k, coeff_k, basis_v, coeff_v, dims, max_seq_len, scale, dtype, workspace, L, stream,
                      fn, k_new, v_new, enc_k, nullptr, nullptr, seq_lens, here, out, lse);
  if (st != LRKV_OK || here) return st;
  return decode_merge(out, lse, dims, dtype, workspace, L, stream, fn);
}

size_t lrkv_compress_hybrid_workspace_bytes(const lrkv_dims* dims, int64_t n_tokens) {
  if (!dims || n_tokens < 0 || dims->batch < 1 || dims->n_kv_heads < 1) return 0;
  const int64_t tiles = cdiv(n_tokens, kHybridTile);
  const int64_t units = (int64_t)dims->batch * dims->n_kv_heads;
  size_t off = align256((size_t)(units * tiles * kHybridTile));       // flags
  off = align256(off + sizeof(int32_t) * units * tiles);              // counts
  off = align256(off + sizeof(int32_t) * units * tiles * 2);          // offsets
  return off;
}

lrkv_status lrkv_compress_hybrid(const void* k, const void* v, const void* basis_k,
                                 const void* basis_v, float tau, void* coeff_k, void* coeff_v,
                                 int32_t* n_lr, void* k_side, void* v_side, int32_t* side_idx,
                                 int32_t* n_side, uint8_t* flags, int32_t* overflow,
                                 const lrkv_dims* dims, int64_t n_tokens, int64_t pos,
                                 int64_t side_cap, lrkv_dtype dtype, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "lrkv_compress_hybrid";
  lrkv_status st = check_dims(dims, dtype, fn);
  if (st != LRKV_OK) return st;
  if (dtype != LRKV_BF16) return fail(LRKV_ERR_UNSUPPORTED, "%s: only bfloat16 caches are supported", fn);
  if (std::isnan(tau) || tau < 0.f) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: tau must be >= 0", fn);
  if (n_tokens < 0 || pos < 0 || pos + n_tokens > ((int64_t)1 << 31))
    return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: bad n_tokens / pos", fn);
  if (side_cap < 8 || side_cap % 8 || side_cap * dims->head_dim * 4 >= ((int64_t)1 << 31))
    return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: side_cap = %lld must be a positive multiple of 8 below 2^31 bytes",
                fn, (long long)side_cap);
  LRKV_CHECK_PTR(k, fn);
  LRKV_CHECK_PTR(v, fn);
  LRKV_CHECK_PTR(basis_k, fn);
  LRKV_CHECK_PTR(basis_v, fn);
  LRKV_CHECK_PTR(coeff_k, fn);
  LRKV_CHECK_PTR(coeff_v, fn);
  LRKV_CHECK_PTR(k_side, fn);
  LRKV_CHECK_PTR(v_side, fn);
  LRKV_CHECK_PTR(workspace, fn);
  if (!n_lr || !n_side || !side_idx || !overflow)
    return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: n_lr, n_side, side_idx and overflow must not be NULL", fn);
  if (n_tokens == 0) return LRKV_OK;
  const size_t need = lrkv_compress_hybrid_workspace_bytes(dims, n_tokens);
  if (workspace_bytes < need)
    return fail(LRKV_ERR_WORKSPACE_TOO_SMALL, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
  const int64_t tiles = cdiv(n_tokens, kHybridTile);
  if (tiles > 0x7fffffff) return fail(LRKV_ERR_UNSUPPORTED, "%s: too many tokens", fn);
  const int64_t units = (int64_t)dims->batch * dims->n_kv_heads;
  char* ws = static_cast<char*>(workspace);
  HybridArgs a{};
  a.k = k; a.v = v; a.bk = basis_k; a.bv = basis_v;
  a.tau2 = std::isinf(tau) ? INFINITY : tau * tau;
  a.ck = coeff_k; a.cv = coeff_v; a.n_lr = n_lr;
  a.k_side = k_side; a.v_side = v_side; a.side_idx = side_idx; a.n_side = n_side;
  a.flags = flags; a.overflow = overflow;
  a.batch = dims->batch; a.hkv = dims->n_kv_heads; a.d = dims->head_dim;
  a.rk = dims->rank_k; a.rv = dims->rank_v;
  a.n_tokens = n_tokens; a.pos = pos; a.cap = dims->capacity; a.side_cap = side_cap;
  size_t off = 0;
  a.ws_flags = reinterpret_cast<uint8_t*>(ws + off); off = align256(off + (size_t)(units * tiles * kHybridTile));
  a.ws_counts = reinterpret_cast<int32_t*>(ws + off); off = align256(off + sizeof(int32_t) * units * tiles);
  a.ws_offsets = reinterpret_cast<int32_t*>(ws + off);
  a.n_tiles = (int)tiles;
  a.cus = device_cu_count();
  const hipError_t e = launch_hybrid_bf16(a, stream);
  return e == hipSuccess ? LRKV_OK : device_fail(fn, e);
}

lrkv_status lrkv_decode_attn_hybrid(const void* q, const void* basis_k, const void* coeff_k,
                                    const void* basis_v, const void* coeff_v,
                                    const int32_t* n_lr, const void* k_side, const void* v_side,
                                    const int32_t* n_side, int64_t side_cap, void* out,
                                    float* lse, const lrkv_dims* dims, float scale,
                                    lrkv_dtype dtype, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  const char* fn = "lrkv_decode_attn_hybrid";
  lrkv_status st = check_dims(dims, dtype, fn);
  if (st != LRKV_OK) return st;
  if (side_cap < 8 || side_cap % 8 || side_cap * dims->head_dim * 4 >= ((int64_t)1 << 31))
    return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: side_cap = %lld must be a positive multiple of 8 below 2^31 bytes",
                fn, (long long)side_cap);
  if (!std::isfinite(scale)) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: scale is not finite", fn);
  LRKV_CHECK_PTR(q, fn);
  LRKV_CHECK_PTR(basis_k, fn);
  LRKV_CHECK_PTR(coeff_k, fn);
  LRKV_CHECK_PTR(basis_v, fn);
  LRKV_CHECK_PTR(coeff_v, fn);
  LRKV_CHECK_PTR(k_side, fn);
  LRKV_CHECK_PTR(v_side, fn);
  LRKV_CHECK_PTR(out, fn);
  LRKV_CHECK_PTR(workspace, fn);
  if (!n_lr || !n_side) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: n_lr and n_side must not be NULL", fn);
  if (lse && !aligned16(lse)) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: lse is not 16-byte aligned", fn);
  if (dtype != LRKV_BF16) return fail(LRKV_ERR_UNSUPPORTED, "%s: only bfloat16 caches are supported", fn);
  const DecodeLayout L = decode_layout(*dims, dims->capacity, side_cap);
  if (workspace_bytes < L.total)
    return fail(LRKV_ERR_WORKSPACE_TOO_SMALL, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, L.total);
  char* ws = static_cast<char*>(workspace);
  const int g = dims->n_q_heads / dims->n_kv_heads;

  SplitArgs sa{};
  sa.q = q; sa.basis_k = basis_k; sa.ck = coeff_k; sa.cv = coeff_v; sa.basis_v = basis_v;
  sa.cap = dims->capacity; sa.rk = dims->rank_k; sa.rv = dims->rank_v; sa.d = dims->head_dim;
  sa.g = g; sa.hq = dims->n_q_heads; sa.hkv = dims->n_kv_heads; sa.batch = dims->batch;
  sa.n_static = 0; sa.n_dev = n_lr;
  sa.n_parts = L.parts;   // chunks per split are planned on the device
  sa.qscale = resolve_scale(scale, dims->head_dim) * kLog2eHost;
  sa.part_o = reinterpret_cast<float*>(ws + L.o);
  sa.part_ml = reinterpret_cast<float*>(ws + L.ml);
  SplitArgs ss = sa;   // side list: full-rank rows, no fold and no lift
  ss.basis_k = nullptr; ss.basis_v = nullptr; ss.ck = k_side; ss.cv = v_side; ss.cap = side_cap;
  ss.rk = dims->head_dim; ss.rv = dims->head_dim; ss.n_dev = n_side;
  // the merge runs in the same launch (the last workgroup of each unit):
  // 52.2 against 53.1 us per call with a merge launch at 131072 tokens
  sa.merge_cnt = reinterpret_cast<uint32_t*>(ws + L.cnt);
  sa.merge_out = out;
  sa.merge_lse = lse;
  const hipError_t e = launch_split_bf16_hybrid(sa, ss, L.parts, stream);
  return e == hipSuccess ? LRKV_OK : device_fail(fn, e);
}

size_t lrkv_oja_workspace_bytes(int32_t batch, int32_t n_kv_heads, int32_t head_dim, int32_t rank,
                                int64_t n_tokens) {
  if (batch < 1 || n_kv_heads < 1 || head_dim < 16 || rank < 1 || n_tokens < 0) return 0;
  const int n_wg = oja_workgroups(n_kv_heads, (int64_t)batch * n_tokens);
  return sizeof(float) * oja_workspace_floats(n_kv_heads, head_dim, rank, n_wg);
}

lrkv_status lrkv_oja_update(const void* x, float* basis, void* basis_bf16, int32_t batch,
                            int32_t n_kv_heads, int32_t head_dim, int32_t rank, int64_t n_tokens,
                            float eta, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "lrkv_oja_update";
  if (batch < 1 || n_kv_heads < 1) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: batch and n_kv_heads must be >= 1", fn);
  if (n_kv_heads > 65535) return fail(LRKV_ERR_UNSUPPORTED, "%s: n_kv_heads must be <= 65535", fn);
  if (head_dim != 64 && head_dim != 128)
    return fail(LRKV_ERR_UNSUPPORTED, "%s: head_dim = %d (supported: 64, 128)", fn, head_dim);
  lrkv_status st = check_rank(rank, head_dim, LRKV_BF16, fn, "rank");
  if (st != LRKV_OK) return st;
  if (n_tokens < 0) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: n_tokens = %lld < 0", fn, (long long)n_tokens);
  if (!std::isfinite(eta)) return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: eta is not finite", fn);
  LRKV_CHECK_PTR(basis, fn);
  if (basis_bf16 && !aligned16(basis_bf16))
    return fail(LRKV_ERR_INVALID_ARGUMENT, "%s: basis_bf16 is not 16-byte aligned", fn);
  if (n_tokens == 0) return LRKV_OK;   // x may be NULL then
  LRKV_CHECK_PTR(x, fn);
  const int64_t tokens = (int64_t)batch * n_tokens;
  if (tokens * n_kv_heads * head_dim > ((int64_t)1 << 40))
    return fail(LRKV_ERR_UNSUPPORTED, "%s: chunk of %lld tokens is too large", fn, (long long)tokens);
  LRKV_CHECK_PTR(workspace, fn);
  const size_t need = lrkv_oja_workspace_bytes(batch, n_kv_heads, head_dim, rank, n_tokens);
  if (workspace_bytes < need)
    return fail(LRKV_ERR_WORKSPACE_TOO_SMALL, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
  OjaArgs a{};
  a.x = x; a.basis = basis; a.basis_bf16 = basis_bf16;
  a.hkv = n_kv_heads; a.d = head_dim; a.rank = rank; a.n_tokens = tokens; a.eta = eta;
  a.n_wg = oja_workgroups(n_kv_heads, tokens);
  a.ws = static_cast<float*>(workspace);
  a.ws_sum = a.ws + oja_partial_floats(n_kv_heads, head_dim, a.n_wg);
  const hipError_t e = launch_oja_update(a, stream);
  return e == hipSuccess ? LRKV_OK : device_fail(fn, e);
}

}  // extern "C"
