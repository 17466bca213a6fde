// Host-only build of the library's C-ABI layer (lrkv_host.cpp) under
// AddressSanitizer and UndefinedBehaviorSanitizer.
//
// The kernel launchers are replaced by stubs that run on the host: each one
// touches every byte the real launch would write (and reads every byte its
// second phase would read) in the caller's workspace and outputs, and checks
// that the split plan it was given covers every chunk of the context.  The
// driver allocates each workspace and output with exactly the size the
// library asks for, so a layout or planning mistake in the host code shows up
// as a heap overflow or a failed check.  The HIP runtime calls of the host
// code are stubbed too (a device with a chosen compute-unit count).
//
// Exit status 0 when every call returned what it should; sanitizer reports
// abort the run.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "lrkv.h"
#include "lrkv_internal.h"

// ---------------------------------------------------------------- HIP stubs
static int g_cus = 256;

extern "C" {
hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int) {
  *v = attr == hipDeviceAttributeMultiprocessorCount ? g_cus : 0;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stub error"; }
}

// ---------------------------------------------------------------- touching
static volatile unsigned char g_sink;
static int g_failures = 0;

#define EXPECT(cond, ...)                        \
  do {                                           \
    if (!(cond)) {                               \
      std::fprintf(stderr, "FAILED %s:%d: ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);         \
      std::fprintf(stderr, "\n");                \
      ++g_failures;                              \
    }                                            \
  } while (0)

template <typename T>
static void touch_write(T* p, int64_t n) {
  if (n > 0) std::memset(static_cast<void*>(p), 0x5a, sizeof(T) * (size_t)n);
}
template <typename T>
static void touch_read(const T* p, int64_t n) {
  const unsigned char* c = reinterpret_cast<const unsigned char*>(p);
  unsigned char x = 0;
  for (int64_t i = 0; i < (int64_t)sizeof(T) * n; ++i) x ^= c[i];
  g_sink = x;
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

namespace lrkv {

// Partials of a split launch: every (batch, q head) row has n_parts slots of
// `width` floats and (max, sum); with final outputs, out [B, Hq, d] and lse.
static void split_writes(const SplitArgs& a, int grid_x, int width) {
  const int64_t rows = (int64_t)a.batch * a.hq;
  EXPECT(grid_x >= 1, "empty grid");
  if (a.out) {
    touch_write(static_cast<uint16_t*>(a.out), rows * a.d);
    if (a.lse) touch_write(a.lse, rows);
    return;
  }
  touch_write(a.part_o, rows * a.n_parts * width);
  touch_write(a.part_ml, rows * a.n_parts * 2);
}

static void check_cover(const SplitArgs& a, int attn_wgs) {
  if (a.n_ctx_b) {   // device lengths: the planned splits fit the attention workgroups
    EXPECT(a.n_splits >= 1 && cdiv(a.n_splits, 4) <= attn_wgs, "n_splits %d for %d workgroups", a.n_splits,
           attn_wgs);
    return;
  }
  const int64_t chunks = cdiv(a.n_static, kChunk);
  EXPECT(a.chunks_per_split >= 1, "chunks_per_split %d", a.chunks_per_split);
  EXPECT(cdiv(chunks, 4LL * a.chunks_per_split) <= attn_wgs, "%lld chunks not covered by %d workgroups",
         (long long)chunks, attn_wgs);
}

hipError_t launch_split_bf16(const SplitArgs& a, hipStream_t) {
  const int grid_x = a.k_new ? a.n_parts - 1 : a.n_parts;
  check_cover(a, grid_x);
  if (a.k_new) EXPECT(a.append_row == a.n_static, "append row %lld after %lld rows", (long long)a.append_row,
                      (long long)a.n_static);
  split_writes(a, grid_x, a.d);
  return hipSuccess;
}
hipError_t launch_split_bf16_latent(const SplitArgs& a, hipStream_t) {
  check_cover(a, a.n_parts);
  split_writes(a, a.n_parts, a.rv);
  return hipSuccess;
}
hipError_t launch_split_f32(const SplitArgs& a, hipStream_t) {
  const int grid_x = (int)cdiv(a.n_splits, 4);
  check_cover(a, grid_x);
  EXPECT(grid_x <= a.n_parts, "f32 grid %d > %d partials", grid_x, a.n_parts);
  split_writes(a, grid_x, a.basis_v ? a.d : a.rv);
  return hipSuccess;
}
hipError_t launch_split_bf16_hybrid(const SplitArgs& lr, const SplitArgs& side, int wgs, hipStream_t) {
  EXPECT(wgs == lr.n_parts && side.rk == lr.d && side.rv == lr.d, "hybrid launch shape");
  split_writes(lr, wgs, lr.d);
  return hipSuccess;
}
hipError_t launch_merge(const MergeArgs& a, bool bf16, hipStream_t) {
  const int64_t rows = (int64_t)a.batch * a.hq;
  touch_read(a.part_o, rows * a.n_parts * a.d);
  touch_read(a.part_ml, rows * a.n_parts * 2);
  if (bf16) touch_write(static_cast<uint16_t*>(a.out), rows * a.d);
  else touch_write(static_cast<float*>(a.out), rows * a.d);
  if (a.lse) touch_write(a.lse, rows);
  return hipSuccess;
}
hipError_t launch_compress_bf16(const CompressArgs& a, hipStream_t) {
  EXPECT(a.pos + a.n_tokens <= a.cap, "compress rows past the capacity");
  return hipSuccess;
}
hipError_t launch_compress_pair_bf16(const CompressArgs& k, const CompressArgs& v, hipStream_t) {
  EXPECT(k.n_tokens == v.n_tokens && k.values_layout == 0 && v.values_layout == 1, "pair compress");
  return hipSuccess;
}
hipError_t launch_compress_f32(const CompressArgs& a, hipStream_t) {
  EXPECT(a.pos + a.n_tokens <= a.cap, "compress rows past the capacity");
  return hipSuccess;
}
hipError_t launch_compress_kv_small_bf16(const CompressKvArgs& a, hipStream_t) {
  EXPECT(a.n_tokens <= kSmallT, "small compress of %lld tokens", (long long)a.n_tokens);
  return hipSuccess;
}
hipError_t launch_hybrid_bf16(const HybridArgs& a, hipStream_t) {
  const int64_t units = (int64_t)a.batch * a.hkv;
  touch_write(a.ws_flags, units * a.n_tiles * kHybridTile);
  touch_write(a.ws_counts, units * a.n_tiles);
  touch_write(a.ws_offsets, units * a.n_tiles * 2);
  EXPECT((int64_t)a.n_tiles * kHybridTile >= a.n_tokens, "tiles do not cover the tokens");
  return hipSuccess;
}
hipError_t launch_oja_update(const OjaArgs& a, hipStream_t) {
  EXPECT(a.n_tokens >= 1, "Oja update of no tokens launched");
  if (a.n_tokens <= kOjaSmallTokens) return hipSuccess;   // one workgroup per head, no workspace
  const int64_t per_head = oja_head_floats(a.d, oja_rank_pad(a.rank));
  const int64_t partials = (int64_t)a.hkv * a.n_wg * a.d * a.d;   // the runs' Gram matrices
  EXPECT(a.ws_sum == a.ws + partials, "Oja sums not after the partials");
  touch_write(a.ws, partials);
  touch_write(a.ws_sum, (int64_t)a.hkv * per_head);
  touch_read(a.ws, partials);
  EXPECT(a.n_wg >= 1, "no Oja workgroups");
  return hipSuccess;
}

}  // namespace lrkv

// ---------------------------------------------------------------- driver
// Device pointers the stubs never dereference (16-byte aligned, non-null).
static void* const P = reinterpret_cast<void*>(uintptr_t(1) << 20);

struct Buf {
  unsigned char* p;
  size_t n;
  explicit Buf(size_t bytes) : p(static_cast<unsigned char*>(std::malloc(bytes ? bytes : 1))), n(bytes) {}
  ~Buf() { std::free(p); }
};

static void expect_status(lrkv_status got, lrkv_status want, const char* what) {
  EXPECT(got == want, "%s: status %d, expected %d (%s)", what, (int)got, (int)want, lrkv_last_error());
}

static void decode_shapes(const lrkv_dims& d, int64_t n) {
  const int64_t rows = (int64_t)d.batch * d.n_q_heads;
  for (lrkv_dtype dt : {LRKV_BF16, LRKV_F32}) {
    const size_t elem = dt == LRKV_BF16 ? 2 : 4;
    Buf out(rows * d.head_dim * elem), lse(rows * 4);
    {
      Buf ws(lrkv_decode_workspace_bytes(&d, n, 0));
      expect_status(lrkv_decode_attn(P, P, P, P, P, out.p, reinterpret_cast<float*>(lse.p), &d, n, 0.f, dt, ws.p,
                                     ws.n, nullptr), LRKV_OK, "decode_attn");
      expect_status(lrkv_decode_attn_partial(P, P, P, P, P, &d, n, 0.f, dt, ws.p, ws.n, nullptr), LRKV_OK,
                    "decode_attn_partial");
      expect_status(lrkv_decode_attn_merge(out.p, nullptr, &d, n, dt, ws.p, ws.n, nullptr), LRKV_OK,
                    "decode_attn_merge");
      expect_status(lrkv_decode_attn(P, P, P, P, P, out.p, nullptr, &d, n, 0.f, dt, ws.p, ws.n - 1, nullptr),
                    LRKV_ERR_WORKSPACE_TOO_SMALL, "decode_attn short workspace");
      Buf lat(rows * d.rank_v * elem);
      expect_status(lrkv_decode_attn_latent(P, P, P, lat.p, reinterpret_cast<float*>(lse.p), &d, n, 0.f, dt, ws.p,
                                            ws.n, nullptr), LRKV_OK, "decode_attn_latent");
    }
    {
      Buf ws(lrkv_decode_step_workspace_bytes(&d, n));
      expect_status(lrkv_decode_step(P, P, P, P, P, P, P, nullptr, out.p, reinterpret_cast<float*>(lse.p), &d, n,
                                     0.f, dt, ws.p, ws.n, nullptr), LRKV_OK, "decode_step");
      expect_status(lrkv_decode_step(P, P, P, P, P, P, P, P, out.p, nullptr, &d, n, 0.f, dt, ws.p, ws.n, nullptr),
                    LRKV_OK, "decode_step with an encoder");
      expect_status(lrkv_decode_step_partial(P, P, P, P, P, P, P, nullptr, &d, n, 0.f, dt, ws.p, ws.n, nullptr),
                    LRKV_OK, "decode_step_partial");
      expect_status(lrkv_decode_step_merge(out.p, reinterpret_cast<float*>(lse.p), &d, n, dt, ws.p, ws.n, nullptr),
                    LRKV_OK, "decode_step_merge");
      if (dt == LRKV_BF16) {
        expect_status(lrkv_decode_step_seqlens(P, P, P, P, P, P, P, nullptr, out.p, reinterpret_cast<float*>(lse.p),
                                               &d, reinterpret_cast<const int32_t*>(P), n, 0.f, dt, ws.p, ws.n,
                                               nullptr), LRKV_OK, "decode_step_seqlens");
      }
    }
    if (dt == LRKV_BF16) {
      Buf ws(lrkv_decode_workspace_bytes(&d, n, 0));
      expect_status(lrkv_decode_attn_seqlens(P, P, P, P, P, out.p, nullptr, &d, reinterpret_cast<const int32_t*>(P), n,
                                             0.f, dt, ws.p, ws.n, nullptr), LRKV_OK, "decode_attn_seqlens");
      const int64_t side_cap = 64;
      Buf hws(lrkv_decode_workspace_bytes(&d, n, side_cap));
      expect_status(lrkv_decode_attn_hybrid(P, P, P, P, P, reinterpret_cast<const int32_t*>(P), P, P,
                                            reinterpret_cast<const int32_t*>(P), side_cap, out.p,
                                            reinterpret_cast<float*>(lse.p), &d, 0.f, dt, hws.p, hws.n, nullptr),
                    LRKV_OK, "decode_attn_hybrid");
      const int64_t T = std::min<int64_t>(n, d.capacity);
      Buf cws(lrkv_compress_hybrid_workspace_bytes(&d, T));
      expect_status(lrkv_compress_hybrid(P, P, P, P, 0.5f, P, P, reinterpret_cast<int32_t*>(P), P, P,
                                         reinterpret_cast<int32_t*>(P), reinterpret_cast<int32_t*>(P), nullptr,
                                         reinterpret_cast<int32_t*>(P), &d, T, 0, side_cap, dt, cws.p, cws.n, nullptr),
                    LRKV_OK, "compress_hybrid");
    }
    expect_status(lrkv_compress_kv(P, P, P, P, P, P, &d, std::min<int64_t>(n, 4096), 0, dt, nullptr), LRKV_OK,
                  "compress_kv");
    expect_status(lrkv_compress_kv(P, P, P, P, P, P, &d, 1, n - 1, dt, nullptr), LRKV_OK, "compress_kv one token");
  }
  for (int rank : {d.rank_k, d.rank_v}) {
    for (int64_t T : {int64_t(1), int64_t(64), int64_t(65), int64_t(333), n}) {
      Buf ws(lrkv_oja_workspace_bytes(d.batch, d.n_kv_heads, d.head_dim, rank, T));
      std::vector<float> basis((size_t)d.n_kv_heads * d.head_dim * rank);
      expect_status(lrkv_oja_update(P, basis.data(), nullptr, d.batch, d.n_kv_heads, d.head_dim, rank, T, 1e-3f, ws.p,
                                    ws.n, nullptr), LRKV_OK, "oja_update");
    }
  }
}

int main() {
  struct Shape { int B, Hq, Hkv, d, rk, rv; int64_t cap, n; };
  const Shape shapes[] = {
      {1, 4, 1, 64, 16, 16, 256, 256},        // tiny
      {1, 32, 8, 128, 64, 80, 2048, 2048},    // one Llama layer
      {1, 32, 8, 128, 56, 72, 8192, 1},       // a one-token context
      {1, 32, 8, 128, 56, 72, 8192, 257},
      {16, 32, 8, 128, 48, 112, 32768, 32768},// the batched step
      {1, 32, 8, 128, 64, 64, 131072, 131072},// long context
      {3, 24, 3, 64, 40, 24, 1000, 999},
      {64, 64, 8, 128, 128, 128, 4096, 4096},
  };
  for (int cus : {256, 80, 1}) {
    g_cus = cus;
    for (const Shape& s : shapes) {
      lrkv_dims d{s.B, s.Hq, s.Hkv, s.d, s.rk, s.rv, s.cap};
      decode_shapes(d, s.n);
    }
  }
  // invalid calls: a status, no launch
  lrkv_dims d{1, 8, 2, 128, 32, 64, 256};
  Buf ws(lrkv_decode_workspace_bytes(&d, 100, 0));
  expect_status(lrkv_decode_attn(P, P, P, P, P, P, nullptr, &d, 0, 0.f, LRKV_BF16, ws.p, ws.n, nullptr),
                LRKV_ERR_INVALID_ARGUMENT, "n_ctx 0");
  expect_status(lrkv_decode_attn(P, P, P, P, P, P, nullptr, nullptr, 10, 0.f, LRKV_BF16, ws.p, ws.n, nullptr),
                LRKV_ERR_INVALID_ARGUMENT, "null dims");
  lrkv_dims bad = d;
  bad.head_dim = 96;
  expect_status(lrkv_decode_attn(P, P, P, P, P, P, nullptr, &bad, 10, 0.f, LRKV_BF16, ws.p, ws.n, nullptr),
                LRKV_ERR_UNSUPPORTED, "head_dim 96");
  bad = d;
  bad.capacity = int64_t(1) << 40;
  expect_status(lrkv_decode_attn(P, P, P, P, P, P, nullptr, &bad, 10, 0.f, LRKV_BF16, ws.p, ws.n, nullptr),
                LRKV_ERR_UNSUPPORTED, "huge capacity");
  expect_status(lrkv_compress(P, P, P, LRKV_KEYS, 1, 2, 128, 32, 10, 250, 256, LRKV_BF16, nullptr),
                LRKV_ERR_INVALID_ARGUMENT, "compress past capacity");
  Buf sws(lrkv_decode_step_workspace_bytes(&d, 100));
  expect_status(lrkv_decode_step_seqlens(P, P, P, P, P, P, P, nullptr, P, nullptr, &d, nullptr, 100, 0.f, LRKV_BF16,
                                         sws.p, sws.n, nullptr), LRKV_ERR_INVALID_ARGUMENT, "null seq_lens");
  EXPECT(std::strlen(lrkv_status_string(LRKV_ERR_DEVICE)) > 0, "status string");
  if (g_failures) {
    std::fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  std::printf("host ABI checks passed\n");
  return 0;
}
