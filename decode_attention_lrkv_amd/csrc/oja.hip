// Online basis update by Oja's subspace rule (gfx950).
//
// For the basis B [d, r] of one kv head and the new tokens x_t of a chunk
// (every batch row): Y = X B, then B <- B + eta (X^T Y - B Y^T Y).  The basis
// is kept in float32 (steps of the size Oja's rule takes fall below bfloat16
// resolution), and a rounded bfloat16 copy is written for the compress and
// decode calls.
//
// Both statistics are products with the chunk's d x d Gram matrix
// G = X^T X (associativity):  X^T Y = G B,  Y^T Y = B^T G B.  G does not
// depend on the rank, its bfloat16 x bfloat16 products are exact in the
// matrix cores' float32 accumulation, and forming it streams the chunk once.
// Three launches, all deterministic (fixed summation orders, no atomics):
//   gram   per (run of 128-token steps, kv head): the run's partial G on the
//          matrix cores.  A step's tokens are staged in LDS token-major; each
//          matrix-core operand (16 dims x 8 consecutive tokens per lane
//          group) is read transposed with ds_read_b64_tr_b16, and the same
//          operand serves as row operand (G's row block) and as column
//          operand (its column block).  Loads run two steps ahead.
//   s1     per 4 rows of G: the runs' partials summed in a fixed order,
//          then those rows of S1 = G B, float32; the workgroup also copies
//          its 4 rows of B to the workspace (the basis before the step).
//   apply  per 4-row block of B: B + eta (S1 - B S2) with
//          B S2 = B B^T S1 = (B_rows B^T) S1 formed from the copies of B
//          and S1 (so S2 itself is never formed), float32, written back to
//          the float32 basis and, rounded to nearest even, to the bfloat16
//          copy (the copy of B keeps other workgroups' in-place writes out
//          of each workgroup's reads).
// Chunks of at most kOjaSmallTokens tokens per head take a single launch
// instead (oja_small_kernel, the same update in its per-token form).
#include <type_traits>

#include "lrkv_device.h"
#include "lrkv_internal.h"

namespace lrkv {

namespace {

// LDS of a gram workgroup: two step tiles of kOjaGramStep token rows, each
// row 128 elements (256 bytes, one pass of the LDS banks; head_dim 64 uses
// half of it).  The 16-byte chunks of row t are permuted by an xor with
// gram_swz(t), an even value that takes eight different values on the rows
// t0 .. t0 + 3 and t0 + 8 .. t0 + 11 (t0 a multiple of 4): a transposed read
// of half a wave covers exactly those rows, 32 bytes (two chunks) of each,
// which then land in sixteen different chunks, i.e. all 64 banks once.
constexpr int kGramRow = 128;
__device__ __forceinline__ int gram_swz(int row) { return 2 * ((row & 3) | (((row >> 3) & 1) << 2)); }
__device__ __forceinline__ int gram_off(int row, int chunk) { return row * kGramRow + ((chunk ^ gram_swz(row)) << 3); }

// One workgroup per (run of tokens, kv head), four waves.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void oja_gram_kernel(OjaArgs a) {
  constexpr int NBLK = D / 16;                       // 16-dim blocks
  constexpr int CPR = D / 8;                         // 16-byte chunks per token row
  constexpr int PIECES = kOjaGramStep * CPR / 256;   // 16-byte loads per thread per step
  __shared__ __attribute__((aligned(16))) uint16_t tile[2][kOjaGramStep * kGramRow];
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int n16 = lane & 15, grp = lane >> 4;
  const int h = blockIdx.y, wg = blockIdx.x;
  const int64_t n = a.n_tokens;
  const int64_t t_begin = n * wg / a.n_wg, t_end = n * (wg + 1) / a.n_wg;
  const int steps = (int)((t_end - t_begin + kOjaGramStep - 1) / kOjaGramStep);
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const int64_t row_stride = (int64_t)a.hkv * D;   // elements from one token of a head to the next

  // Step s: piece p = tid + 256 u is chunk p % CPR of token p / CPR.  Tokens
  // past the run (and every token of a step past the last) read zero: the
  // buffer range ends with the last valid token's row.
  auto load = [&](u32x4 (&buf)[PIECES], int s) {
    const int64_t t0 = t_begin + (int64_t)s * kOjaGramStep;
    const int64_t left = s < steps ? t_end - t0 : 0;
    const int nt = left < kOjaGramStep ? (int)left : kOjaGramStep;
    const uint32_t bytes = nt > 0 ? (uint32_t)(((int64_t)(nt - 1) * row_stride + D) * 2) : 0u;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(s < steps ? x + (t0 * a.hkv + h) * D : x, bytes);
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
      const int p = tid + 256 * u;
      buf[u] = buf_load16_stream(rs, (uint32_t)(((p / CPR) * row_stride + (p % CPR) * 8) * 2));
    }
  };
  auto stage = [&](const u32x4 (&buf)[PIECES], uint16_t* t) {
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
      const int p = tid + 256 * u;
      *reinterpret_cast<u32x4*>(t + gram_off(p / CPR, p % CPR)) = buf[u];
    }
  };
  // Operand of dim block blk for tokens k0 .. k0 + 31: lane (n16, grp) holds
  // dim 16 blk + n16 of tokens k0 + 8 grp .. + 7 (two transposed reads of
  // four tokens each).
  auto operand = [&](const uint16_t* t, int blk, int k0) {
    const int c = 2 * blk + ((n16 >> 1) & 1), hf = n16 & 1;
    const int r = k0 + 8 * grp + (n16 >> 2);
    const u32x2 lo = lds_read_tr16(t + gram_off(r, c) + 4 * hf);
    const u32x2 hi = lds_read_tr16(t + gram_off(r + 4, c) + 4 * hf);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };

  // G is symmetric, so only its tiles (I, J) with I <= J are formed.  Wave
  // w < NBLK / 2 owns the row blocks P = w and Q = NBLK - 1 - w: the tiles
  // (P, J >= P) and (Q, J >= Q), NBLK + 1 of them (9 at D = 128, every wave;
  // 5 at D = 64, waves 0 and 1), from the column operands J >= P.  The
  // wave's work is a compile-time function of w, so each wave runs its own
  // instantiation of the loop (all of them pass the same barriers).
  u32x4 b0[PIECES], b1[PIECES];
  float* out = a.ws + ((int64_t)h * a.n_wg + wg) * D * D;
  auto run = [&](auto wtag) {
    constexpr int W = decltype(wtag)::value;
    constexpr bool kOwns = W < NBLK / 2;
    constexpr int P = W, Q = NBLK - 1 - W;
    constexpr int NP = kOwns ? NBLK - P : 0, NQ = kOwns ? NBLK - Q : 0;
    f32x4 ap[NP > 0 ? NP : 1], aq[NQ > 0 ? NQ : 1];
#pragma unroll
    for (int j = 0; j < NP; ++j) ap[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NQ; ++j) aq[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto accumulate = [&](const uint16_t* t) {
      if (!kOwns) return;
#pragma unroll
      for (int k0 = 0; k0 < kOjaGramStep; k0 += 32) {
        u32x4 col[NP > 0 ? NP : 1];   // column blocks P .. NBLK - 1
#pragma unroll
        for (int j = 0; j < NP; ++j) col[j] = operand(t, P + j, k0);
#pragma unroll
        for (int j = 0; j < NP; ++j) ap[j] = mfma_16x16x32(col[0], col[j], ap[j]);
#pragma unroll
        for (int j = 0; j < NQ; ++j) aq[j] = mfma_16x16x32(col[Q - P], col[Q - P + j], aq[j]);
      }
    };
    // Two register buffers and two LDS tiles, used in turn: step s is staged
    // into tile s % 2 from its registers, which then take step s + 2; after
    // the barrier every wave accumulates the tile.  The barrier also orders
    // every wave's reads of a tile before that tile is staged again.  (Loads
    // three steps ahead, with three tiles, measured the same.)
    auto step = [&](u32x4 (&buf)[PIECES], int s, uint16_t* t) {
      stage(buf, t);
      load(buf, s + 2);
      __syncthreads();
      accumulate(t);
    };
    load(b0, 0);
    load(b1, 1);
    for (int s = 0; s < steps; s += 2) {
      step(b0, s, tile[0]);
      if (s + 1 >= steps) break;
      step(b1, s + 1, tile[1]);
    }
    // The run's partial G, both triangles: lane (n16, grp) register e of
    // tile (I, J) is G[16 I + 4 grp + e][16 J + n16]; an off-diagonal tile is
    // also stored as its mirror, G[16 J + n16][16 I + 4 grp + e .. + 3], four
    // consecutive floats per lane.
    auto put = [&](int I, int J, const f32x4& v) {
#pragma unroll
      for (int e = 0; e < 4; ++e) out[(16 * I + 4 * grp + e) * D + 16 * J + n16] = v[e];
      if (J != I) *reinterpret_cast<f32x4*>(out + (16 * J + n16) * D + 16 * I + 4 * grp) = v;
    };
#pragma unroll
    for (int j = 0; j < NP; ++j) put(P, P + j, ap[j]);
#pragma unroll
    for (int j = 0; j < NQ; ++j) put(Q, Q + j, aq[j]);
  };
  switch (wave) {
    case 0: run(std::integral_constant<int, 0>{}); break;
    case 1: run(std::integral_constant<int, 1>{}); break;
    case 2: run(std::integral_constant<int, 2>{}); break;
    default: run(std::integral_constant<int, 3>{}); break;
  }
}

// n floats (a multiple of 4, both ends 16-byte aligned) from global memory
// to LDS, 16 bytes per load, eight loads per thread in flight before their
// stores (a load-store loop would wait for each load in turn).
__device__ __forceinline__ void copy_to_lds(float* dst, const float* src, int n) {
  const int n4 = n / 4;
  for (int i0 = threadIdx.x; i0 < n4; i0 += 256 * 8) {
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + 256 * u;
      v[u] = i < n4 ? reinterpret_cast<const f32x4*>(src)[i] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + 256 * u;
      if (i < n4) reinterpret_cast<f32x4*>(dst)[i] = v[u];
    }
  }
}

// Rows row0 .. row0 + kS1Rows - 1 of S1 = G B for one head.  The rows of G
// are the sums of the runs' partials: thread t sums float4 column c4 of row
// rr over the runs of one parity (t / 128: even or odd runs, sixteen loads
// in flight), and the row is the even runs' sum plus the odd runs' sum
// (a fixed order).  Columns r .. R - 1 of S1 (R = the rank padded to 16) are
// written as zero.  B is staged in LDS; thread j forms column j of all the
// rows, so each B element it reads serves kS1Rows products.
constexpr int kS1Rows = 4;
__global__ __launch_bounds__(256) void oja_s1_kernel(OjaArgs a, int R) {
  __shared__ __attribute__((aligned(16))) float s_b[128 * 128];
  __shared__ __attribute__((aligned(16))) float s_g[2][kS1Rows][128];
  const int tid = threadIdx.x;
  const int h = blockIdx.y, row0 = kS1Rows * blockIdx.x;
  const int d = a.d, r = a.rank;
  const int q4 = d / 4;   // float4 columns per row
  const int par = tid >> 7, t = tid & 127;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  const bool summer = t < kS1Rows * q4;
  const int rr = t / q4, c4 = t - rr * q4;
  if (summer) {
    const f32x4* src = reinterpret_cast<const f32x4*>(a.ws + (int64_t)h * a.n_wg * d * d + (int64_t)(row0 + rr) * d) + c4;
    const int64_t stride4 = (int64_t)d * d / 4;
    for (int w0 = par; w0 < a.n_wg; w0 += 32) {
      f32x4 v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int w = w0 + 2 * u;
        v[u] = w < a.n_wg ? src[(int64_t)w * stride4] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (w0 + 2 * u < a.n_wg) acc += v[u];
    }
  }
  copy_to_lds(s_b, a.basis + (int64_t)h * d * r, d * r);
  if (summer) *reinterpret_cast<f32x4*>(&s_g[par][rr][4 * c4]) = acc;
  __syncthreads();
  for (int i = tid; i < kS1Rows * d; i += 256) {
    const int r2 = i / d, c = i - r2 * d;
    s_g[0][r2][c] += s_g[1][r2][c];
  }
  __syncthreads();
  float* s1 = a.ws_sum + (int64_t)h * oja_head_floats(d, R);
  // the basis before the step, rows row0 .. row0 + kS1Rows - 1 (from LDS)
  float* b_old = s1 + (int64_t)d * R;
  for (int i = tid; i < kS1Rows * r; i += 256) b_old[(int64_t)row0 * r + i] = s_b[row0 * r + i];
  for (int j = tid; j < R; j += 256) {
    float o[kS1Rows];
#pragma unroll
    for (int q = 0; q < kS1Rows; ++q) o[q] = 0.f;
    if (j < r) {
      for (int k = 0; k < d; k += 4) {
        const float b0 = s_b[k * r + j], b1 = s_b[(k + 1) * r + j], b2 = s_b[(k + 2) * r + j],
                    b3 = s_b[(k + 3) * r + j];
#pragma unroll
        for (int q = 0; q < kS1Rows; ++q) {
          const f32x4 g4 = *reinterpret_cast<const f32x4*>(&s_g[0][q][k]);
          o[q] = fmaf(g4[3], b3, fmaf(g4[2], b2, fmaf(g4[1], b1, fmaf(g4[0], b0, o[q]))));
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kS1Rows; ++q) s1[(int64_t)(row0 + q) * R + j] = o[q];
  }
}

// B <- B + eta (S1 - B S2) for kOjaRows rows of one head's basis, with
// B_rows S2 = (B_rows B^T) S1: P = B_rows B^T [kOjaRows][d] (thread k forms
// column k), then thread j forms column j of P S1.  The whole basis before
// the step and S1 come from the workspace (staged in LDS); the workgroup's
// rows of the float32 basis are written only after that.
constexpr int kOjaRows = 4;
template <int R>
__global__ __launch_bounds__(256) void oja_apply_kernel(OjaArgs a) {
  __shared__ __attribute__((aligned(16))) float s_s1[128 * R];
  __shared__ __attribute__((aligned(16))) float s_bo[128 * R];
  __shared__ __attribute__((aligned(16))) float s_p[kOjaRows][128];
  const int h = blockIdx.y, row0 = kOjaRows * blockIdx.x;
  const int tid = threadIdx.x;
  const int r = a.rank, d = a.d;
  const float* sum = a.ws_sum + (int64_t)h * oja_head_floats(d, R);
  const float* b_old = sum + (int64_t)d * R;
  copy_to_lds(s_s1, sum, d * R);
  copy_to_lds(s_bo, b_old, d * r);
  __syncthreads();
  // P = B_rows B^T
  for (int k = tid; k < d; k += 256) {
    float p[kOjaRows];
#pragma unroll
    for (int q = 0; q < kOjaRows; ++q) p[q] = 0.f;
    for (int c = 0; c < r; c += 4) {   // r is a multiple of 8
      const f32x4 bk = *reinterpret_cast<const f32x4*>(&s_bo[k * r + c]);
#pragma unroll
      for (int q = 0; q < kOjaRows; ++q) {
        const f32x4 bq = *reinterpret_cast<const f32x4*>(&s_bo[(row0 + q) * r + c]);
        p[q] = fmaf(bq[3], bk[3], fmaf(bq[2], bk[2], fmaf(bq[1], bk[1], fmaf(bq[0], bk[0], p[q]))));
      }
    }
#pragma unroll
    for (int q = 0; q < kOjaRows; ++q) s_p[q][k] = p[q];
  }
  __syncthreads();
  float* bs = a.basis + (int64_t)h * d * r;
  uint16_t* bb = static_cast<uint16_t*>(a.basis_bf16);
  for (int j = tid; j < r; j += 256) {
    float dot[kOjaRows];
#pragma unroll
    for (int q = 0; q < kOjaRows; ++q) dot[q] = 0.f;
    for (int k = 0; k < d; k += 4) {
      const float s0 = s_s1[k * R + j], s1 = s_s1[(k + 1) * R + j], s2 = s_s1[(k + 2) * R + j],
                  s3 = s_s1[(k + 3) * R + j];
#pragma unroll
      for (int q = 0; q < kOjaRows; ++q) {
        const f32x4 p4 = *reinterpret_cast<const f32x4*>(&s_p[q][k]);
        dot[q] = fmaf(p4[3], s3, fmaf(p4[2], s2, fmaf(p4[1], s1, fmaf(p4[0], s0, dot[q]))));
      }
    }
#pragma unroll
    for (int q = 0; q < kOjaRows; ++q) {
      const float v = s_bo[(row0 + q) * r + j] + a.eta * (s_s1[(row0 + q) * R + j] - dot[q]);
      const int64_t o = (int64_t)(row0 + q) * r + j;
      bs[o] = v;
      if (bb) bb[(int64_t)h * d * r + o] = f32_to_bf16(v);
    }
  }
}

// Chunks of at most kOjaSmallTokens tokens per head (a decode step's
// tokens): the whole update of a head's basis in one workgroup, in float32
// on the vector ALUs, in the per-token form of the rule.  With
// Y = X B and the residuals R = X - Y B^T,
//   X^T Y - B Y^T Y = (X - Y B^T)^T Y = R^T Y,
// which takes 3 n d r multiply-adds against the d r^2 of forming B Y^T Y,
// and one launch instead of three.  The workgroup reads its head's basis
// into LDS before anything is written, and no other workgroup touches that
// head, so the update is in place.
// 1024 threads (four waves per SIMD) hide more of each phase's dependent
// LDS-and-multiply chains than 512: 11.1 / 17.2 against 11.7 / 19.6 us at
// ranks 32 / 112 (batch 16, one token).
constexpr int kOjaSmallThreads = 1024;
template <int D>
__global__ __launch_bounds__(kOjaSmallThreads) void oja_small_kernel(OjaArgs a) {
  constexpr int P = D + 4;                  // row pitch of the token-by-dim and basis rows (floats)
  __shared__ __attribute__((aligned(16))) float s_x[kOjaSmallTokens][P];   // X, then R
  __shared__ __attribute__((aligned(16))) float s_b[D][P];                 // B [dim][coefficient]
  __shared__ __attribute__((aligned(16))) float s_y[kOjaSmallTokens][P];   // Y [token][coefficient]
  const int tid = threadIdx.x, h = blockIdx.x;
  const int r = a.rank, n = (int)a.n_tokens;
  float* bs = a.basis + (int64_t)h * D * r;
  // 1. the basis and the tokens (zero rows past n) into LDS, as float32;
  //    every load of a thread is issued before the first store
  constexpr int kBPieces = D * D / 4;                 // float4 of B, at most
  constexpr int kXPieces = kOjaSmallTokens * D / 8;   // 8-element pieces of the token rows
  constexpr int kB4 = (kBPieces + kOjaSmallThreads - 1) / kOjaSmallThreads;   // per thread
  constexpr int kX8 = (kXPieces + kOjaSmallThreads - 1) / kOjaSmallThreads;
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  f32x4 bv[kB4];
  u32x4 xv[kX8];
#pragma unroll
  for (int k = 0; k < kB4; ++k) {
    const int i = tid + kOjaSmallThreads * k;
    if (i < D * r / 4) bv[k] = *reinterpret_cast<const f32x4*>(bs + 4 * i);
  }
#pragma unroll
  for (int k = 0; k < kX8; ++k) {
    const int i = tid + kOjaSmallThreads * k;
    const int t = (8 * i) / D, e = (8 * i) % D;
    xv[k] = i < kXPieces && t < n ? *reinterpret_cast<const u32x4*>(x + ((int64_t)t * a.hkv + h) * D + e)
                                   : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int k = 0; k < kB4; ++k) {
    const int i = tid + kOjaSmallThreads * k;
    const int e = (4 * i) / r, c = (4 * i) % r;   // r is a multiple of 8
    if (i < D * r / 4) *reinterpret_cast<f32x4*>(&s_b[e][c]) = bv[k];
  }
#pragma unroll
  for (int k = 0; k < kX8; ++k) {
    const int i = tid + kOjaSmallThreads * k;
    const int t = (8 * i) / D, e = (8 * i) % D;
    if (i >= kXPieces) continue;
    *reinterpret_cast<f32x4*>(&s_x[t][e]) = f32x4{bf16_lo(xv[k][0]), bf16_hi(xv[k][0]), bf16_lo(xv[k][1]), bf16_hi(xv[k][1])};
    *reinterpret_cast<f32x4*>(&s_x[t][e + 4]) = f32x4{bf16_lo(xv[k][2]), bf16_hi(xv[k][2]), bf16_lo(xv[k][3]), bf16_hi(xv[k][3])};
  }
  __syncthreads();
  // 2. Y = X B: a thread takes one token and 8 coefficients, contracting
  //    over the dims (a broadcast X value and two 16-byte rows of B per dim).
  //    (Pairs of lanes each taking half of the dims, added with one lane
  //    exchange, measured slower: 19.5 against 17.2 us at rank 112.)
  for (int i = tid; i < n * (r / 8); i += kOjaSmallThreads) {
    const int t = i / (r / 8), c0 = 8 * (i % (r / 8));
    float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int e = 0; e < D; ++e) {
      const float xv = s_x[t][e];
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(&s_b[e][c0]);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(&s_b[e][c0 + 4]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        y[q] = fmaf(xv, b0[q], y[q]);
        y[4 + q] = fmaf(xv, b1[q], y[4 + q]);
      }
    }
    *reinterpret_cast<f32x4*>(&s_y[t][c0]) = f32x4{y[0], y[1], y[2], y[3]};
    *reinterpret_cast<f32x4*>(&s_y[t][c0 + 4]) = f32x4{y[4], y[5], y[6], y[7]};
  }
  __syncthreads();
  // 3. R = X - Y B^T in place of X: a thread takes one (token, dim),
  //    contracting over the coefficients; the lanes of a wave take
  //    consecutive dims of one token, so the Y row is a broadcast and the B
  //    rows (pitch D + 4 floats) fall in distinct banks (with four dims per
  //    lane the rows read together are four apart: 16-way bank conflicts);
  //    four partial sums, one per float4 lane, keep the chains r / 4 long
  for (int i = tid; i < n * D; i += kOjaSmallThreads) {
    const int t = i / D, e = i % D;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int c = 0; c < r; c += 4) {
      const f32x4 yv = *reinterpret_cast<const f32x4*>(&s_y[t][c]);
      const f32x4 bv = *reinterpret_cast<const f32x4*>(&s_b[e][c]);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fmaf(yv[q], bv[q], acc[q]);
    }
    s_x[t][e] -= (acc[0] + acc[1]) + (acc[2] + acc[3]);
  }
  __syncthreads();
  // 4. B += eta R^T Y: a thread takes one dim and 8 coefficients,
  //    contracting over the tokens; float32 result and its bfloat16 copy
  uint16_t* bb = a.basis_bf16 ? static_cast<uint16_t*>(a.basis_bf16) + (int64_t)h * D * r : nullptr;
  for (int i = tid; i < D * (r / 8); i += kOjaSmallThreads) {
    const int e = i / (r / 8), c0 = 8 * (i % (r / 8));
    float g[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int t = 0; t < n; ++t) {
      const float rv = s_x[t][e];
      const f32x4 y0 = *reinterpret_cast<const f32x4*>(&s_y[t][c0]);
      const f32x4 y1 = *reinterpret_cast<const f32x4*>(&s_y[t][c0 + 4]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        g[q] = fmaf(rv, y0[q], g[q]);
        g[4 + q] = fmaf(rv, y1[q], g[4 + q]);
      }
    }
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = fmaf(a.eta, g[q], s_b[e][c0 + q]);
    *reinterpret_cast<f32x4*>(bs + (int64_t)e * r + c0) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(bs + (int64_t)e * r + c0 + 4) = f32x4{v[4], v[5], v[6], v[7]};
    if (bb) {
      *reinterpret_cast<u32x4*>(bb + (int64_t)e * r + c0) =
          u32x4{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7])};
    }
  }
}

}  // namespace

hipError_t launch_oja_update(const OjaArgs& a, hipStream_t s) {
  const int nb = (a.rank + 15) / 16;
  if (a.d != 64 && a.d != 128) return hipErrorInvalidValue;
  if (nb < 1 || nb > a.d / 16 || a.rank % 8) return hipErrorInvalidValue;
  if (a.n_tokens <= kOjaSmallTokens) {   // a decode step's tokens: one launch
    if (a.d == 128) hipLaunchKernelGGL(oja_small_kernel<128>, dim3(a.hkv), dim3(kOjaSmallThreads), 0, s, a);
    else hipLaunchKernelGGL(oja_small_kernel<64>, dim3(a.hkv), dim3(kOjaSmallThreads), 0, s, a);
    return hipGetLastError();
  }
  if (a.n_wg < 1) return hipErrorInvalidValue;
  const int R = 16 * nb;
  if (a.d == 128) hipLaunchKernelGGL(oja_gram_kernel<128>, dim3(a.n_wg, a.hkv), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(oja_gram_kernel<64>, dim3(a.n_wg, a.hkv), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(oja_s1_kernel, dim3(a.d / kS1Rows, a.hkv), dim3(256), 0, s, a, R);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 agrid((unsigned)(a.d / kOjaRows), a.hkv);
  switch (nb) {
    case 1: hipLaunchKernelGGL(oja_apply_kernel<16>, agrid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(oja_apply_kernel<32>, agrid, dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL(oja_apply_kernel<48>, agrid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL(oja_apply_kernel<64>, agrid, dim3(256), 0, s, a); break;
    case 5: hipLaunchKernelGGL(oja_apply_kernel<80>, agrid, dim3(256), 0, s, a); break;
    case 6: hipLaunchKernelGGL(oja_apply_kernel<96>, agrid, dim3(256), 0, s, a); break;
    case 7: hipLaunchKernelGGL(oja_apply_kernel<112>, agrid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL(oja_apply_kernel<128>, agrid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lrkv
