// Online basis update by Oja's subspace rule (gfx950).
//
// For the basis B [d, r] of one kv head and the new tokens x_t of a chunk
// (every batch row): Y = X B, then B <- B + eta (X^T Y - B Y^T Y).  The basis
// is kept in float32 (steps of the size Oja's rule takes fall below bfloat16
// resolution), and a rounded bfloat16 copy is written for the compress and
// decode calls.  Three launches, all deterministic:
//   stats   per (run of 16 W-token steps, kv head).  A step's tokens go to LDS
//           (as X, and as X^T transposed on the matrix cores; tiles in a
//           bank-conflict-free swizzled layout), loaded three
//           steps ahead; each wave owns some 16-column coefficient blocks,
//           computes their Y on the matrix cores (B split into high and low
//           bfloat16 parts, held in registers, so Y keeps float32 accuracy),
//           stores it (again as high + low parts) and accumulates its columns
//           of S1 = X^T Y [d, r] and its half of the symmetric S2 = Y^T Y
//           [r, r], contracting over the step's tokens.  The workgroup writes
//           its partial sums.
//   reduce  sums every kv head's partials in a fixed order.
//   apply   B + eta (S1 - B S2) in float32 per 4-row block of B, written
//           back to the float32 basis and, rounded to nearest even, to the
//           bfloat16 copy.
// Chunks of at most kOjaSmallTokens tokens per head take a single launch
// instead (oja_small_kernel, the same update in its per-token form).
#include "lrkv_device.h"
#include "lrkv_internal.h"

namespace lrkv {

namespace {

// W waves per stats workgroup; a step is 16 tokens per wave.
template <int W> constexpr int oja_step() { return 16 * W; }

// The step's bfloat16 tiles use the swizzled LDS layout of lds_swz (rows of
// 64 or 128 elements), so that the matrix-core operand reads are free of bank
// conflicts.
template <int D, int NB, int W>
struct OjaSmem {
  static constexpr int R = 16 * NB;        // rank padded to whole 16-column blocks
  static constexpr int S = oja_step<W>();
  uint16_t xs[S * D];                      // X of the step, token-major [token][dim] (Y's row operand)
  uint16_t xt[D * S];                      // X^T of the step: [dim][token] (S1's row operand)
  uint16_t yt_hi[R * S];                   // Y^T of the step: [coefficient][token], high parts
  uint16_t yt_lo[R * S];                   // low parts: Y - high
};

// S2 = Y^T Y is symmetric, so of its 16 x 16 tiles (row block na, column
// block nb) only one of each mirrored pair is formed: the tiles
// ((nb + j) mod NB, nb) for j < NB / 2 + 1; when NB is even the tile at
// j = NB / 2 has its mirror at j = NB / 2 too, so it is formed only for
// nb < NB / 2.  Every unordered pair of blocks is then formed exactly once,
// and each column block forms about half a column.  Tiles that are not
// formed hold no partial sums (their reduced values are never read); the
// apply step reads them transposed from their mirrors.
__host__ __device__ constexpr bool oja_s2_formed(int na, int nb, int nb_total) {
  return ((na - nb + nb_total) % nb_total) < (nb_total + 1) / 2 ||
         (nb_total % 2 == 0 && (na - nb + nb_total) % nb_total == nb_total / 2 && nb < nb_total / 2);
}

// Per-head partial sums of one stats workgroup: S1 [D][R] then S2 [R][R]
// (the tiles oja_s2_formed names; the others are not written); the layout
// helper oja_head_floats is in lrkv_internal.h.

// Wave w owns the 16-column coefficient blocks w, w + W, ... (NBW of them at
// most): it keeps their B^T rows in registers for the whole launch, computes
// their Y for all tokens of a step, and accumulates their columns of S1 and
// S2, so each Y operand it reads from LDS serves every row block.  W = 8 for
// ranks above 64 (one block per wave, registers for two waves per SIMD).
template <int D, int NB, int W>
__global__ __launch_bounds__(64 * W) void oja_stats_kernel(OjaArgs a) {
  constexpr int R = 16 * NB;
  constexpr int NBW = (NB + W - 1) / W;    // coefficient blocks per wave
  constexpr int KD = D / 32;               // 32-dim k-steps of Y = X B
  constexpr int STEP = oja_step<W>();
  constexpr int UNROLL = W == 4 ? 4 : 2;   // token-block and k-step loops (full unroll at 8 waves spills)
  __shared__ __attribute__((aligned(16))) OjaSmem<D, NB, W> sm;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int n16 = lane & 15, grp = lane >> 4;
  const int h = blockIdx.y;
  const int r = a.rank;
  // With fewer coefficient blocks than waves (W a multiple of NB), the
  // G = W / NB waves of a block share its work: wave w takes block w mod NB,
  // and of the token blocks, S1 row blocks and S2 tiles of that block the
  // ones numbered part, part + G, ... (part = w / NB).
  constexpr int G = (NB < W && W % NB == 0) ? W / NB : 1;
  constexpr int DBW = D / 16 / G;           // S1 row blocks per wave
  constexpr int NJW = (NB / 2 + G) / G;     // S2 tiles per wave and block
  const int part = G > 1 ? wave / NB : 0;
  const int bw = G > 1 ? wave % NB : wave;  // the wave's first coefficient block

  // this wave's B^T rows as matrix-core row operands, high and low bfloat16
  // parts: lane (n16, grp) of block k, step c holds B[32 c + 8 grp + e][16 nb + n16]
  u32x4 bt_hi[NBW][KD], bt_lo[NBW][KD];
  {
    const float* bs = a.basis + (int64_t)h * D * r;
#pragma unroll
    for (int k = 0; k < NBW; ++k) {
      const int col = 16 * (bw + W * k) + n16;
#pragma unroll
      for (int c = 0; c < KD; ++c) {
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r0 = 32 * c + 8 * grp + 2 * e;
          const float v0 = col < r ? bs[r0 * r + col] : 0.f;
          const float v1 = col < r ? bs[(r0 + 1) * r + col] : 0.f;
          hi[e] = pack_bf16(v0, v1);
          lo[e] = pack_bf16(v0 - bf16_lo(hi[e]), v1 - bf16_hi(hi[e]));
        }
        bt_hi[k][c] = u32x4{hi[0], hi[1], hi[2], hi[3]};
        bt_lo[k][c] = u32x4{lo[0], lo[1], lo[2], lo[3]};
      }
    }
  }

  constexpr int NJ = NB / 2 + 1;            // S2 tiles per column block: row blocks (nb + j) mod NB
  f32x4 s1[DBW][NBW], s2[NJW][NBW];
#pragma unroll
  for (int k = 0; k < NBW; ++k) {
#pragma unroll
    for (int i = 0; i < DBW; ++i) s1[i][k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < NJW; ++jj) s2[jj][k] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int64_t n_tok = a.n_tokens;
  const int64_t n_steps = (n_tok + STEP - 1) / STEP;
  const int64_t per_wg = (n_steps + gridDim.x - 1) / gridDim.x;
  const int64_t s_begin = (int64_t)blockIdx.x * per_wg;
  const int64_t s_end = s_begin + per_wg < n_steps ? s_begin + per_wg : n_steps;

  // this wave's 16 tokens of a step as loaded: lane (n16, grp) holds token
  // n16's dims 32 c + 8 grp .. + 7; tokens past the end read zero
  auto load_x = [&](u32x4 (&xa)[KD], int64_t step) {
    const int64_t t0 = step * STEP + 16 * wave;
    const int64_t left = n_tok - t0;
    const int nt = left <= 0 ? 0 : (left < 16 ? (int)left : 16);
    const int64_t t_base = nt > 0 ? t0 : 0;
    const uint16_t* x = static_cast<const uint16_t*>(a.x) + (t_base * a.hkv + h) * D;
    const uint32_t bytes = nt > 0 ? (uint32_t)(((nt - 1) * a.hkv + 1) * D * 2) : 0u;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(x, bytes);
    const uint32_t voff = (uint32_t)((n16 * a.hkv * D + 8 * grp) * 2);
#pragma unroll
    for (int c = 0; c < KD; ++c) xa[c] = buf_load16(rs, voff + 64 * c);
  };

  // 32 x 16 slices of the identity as column operands: lane (n16, grp) slot
  // e of slice hf is 1 where 8 grp + e = 16 hf + n16
  u32x4 eye[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      eye[hf][q] = (8 * grp + 2 * q == 16 * hf + n16 ? 0x3F80u : 0u) |
                   (8 * grp + 2 * q + 1 == 16 * hf + n16 ? 0x3F800000u : 0u);
  // only waves that own a coefficient block take part in Y, S1 and S2
  const bool owns = bw < NB;

  // A step's tokens are loaded kAhead steps before it runs, into a ring of
  // kAhead + 1 register buffers that the loop below rotates by name (a copy
  // between buffers would wait for the newest load).
  constexpr int kAhead = 3;
  static_assert(kAhead == 3, "the ring below has four buffers");
  u32x4 x0[KD], x1[KD], x2[KD], x3[KD];
  if (s_begin < s_end) load_x(x0, s_begin);
  if (s_begin + 1 < s_end) load_x(x1, s_begin + 1);
  if (s_begin + 2 < s_end) load_x(x2, s_begin + 2);
  auto run_step = [&](const u32x4 (&xa)[KD], u32x4 (&ahead)[KD], int64_t step) {
    if (step + kAhead < s_end) load_x(ahead, step + kAhead);
    // 1. X (token-major) and X^T into LDS.  The wave's own 16 tokens are
    //    transposed on the matrix cores: X times a slice of the identity puts
    //    dim 32 c + 16 hf + n16 of tokens 4 grp .. + 3 in lane (n16, grp)
    //    (exactly for finite tokens: each sum is one product by one and the
    //    rest products by zero), so
    //    X^T is stored four tokens at a time
    const int tok = 16 * wave + n16;
#pragma unroll
    for (int c = 0; c < KD; ++c) {
      *reinterpret_cast<u32x4*>(&sm.xs[lds_swz<D>(tok, 32 * c + 8 * grp)]) = xa[c];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const f32x4 t = mfma_16x16x32(xa[c], eye[hf], f32x4{0.f, 0.f, 0.f, 0.f});
        const u32x2 w = u32x2{(__float_as_uint(t[0]) >> 16) | (__float_as_uint(t[1]) & 0xFFFF0000u),
                              (__float_as_uint(t[2]) >> 16) | (__float_as_uint(t[3]) & 0xFFFF0000u)};
        *reinterpret_cast<u32x2*>(&sm.xt[lds_swz<STEP>(32 * c + 16 * hf + n16, 16 * wave + 4 * grp)]) = w;
      }
    }
    __syncthreads();
    // 2. Y of this wave's coefficient blocks for the step's W 16-token
    //    blocks, with the tokens as rows: lane (n16, grp) register i is
    //    coefficient 16 nb + n16 of token 16 tb + 4 grp + i, so its Y^T row
    //    is stored four tokens at a time, as high and low parts
    if (owns) {
#pragma unroll UNROLL
      for (int ti = 0; ti < W / G; ++ti) {
        const int tb = part + G * ti;
        u32x4 xo[KD];
#pragma unroll
        for (int c = 0; c < KD; ++c) xo[c] = *reinterpret_cast<const u32x4*>(&sm.xs[lds_swz<D>(16 * tb + n16, 32 * c + 8 * grp)]);
#pragma unroll
        for (int k = 0; k < NBW; ++k) {
          const int nb = bw + W * k;
          if (nb < NB) {
            f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < KD; ++c) {
              y = mfma_16x16x32(xo[c], bt_hi[k][c], y);
              y = mfma_16x16x32(xo[c], bt_lo[k][c], y);
            }
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              hi[i] = f32_to_bf16(y[i]);
              lo[i] = f32_to_bf16(y[i] - bf16_to_f32((uint16_t)hi[i]));
            }
            const int yo = lds_swz<STEP>(16 * nb + n16, 16 * tb + 4 * grp);
            *reinterpret_cast<u32x2*>(&sm.yt_hi[yo]) = u32x2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
            *reinterpret_cast<u32x2*>(&sm.yt_lo[yo]) = u32x2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
          }
        }
      }
    }
    __syncthreads();
    // 3. S1 += X^T Y and S2 += Y^T Y over the step's 16 W tokens, for this
    //    wave's coefficient columns: k-slots are tokens 32 kk + 8 grp .. + 7
    if (owns) {
#pragma unroll UNROLL
      for (int kk = 0; kk < W / 2; ++kk) {
        const int t = 32 * kk + 8 * grp;
        u32x4 bh[NBW], bl[NBW];
#pragma unroll
        for (int k = 0; k < NBW; ++k) {
          const int nb = bw + W * k < NB ? bw + W * k : 0;
          bh[k] = *reinterpret_cast<const u32x4*>(&sm.yt_hi[lds_swz<STEP>(16 * nb + n16, t)]);
          bl[k] = *reinterpret_cast<const u32x4*>(&sm.yt_lo[lds_swz<STEP>(16 * nb + n16, t)]);
        }
#pragma unroll
        for (int i = 0; i < DBW; ++i) {
          const int db = part + G * i;
          const u32x4 xr = *reinterpret_cast<const u32x4*>(&sm.xt[lds_swz<STEP>(16 * db + n16, t)]);
#pragma unroll
          for (int k = 0; k < NBW; ++k) {
            if (bw + W * k < NB) {
              s1[i][k] = mfma_16x16x32(xr, bh[k], s1[i][k]);
              s1[i][k] = mfma_16x16x32(xr, bl[k], s1[i][k]);
            }
          }
        }
#pragma unroll
        for (int k = 0; k < NBW; ++k) {
          const int nb = bw + W * k;
          if (nb < NB) {
#pragma unroll
            for (int jj = 0; jj < NJW; ++jj) {
              const int j = part + G * jj;
              const int na = (nb + j) % NB;
              if (j < NJ && oja_s2_formed(na, nb, NB)) {
                const u32x4 ah = *reinterpret_cast<const u32x4*>(&sm.yt_hi[lds_swz<STEP>(16 * na + n16, t)]);
                const u32x4 al = *reinterpret_cast<const u32x4*>(&sm.yt_lo[lds_swz<STEP>(16 * na + n16, t)]);
                s2[jj][k] = mfma_16x16x32(ah, bh[k], s2[jj][k]);
                s2[jj][k] = mfma_16x16x32(ah, bl[k], s2[jj][k]);
                s2[jj][k] = mfma_16x16x32(al, bh[k], s2[jj][k]);
              }
            }
          }
        }
      }
    }
    __syncthreads();   // the next step rewrites X, X^T and Y^T
  };
  for (int64_t step = s_begin; step < s_end; step += kAhead + 1) {
    run_step(x0, x3, step);
    if (step + 1 < s_end) run_step(x1, x0, step + 1);
    if (step + 2 < s_end) run_step(x2, x1, step + 2);
    if (step + 3 < s_end) run_step(x3, x2, step + 3);
  }

  // partial sums of this workgroup (zeros when it had no steps); result lane
  // (n16, grp) register i holds row 4 grp + i, column n16 of its tile
  float* w1 = a.ws + ((int64_t)h * gridDim.x + blockIdx.x) * oja_head_floats(D, R);
  float* w2 = w1 + (int64_t)D * R;
#pragma unroll
  for (int k = 0; k < NBW; ++k) {
    const int nb = bw + W * k;
    if (nb < NB) {
#pragma unroll
      for (int di = 0; di < DBW; ++di) {
        const int db = part + G * di;
#pragma unroll
        for (int i = 0; i < 4; ++i) w1[(16 * db + 4 * grp + i) * R + 16 * nb + n16] = s1[di][k][i];
      }
#pragma unroll
      for (int jj = 0; jj < NJW; ++jj) {
        const int j = part + G * jj;
        const int na = (nb + j) % NB;
        if (j < NJ && oja_s2_formed(na, nb, NB)) {
#pragma unroll
          for (int i = 0; i < 4; ++i) w2[(16 * na + 4 * grp + i) * R + 16 * nb + n16] = s2[jj][k][i];
        }
      }
    }
  }
}

// Sum of the stats workgroups' partials of every head, in workgroup order.
__global__ __launch_bounds__(256) void oja_reduce_kernel(OjaArgs a, int64_t per_head) {
  const int h = blockIdx.y;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= per_head) return;
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
  const float* src = a.ws + (int64_t)h * a.n_wg * per_head + i;
  // the loads of eight partials in flight; the sum keeps workgroup order
#pragma unroll 8
  for (int w = 0; w < a.n_wg; ++w) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(src + (int64_t)w * per_head);
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] += v[e];
  }
  *reinterpret_cast<f32x4*>(a.ws_sum + (int64_t)h * per_head + i) = s;
}

// B <- B + eta (S1 - B S2) for kOjaRows rows of one head's basis.  The rows
// are staged in LDS before any is written, and no other workgroup touches
// them.
constexpr int kOjaRows = 4;
template <int R>
__global__ __launch_bounds__(256) void oja_apply_kernel(OjaArgs a) {
  __shared__ float s_s2[R][R + 1];
  __shared__ float s_b[kOjaRows][R + 1];
  const int h = blockIdx.y, row0 = kOjaRows * blockIdx.x;
  const int tid = threadIdx.x;
  const int r = a.rank, d = a.d;
  const int64_t per_head = oja_head_floats(d, R);
  const float* sum = a.ws_sum + (int64_t)h * per_head;
  float* bs = a.basis + (int64_t)h * d * r;
  // tiles that were not formed are the transposes of their mirrors
  for (int i = tid; i < R * R; i += 256) {
    const int k = i / R, j = i % R;
    s_s2[k][j] = oja_s2_formed(k / 16, j / 16, R / 16) ? sum[(int64_t)d * R + i] : sum[(int64_t)d * R + j * R + k];
  }
  for (int i = tid; i < kOjaRows * r; i += 256) s_b[i / r][i % r] = bs[(int64_t)(row0 + i / r) * r + i % r];
  __syncthreads();
  uint16_t* bb = static_cast<uint16_t*>(a.basis_bf16);
  for (int i = tid; i < kOjaRows * r; i += 256) {
    const int rr = i / r, j = i % r;
    // four partial sums (r is a multiple of 8): no single dependent chain
    float d4[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < r; k += 4)
#pragma unroll
      for (int u = 0; u < 4; ++u) d4[u] = fmaf(s_b[rr][k + u], s_s2[k + u][j], d4[u]);
    const float dot = (d4[0] + d4[1]) + (d4[2] + d4[3]);
    const float v = s_b[rr][j] + a.eta * (sum[(int64_t)(row0 + rr) * R + j] - dot);
    const int64_t o = (int64_t)(row0 + rr) * r + j;
    bs[o] = v;
    if (bb) bb[(int64_t)h * d * r + o] = f32_to_bf16(v);
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
constexpr int kOjaSmallThreads = 512;
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
  constexpr int kB4 = D * D / 4 / kOjaSmallThreads;              // float4 of B per thread, at most
  constexpr int kX8 = kOjaSmallTokens * D / 8 / kOjaSmallThreads; // 8-token-element pieces per thread
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
    xv[k] = t < n ? *reinterpret_cast<const u32x4*>(x + ((int64_t)t * a.hkv + h) * D + e) : u32x4{0u, 0u, 0u, 0u};
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
    *reinterpret_cast<f32x4*>(&s_x[t][e]) = f32x4{bf16_lo(xv[k][0]), bf16_hi(xv[k][0]), bf16_lo(xv[k][1]), bf16_hi(xv[k][1])};
    *reinterpret_cast<f32x4*>(&s_x[t][e + 4]) = f32x4{bf16_lo(xv[k][2]), bf16_hi(xv[k][2]), bf16_lo(xv[k][3]), bf16_hi(xv[k][3])};
  }
  __syncthreads();
  // 2. Y = X B: a thread takes one token and 8 coefficients, contracting
  //    over the dims (a broadcast X value and two 16-byte rows of B per dim)
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
  // 3. R = X - Y B^T in place of X: a thread takes one token and 4 dims,
  //    contracting over the coefficients (both rows contiguous in them)
  for (int i = tid; i < n * (D / 4); i += kOjaSmallThreads) {
    const int t = i / (D / 4), e0 = 4 * (i % (D / 4));
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int c = 0; c < r; c += 4) {
      const f32x4 yv = *reinterpret_cast<const f32x4*>(&s_y[t][c]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 bv = *reinterpret_cast<const f32x4*>(&s_b[e0 + q][c]);
        acc[q] = fmaf(yv[0], bv[0], fmaf(yv[1], bv[1], fmaf(yv[2], bv[2], fmaf(yv[3], bv[3], acc[q]))));
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) s_x[t][e0 + q] -= acc[q];
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

#define LRKV_OJA_CASE4(D, NB)                                                                   \
  case NB:                                                                                      \
    hipLaunchKernelGGL((oja_stats_kernel<D, NB, 4>), dim3(a.n_wg, a.hkv), dim3(256), 0, s, a); \
    break;
#define LRKV_OJA_CASE8(D, NB)                                                                   \
  case NB:                                                                                      \
    hipLaunchKernelGGL((oja_stats_kernel<D, NB, 8>), dim3(a.n_wg, a.hkv), dim3(512), 0, s, a); \
    break;

hipError_t launch_oja_update(const OjaArgs& a, hipStream_t s) {
  const int nb = (a.rank + 15) / 16;
  if (a.d != 64 && a.d != 128) return hipErrorInvalidValue;
  if (nb < 1 || nb > a.d / 16 || a.rank % 8) return hipErrorInvalidValue;
  if (a.n_tokens <= kOjaSmallTokens) {   // a decode step's tokens: one launch
    if (a.d == 128) hipLaunchKernelGGL(oja_small_kernel<128>, dim3(a.hkv), dim3(kOjaSmallThreads), 0, s, a);
    else hipLaunchKernelGGL(oja_small_kernel<64>, dim3(a.hkv), dim3(kOjaSmallThreads), 0, s, a);
    return hipGetLastError();
  }
  if (a.d == 128) {
    switch (nb) {
      LRKV_OJA_CASE4(128, 1) LRKV_OJA_CASE4(128, 2) LRKV_OJA_CASE4(128, 3) LRKV_OJA_CASE4(128, 4)
      LRKV_OJA_CASE8(128, 5) LRKV_OJA_CASE8(128, 6) LRKV_OJA_CASE8(128, 7) LRKV_OJA_CASE8(128, 8)
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (nb) {
      LRKV_OJA_CASE4(64, 1) LRKV_OJA_CASE4(64, 2) LRKV_OJA_CASE4(64, 3) LRKV_OJA_CASE4(64, 4)
      default: return hipErrorInvalidValue;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t per_head = oja_head_floats(a.d, 16 * nb);
  const dim3 rgrid((unsigned)((per_head / 4 + 255) / 256), a.hkv);
  hipLaunchKernelGGL(oja_reduce_kernel, rgrid, dim3(256), 0, s, a, per_head);
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
