// Online basis update by Oja's subspace rule (gfx950).
//
// For the basis B [d, r] of one kv head and the new tokens x_t of a chunk
// (every batch row): Y = X B, then B <- B + eta (X^T Y - B Y^T Y).  The basis
// is kept in float32 (steps of the size Oja's rule takes fall below bfloat16
// resolution), and a rounded bfloat16 copy is written for the compress and
// decode calls.  Three launches, all deterministic:
//   stats   per (run of 64-token steps, kv head).  Each wave takes 16 tokens
//           of a step and computes their Y on the matrix cores (B split into
//           high and low bfloat16 parts, so Y keeps float32 accuracy).  X^T
//           and Y^T (again as high + low parts) go to LDS, and each wave
//           accumulates its tiles of S1 = X^T Y [d, r] and S2 = Y^T Y [r, r]
//           on the matrix cores, contracting over the step's 64 tokens.  The
//           workgroup writes its partial sums.
//   reduce  sums every kv head's partials in a fixed order.
//   apply   B + eta (S1 - B S2) in float32 per 16-row block of B, written
//           back to the float32 basis and, rounded to nearest even, to the
//           bfloat16 copy.
#include "lrkv_device.h"
#include "lrkv_internal.h"

namespace lrkv {

namespace {

constexpr int kOjaWaves = 4;
constexpr int kOjaStep = 16 * kOjaWaves;   // tokens per step, 16 per wave
constexpr int kOjaPitchT = kOjaStep + 8;   // bf16 pitch of the token-major LDS rows (144 bytes)

template <int D, int NB>
struct OjaSmem {
  static constexpr int R = 16 * NB;        // rank padded to whole 16-column blocks
  uint16_t bt_hi[R][D + 8];                // B^T (row = coefficient), high parts; rows >= rank are zero
  uint16_t bt_lo[R][D + 8];                // low parts: B - high
  uint16_t xt[D][kOjaPitchT];              // X^T of the step: [dim][token]
  uint16_t yt_hi[R][kOjaPitchT];           // Y^T of the step: [coefficient][token]
  uint16_t yt_lo[R][kOjaPitchT];
};

// Per-head partial sums of one stats workgroup: S1 [D][R] then S2 [R][R].
__host__ __device__ inline int64_t oja_head_floats(int d, int r_pad) { return (int64_t)d * r_pad + (int64_t)r_pad * r_pad; }

template <int D, int NB>
__global__ __launch_bounds__(256) void oja_stats_kernel(OjaArgs a) {
  constexpr int R = 16 * NB;
  constexpr int DB = D / 64;               // 16-dim blocks of S1 per wave (blocks wave, wave + 4, ...)
  constexpr int NA = (NB + 3) / 4;         // 16-row blocks of S2 per wave (blocks wave, wave + 4, ...)
  __shared__ __attribute__((aligned(16))) OjaSmem<D, NB> sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n16 = lane & 15, grp = lane >> 4;
  const int h = blockIdx.y;
  const int r = a.rank;

  // B^T as high and low bfloat16 parts; consecutive threads read consecutive
  // coefficients of one basis row
  const float* bs = a.basis + (int64_t)h * D * r;
  for (int i = tid; i < R * D; i += 256) {
    const int j = i % R, dd = i / R;
    const float v = j < r ? bs[dd * r + j] : 0.f;
    const uint16_t hi = f32_to_bf16(v);
    sm.bt_hi[j][dd] = hi;
    sm.bt_lo[j][dd] = f32_to_bf16(v - bf16_to_f32(hi));
  }

  f32x4 s1[DB][NB], s2[NA][NB];
#pragma unroll
  for (int k = 0; k < DB; ++k)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) s1[k][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < NA; ++k)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) s2[k][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t n_tok = a.n_tokens;
  const int64_t n_steps = (n_tok + kOjaStep - 1) / kOjaStep;
  const int64_t per_wg = (n_steps + gridDim.x - 1) / gridDim.x;
  const int64_t s_begin = (int64_t)blockIdx.x * per_wg;
  const int64_t s_end = s_begin + per_wg < n_steps ? s_begin + per_wg : n_steps;

  // this wave's 16 tokens of a step as matrix-core operands: lane (n16, grp)
  // holds token n16's dims 32 c + 8 grp .. + 7; tokens past the end read zero
  auto load_x = [&](u32x4 (&xa)[D / 32], int64_t step) {
    const int64_t t0 = step * kOjaStep + 16 * wave;
    const int64_t left = n_tok - t0;
    const int nt = left <= 0 ? 0 : (left < 16 ? (int)left : 16);
    const int64_t t_base = nt > 0 ? t0 : 0;
    const uint16_t* x = static_cast<const uint16_t*>(a.x) + (t_base * a.hkv + h) * D;
    const uint32_t bytes = nt > 0 ? (uint32_t)(((nt - 1) * a.hkv + 1) * D * 2) : 0u;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(x, bytes);
    const uint32_t voff = (uint32_t)((n16 * a.hkv * D + 8 * grp) * 2);
#pragma unroll
    for (int c = 0; c < D / 32; ++c) xa[c] = buf_load16(rs, voff + 64 * c);
  };

  __syncthreads();   // B^T staged

  u32x4 xa[D / 32], xb[D / 32];
  if (s_begin < s_end) load_x(xa, s_begin);
  for (int64_t step = s_begin; step < s_end; ++step) {
    if (step + 1 < s_end) load_x(xb, step + 1);
    // 1. Y^T of this wave's tokens: lane (n16, grp) register i of block nb is
    //    coefficient 16 nb + 4 grp + i of token n16
    f32x4 y[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      y[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const int k = 32 * c + 8 * grp;
        y[nb] = mfma_16x16x32(*reinterpret_cast<const u32x4*>(&sm.bt_hi[16 * nb + n16][k]), xa[c], y[nb]);
        y[nb] = mfma_16x16x32(*reinterpret_cast<const u32x4*>(&sm.bt_lo[16 * nb + n16][k]), xa[c], y[nb]);
      }
    }
    // 2. X^T and Y^T (high, low) of these tokens into LDS, token column 16 wave + n16
    const int col = 16 * wave + n16;
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sm.xt[32 * c + 8 * grp + 2 * e][col] = (uint16_t)(xa[c][e] & 0xFFFFu);
        sm.xt[32 * c + 8 * grp + 2 * e + 1][col] = (uint16_t)(xa[c][e] >> 16);
      }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = y[nb][i];
        const uint16_t hi = f32_to_bf16(v);
        sm.yt_hi[16 * nb + 4 * grp + i][col] = hi;
        sm.yt_lo[16 * nb + 4 * grp + i][col] = f32_to_bf16(v - bf16_to_f32(hi));
      }
    __syncthreads();
    // 3. S1 += X^T Y over the step's 64 tokens: row operand X^T (dim 16 db + n16),
    //    column operand Y (coefficient 16 nb + n16), k = tokens 32 kk + 8 grp .. + 7
#pragma unroll
    for (int k = 0; k < DB; ++k) {
      const int db = wave + 4 * k;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int t = 32 * kk + 8 * grp;
        const u32x4 xr = *reinterpret_cast<const u32x4*>(&sm.xt[16 * db + n16][t]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          s1[k][nb] = mfma_16x16x32(xr, *reinterpret_cast<const u32x4*>(&sm.yt_hi[16 * nb + n16][t]), s1[k][nb]);
          s1[k][nb] = mfma_16x16x32(xr, *reinterpret_cast<const u32x4*>(&sm.yt_lo[16 * nb + n16][t]), s1[k][nb]);
        }
      }
    }
    // 4. S2 += Y^T Y: row operand Y^T (coefficient 16 na + n16), column operand
    //    Y (coefficient 16 nb + n16); high x high + high x low + low x high
#pragma unroll
    for (int k = 0; k < NA; ++k) {
      const int na = wave + 4 * k;
      if (na < NB) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int t = 32 * kk + 8 * grp;
          const u32x4 ah = *reinterpret_cast<const u32x4*>(&sm.yt_hi[16 * na + n16][t]);
          const u32x4 al = *reinterpret_cast<const u32x4*>(&sm.yt_lo[16 * na + n16][t]);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const u32x4 bh = *reinterpret_cast<const u32x4*>(&sm.yt_hi[16 * nb + n16][t]);
            const u32x4 bl = *reinterpret_cast<const u32x4*>(&sm.yt_lo[16 * nb + n16][t]);
            s2[k][nb] = mfma_16x16x32(ah, bh, s2[k][nb]);
            s2[k][nb] = mfma_16x16x32(ah, bl, s2[k][nb]);
            s2[k][nb] = mfma_16x16x32(al, bh, s2[k][nb]);
          }
        }
      }
    }
    __syncthreads();   // the next step rewrites X^T and Y^T
#pragma unroll
    for (int c = 0; c < D / 32; ++c) xa[c] = xb[c];
  }

  // partial sums of this workgroup (zeros when it had no steps); result lane
  // (n16, grp) register i holds row 4 grp + i, column n16 of its tile
  float* w1 = a.ws + ((int64_t)h * gridDim.x + blockIdx.x) * oja_head_floats(D, R);
  float* w2 = w1 + (int64_t)D * R;
#pragma unroll
  for (int k = 0; k < DB; ++k)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) w1[(16 * (wave + 4 * k) + 4 * grp + i) * R + 16 * nb + n16] = s1[k][nb][i];
#pragma unroll
  for (int k = 0; k < NA; ++k) {
    const int na = wave + 4 * k;
    if (na < NB) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) w2[(16 * na + 4 * grp + i) * R + 16 * nb + n16] = s2[k][nb][i];
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
  for (int w = 0; w < a.n_wg; ++w) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(src + (int64_t)w * per_head);
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] += v[e];
  }
  *reinterpret_cast<f32x4*>(a.ws_sum + (int64_t)h * per_head + i) = s;
}

// B <- B + eta (S1 - B S2) for 16 rows of one head's basis.  The rows are
// staged in LDS before any is written, and no other workgroup touches them.
template <int R>
__global__ __launch_bounds__(256) void oja_apply_kernel(OjaArgs a) {
  __shared__ float s_s2[R][R + 1];
  __shared__ float s_b[16][R + 1];
  const int h = blockIdx.y, row0 = 16 * blockIdx.x;
  const int tid = threadIdx.x;
  const int r = a.rank, d = a.d;
  const int64_t per_head = oja_head_floats(d, R);
  const float* sum = a.ws_sum + (int64_t)h * per_head;
  float* bs = a.basis + (int64_t)h * d * r;
  for (int i = tid; i < R * R; i += 256) s_s2[i / R][i % R] = sum[(int64_t)d * R + i];
  for (int i = tid; i < 16 * r; i += 256) s_b[i / r][i % r] = bs[(int64_t)(row0 + i / r) * r + i % r];
  __syncthreads();
  uint16_t* bb = static_cast<uint16_t*>(a.basis_bf16);
  for (int i = tid; i < 16 * r; i += 256) {
    const int rr = i / r, j = i % r;
    float dot = 0.f;
    for (int k = 0; k < r; ++k) dot = fmaf(s_b[rr][k], s_s2[k][j], dot);
    const float v = s_b[rr][j] + a.eta * (sum[(int64_t)(row0 + rr) * R + j] - dot);
    const int64_t o = (int64_t)(row0 + rr) * r + j;
    bs[o] = v;
    if (bb) bb[(int64_t)h * d * r + o] = f32_to_bf16(v);
  }
}

}  // namespace

int oja_rank_pad(int rank) { return 16 * ((rank + 15) / 16); }

size_t oja_workspace_floats(int hkv, int d, int rank, int n_wg) {
  const int64_t per_head = oja_head_floats(d, oja_rank_pad(rank));
  return (size_t)((int64_t)hkv * n_wg * per_head + (int64_t)hkv * per_head);
}

#define LRKV_OJA_CASE(D, NB)                                                                 \
  case NB:                                                                                   \
    hipLaunchKernelGGL((oja_stats_kernel<D, NB>), dim3(a.n_wg, a.hkv), dim3(256), 0, s, a); \
    break;

hipError_t launch_oja_update(const OjaArgs& a, hipStream_t s) {
  const int nb = (a.rank + 15) / 16;
  if (a.d != 64 && a.d != 128) return hipErrorInvalidValue;
  if (nb < 1 || nb > a.d / 16) return hipErrorInvalidValue;
  if (a.d == 128) {
    switch (nb) {
      LRKV_OJA_CASE(128, 1) LRKV_OJA_CASE(128, 2) LRKV_OJA_CASE(128, 3) LRKV_OJA_CASE(128, 4)
      LRKV_OJA_CASE(128, 5) LRKV_OJA_CASE(128, 6) LRKV_OJA_CASE(128, 7) LRKV_OJA_CASE(128, 8)
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (nb) {
      LRKV_OJA_CASE(64, 1) LRKV_OJA_CASE(64, 2) LRKV_OJA_CASE(64, 3) LRKV_OJA_CASE(64, 4)
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
  const dim3 agrid((unsigned)(a.d / 16), a.hkv);
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
