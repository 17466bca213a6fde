// Compress / append: coeff[b, h, pos + t, :] = x[b, t, h, :] @ basis[h]  (gfx950).
//
// bfloat16: a 64-token tile per workgroup, 16 tokens per wave, on the matrix
// cores.  The basis of the kv head is staged once per workgroup in LDS,
// transposed, so that both operands are read as 16-byte runs along the
// contraction (head_dim) axis: tokens' rows straight from HBM, basis columns
// from LDS.  float32 accumulation, one rounding to bfloat16 at the store.
// float32: one thread per (token, coefficient) on the vector ALU.
#include "lrkv_device.h"
#include "lrkv_internal.h"

namespace lrkv {

namespace {

constexpr int kTile = 64;
constexpr int kPad = 8;   // LDS row padding (elements) against bank conflicts

__device__ __forceinline__ int64_t coeff_index(int values_layout, int64_t bh, int64_t cap, int r,
                                               int64_t p, int col) {
  return values_layout ? bh * cap * r + ((p >> 3) * r + col) * 8 + (p & 7)
                       : (bh * cap + p) * r + col;
}

template <int D, int NB>
__global__ __launch_bounds__(256) void compress_bf16_kernel(CompressArgs a) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n16 = lane & 15;
  const int grp = lane >> 4;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int r = a.rank;
  const int64_t bh = (int64_t)b * a.hkv + h;

  __shared__ uint16_t s_bt[NB * 16][D + kPad];

  const uint16_t* bs = static_cast<const uint16_t*>(a.basis) + (int64_t)h * D * r;
  for (int i = tid; i < D * r; i += 256) {
    const int dd = i / r, c = i - dd * r;
    s_bt[c][dd] = bs[i];
  }
  for (int i = tid; i < (NB * 16 - r) * D; i += 256) s_bt[r + i / D][i % D] = 0;
  __syncthreads();

  const int64_t t0 = (int64_t)blockIdx.x * kTile + wave * 16;
  const int64_t tok = t0 + n16;
  const bool valid = tok < a.n_tokens;
  const uint16_t* xrow = static_cast<const uint16_t*>(a.x) + ((b * a.n_tokens + tok) * a.hkv + h) * D;

  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    const int k = 32 * c + 8 * grp;
    const u32x4 xa = valid ? *reinterpret_cast<const u32x4*>(xrow + k) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const u32x4 bb = *reinterpret_cast<const u32x4*>(&s_bt[16 * nb + n16][k]);
      acc[nb] = mfma_16x16x32(xa, bb, acc[nb]);
    }
  }
  // lane (n16, grp) holds coefficient 16*nb + n16 of tokens t0 + 4*grp + i
  uint16_t* out = static_cast<uint16_t*>(a.coeff);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int col = 16 * nb + n16;
    if (col < r) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + 4 * grp + i;
        if (t < a.n_tokens)
          out[coeff_index(a.values_layout, bh, a.cap, r, a.pos + t, col)] = f32_to_bf16(acc[nb][i]);
      }
    }
  }
}

__global__ __launch_bounds__(256) void compress_f32_kernel(CompressArgs a) {
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int r = a.rank;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t t = idx / r;
  const int c = (int)(idx - t * r);
  if (t >= a.n_tokens) return;
  const float* x = static_cast<const float*>(a.x) + ((b * a.n_tokens + t) * a.hkv + h) * a.d;
  const float* bs = static_cast<const float*>(a.basis) + (int64_t)h * a.d * r + c;
  float acc = 0.f;
  for (int e = 0; e < a.d; ++e) acc = fmaf(x[e], bs[(int64_t)e * r], acc);
  const int64_t bh = (int64_t)b * a.hkv + h;
  static_cast<float*>(a.coeff)[coeff_index(a.values_layout, bh, a.cap, r, a.pos + t, c)] = acc;
}

}  // namespace

#define LRKV_COMPRESS_CASE(D, NB)                                                        \
  case (D * 16 + NB):                                                                    \
    hipLaunchKernelGGL((compress_bf16_kernel<D, NB>), grid, dim3(256), 0, s, a);         \
    break;

hipError_t launch_compress_bf16(const CompressArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.n_tokens + kTile - 1) / kTile), a.hkv, a.batch);
  const int nb = (a.rank + 15) / 16;
  switch (a.d * 16 + nb) {
    LRKV_COMPRESS_CASE(64, 1) LRKV_COMPRESS_CASE(64, 2) LRKV_COMPRESS_CASE(64, 3)
    LRKV_COMPRESS_CASE(64, 4)
    LRKV_COMPRESS_CASE(128, 1) LRKV_COMPRESS_CASE(128, 2) LRKV_COMPRESS_CASE(128, 3)
    LRKV_COMPRESS_CASE(128, 4) LRKV_COMPRESS_CASE(128, 5) LRKV_COMPRESS_CASE(128, 6)
    LRKV_COMPRESS_CASE(128, 7) LRKV_COMPRESS_CASE(128, 8)
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_compress_f32(const CompressArgs& a, hipStream_t s) {
  const int64_t total = a.n_tokens * a.rank;
  const dim3 grid((unsigned)((total + 255) / 256), a.hkv, a.batch);
  hipLaunchKernelGGL(compress_f32_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lrkv
