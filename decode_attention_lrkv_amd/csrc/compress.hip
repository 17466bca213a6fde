// Compress / append: coeff[b, h, pos + t, :] = x[b, t, h, :] @ basis[h]  (gfx950).
//
// bfloat16: a 128-token tile per workgroup on the matrix cores, 16 tokens per
// wave at a time.  The basis of the kv head is staged once per workgroup in
// LDS, transposed, so that both operands are read as 16-byte runs along the
// contraction (head_dim) axis: tokens' rows straight from HBM, basis columns
// from LDS.  float32 accumulation, one rounding to bfloat16, and the tile's
// coefficients leave through LDS as 16-byte stores (key rows, or whole value
// octets; element stores only for octets cut by the tile's ends).
// float32: one thread per (token, coefficient) on the vector ALU.
#include "lrkv_device.h"
#include "lrkv_internal.h"

namespace lrkv {

namespace {

constexpr int kTile = 128;   // tokens per workgroup (bfloat16 path)

__device__ __forceinline__ int64_t coeff_index(int values_layout, int64_t bh, int64_t cap, int r,
                                               int64_t p, int col) {
  return values_layout ? bh * cap * r + ((p >> 3) * r + col) * 8 + (p & 7)
                       : (bh * cap + p) * r + col;
}

// The LDS of one compress workgroup.
template <int D, int NB>
struct CompressSmem {
  static constexpr int kOutRow = NB * 16 + 4;
  static constexpr int kOutCol = kTile + 12;
  static constexpr int kOutElems = kTile * kOutRow > NB * 16 * kOutCol ? kTile * kOutRow : NB * 16 * kOutCol;
  // basis, transposed; a pitch of 8 x odd dwords keeps the 16-byte operand reads conflict-free
  __attribute__((aligned(16))) uint16_t bt[NB * 16][D + 16];
  // the tile's coefficients: keys as [token][column]; values as [column][slot]
  // with slot = token + (p0 % 8), so each destination octet is 16 aligned
  // bytes.  Both row pitches are 2 x odd dwords, which keeps the 2-byte writes
  // from the matrix-core layout and the 8-byte reads free of bank conflicts.
  __attribute__((aligned(16))) uint16_t out[kOutElems];
};

// One cache's coefficients for this workgroup's run of tiles (stages the basis first).
template <int D, int NB>
__device__ __forceinline__ void compress_part(const CompressArgs& a, CompressSmem<D, NB>& sm) {
  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = tid & 63;
  const int n16 = lane & 15;
  const int grp = lane >> 4;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int r = a.rank;
  const int64_t bh = (int64_t)b * a.hkv + h;
  auto& s_bt = sm.bt;
  uint16_t* s_out = sm.out;
  constexpr int kOutRow = CompressSmem<D, NB>::kOutRow;
  constexpr int kOutCol = CompressSmem<D, NB>::kOutCol;

  // basis rows arrive as 16-byte runs of 8 coefficients (all loads issued
  // before the first wait) and are written transposed
  {
    // piece i = (8-column group, head_dim row); consecutive lanes take
    // consecutive rows, so the transposed 2-byte LDS writes hit distinct banks
    const uint16_t* bs = static_cast<const uint16_t*>(a.basis) + (int64_t)h * D * r;
    const int n = D * (r / 8);
    constexpr int kIter = (D * NB * 16 / 8 + 255) / 256;
    u32x4 w[kIter];
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
      const int i = tid + 256 * it;
      if (i < n) w[it] = *reinterpret_cast<const u32x4*>(bs + (i % D) * r + (i / D) * 8);
    }
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
      const int i = tid + 256 * it;
      if (i < n) {
        const int dd = i % D, c = (i / D) * 8;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s_bt[c + 2 * e][dd] = (uint16_t)(w[it][e] & 0xFFFFu);
          s_bt[c + 2 * e + 1][dd] = (uint16_t)(w[it][e] >> 16);
        }
      }
    }
    for (int i = tid; i < (NB * 16 - r) * D; i += 256) s_bt[r + i / D][i % D] = 0;
  }
  __syncthreads();

  // The workgroup walks a contiguous run of tiles of this (b, h); the basis
  // above is staged once.  Contiguous runs keep a value octet cut by a tile
  // boundary in one workgroup (one L2), so its two partial writes merge
  // before they reach memory.  Each wave takes two 16-token sub-tiles per
  // tile, and the next tile's rows are loaded while the current tile is
  // multiplied and stored.
  constexpr int kSubs = kTile / 16 / 4;
  const int64_t n_tiles = (a.n_tokens + kTile - 1) / kTile;
  auto load_tile = [&](u32x4 (&xa)[kSubs][D / 32], int64_t tile) {
#pragma unroll
    for (int u = 0; u < kSubs; ++u) {
      const int64_t tok = tile * kTile + 16 * (wave + 4 * u) + n16;
      const bool valid = tok < a.n_tokens;
      const uint16_t* xrow = static_cast<const uint16_t*>(a.x) + ((b * a.n_tokens + tok) * a.hkv + h) * D;
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
        xa[u][c] = valid ? *reinterpret_cast<const u32x4*>(xrow + 32 * c + 8 * grp) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  uint16_t* out = static_cast<uint16_t*>(a.coeff);
  u32x4 xa[kSubs][D / 32], xb[kSubs][D / 32];
  const int64_t per_wg = (n_tiles + gridDim.x - 1) / gridDim.x;
  int64_t tile = blockIdx.x * per_wg;
  const int64_t tile_end = tile + per_wg < n_tiles ? tile + per_wg : n_tiles;
  if (tile < tile_end) load_tile(xa, tile);
  for (; tile < tile_end; ++tile) {
    const int64_t next = tile + 1;
    if (next < tile_end) load_tile(xb, next);
    const int64_t t_base = tile * kTile;
    const int64_t left = a.n_tokens - t_base;
    const int nt = left < kTile ? (int)left : kTile;
    const int64_t p0 = a.pos + t_base;                   // destination row of the tile's first token
    const int shift = (int)(p0 & 7);
#pragma unroll
    for (int u = 0; u < kSubs; ++u) {
      const int sub = wave + 4 * u;
      if (16 * sub < nt) {
        f32x4 acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
          const int k = 32 * c + 8 * grp;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            acc[nb] = mfma_16x16x32(xa[u][c], *reinterpret_cast<const u32x4*>(&s_bt[16 * nb + n16][k]), acc[nb]);
        }
        // lane (n16, grp) holds coefficient 16*nb + n16 of tokens 16*sub + 4*grp + i
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tl = 16 * sub + 4 * grp + i, col = 16 * nb + n16;
            const int at = a.values_layout ? col * kOutCol + shift + tl : tl * kOutRow + col;
            s_out[at] = f32_to_bf16(acc[nb][i]);
          }
      }
    }
    __syncthreads();
    if (!a.values_layout) {
      // key rows: each destination row is r/8 aligned 16-byte pieces
      const int per_row = r / 8;
      uint16_t* dst = out + (bh * a.cap + p0) * r;
      for (int i = tid; i < nt * per_row; i += 256) {
        const int tl = i / per_row, c = (i - tl * per_row) * 8;
        const uint2* src = reinterpret_cast<const uint2*>(&s_out[tl * kOutRow + c]);
        const uint2 lo = src[0], hi = src[1];
        *reinterpret_cast<u32x4*>(dst + (int64_t)tl * r + c) = u32x4{lo.x, lo.y, hi.x, hi.y};
      }
    } else {
      // value octets: a whole octet is one 16-byte LDS read and one 16-byte
      // store; octets cut by the tile's ends are written element by element
      const int64_t o_first = p0 >> 3, o_last = (p0 + nt - 1) >> 3;
      const int n_oct = (int)(o_last - o_first + 1);
      uint16_t* dst = out + bh * a.cap * r;
      for (int i = tid; i < n_oct * r; i += 256) {
        const int oi = i / r, col = i - oi * r;
        const int64_t o = o_first + oi;
        const int first = 8 * oi - shift;                  // tile-local token of element 0
        uint16_t* q = dst + (o * r + col) * 8;
        const uint16_t* src = &s_out[col * kOutCol + 8 * oi];
        if (first >= 0 && first + 8 <= nt) {
          const uint2 lo = reinterpret_cast<const uint2*>(src)[0], hi = reinterpret_cast<const uint2*>(src)[1];
          *reinterpret_cast<u32x4*>(q) = u32x4{lo.x, lo.y, hi.x, hi.y};
        } else {
          for (int e = 0; e < 8; ++e) {
            const int tl = first + e;
            if (tl >= 0 && tl < nt) q[e] = src[e];
          }
        }
      }
    }
    __syncthreads();   // s_out is rewritten by the next tile
#pragma unroll
    for (int u = 0; u < kSubs; ++u)
#pragma unroll
      for (int c = 0; c < D / 32; ++c) xa[u][c] = xb[u][c];
  }
}

template <int D, int NB>
__global__ __launch_bounds__(256) void compress_bf16_kernel(CompressArgs a) {
  __shared__ CompressSmem<D, NB> sm;
  compress_part<D, NB>(a, sm);
}

// Both caches of a prefill chunk in one launch: every workgroup writes the
// key coefficients of its run of tiles, then (basis restaged) the value
// coefficients of the same tokens.  NB covers the larger rank.
template <int D, int NB>
__global__ __launch_bounds__(256) void compress_pair_bf16_kernel(CompressArgs k, CompressArgs v) {
  __shared__ CompressSmem<D, NB> sm;
  compress_part<D, NB>(k, sm);
  __syncthreads();   // the value basis is staged over the key basis
  compress_part<D, NB>(v, sm);
}

// Few tokens (an appended decode token): both caches in one launch, one
// workgroup per (batch, kv head), no LDS staging of the bases.  Threads
// 0..127 compute the key coefficients and 128..255 the value coefficients:
// thread (8-column group, 16-row slice of head_dim) accumulates 8 columns
// over 16 rows from 16-byte basis loads, and the slices are summed in LDS.
template <int D>
__global__ __launch_bounds__(256) void compress_kv_small_kernel(CompressKvArgs a) {
  const int tid = threadIdx.x;
  const int kind = tid >> 7;                 // 0: keys, 1: values
  const int t7 = tid & 127;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int r = kind ? a.rv : a.rk;
  const int groups = r / 8;
  constexpr int kSlices = 8, kRows = D / kSlices;
  const int cg = t7 % 16, sl = t7 / 16;      // column group, head_dim slice
  const int64_t bh = (int64_t)b * a.hkv + h;
  const uint16_t* basis = static_cast<const uint16_t*>(kind ? a.bv : a.bk) + (int64_t)h * D * r;
  const uint16_t* x = static_cast<const uint16_t*>(kind ? a.xv : a.xk);

  __shared__ float s_x[2][kSmallT][D];
  __shared__ float s_part[2][kSlices][kSmallT][128];
  for (int i = t7; i < a.n_tokens * D; i += 128) {
    const int t = i / D, e = i - t * D;
    s_x[kind][t][e] = bf16_to_f32(x[((b * a.n_tokens + t) * a.hkv + h) * D + e]);
  }
  u32x4 w[kRows];
  if (cg < groups) {
#pragma unroll
    for (int e = 0; e < kRows; ++e)
      w[e] = *reinterpret_cast<const u32x4*>(basis + (sl * kRows + e) * r + cg * 8);
  }
  __syncthreads();
  if (cg < groups) {
    for (int t = 0; t < a.n_tokens; ++t) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < kRows; ++e) {
        const float xv = s_x[kind][t][sl * kRows + e];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[2 * k] = fmaf(xv, bf16_lo(w[e][k]), acc[2 * k]);
          acc[2 * k + 1] = fmaf(xv, bf16_hi(w[e][k]), acc[2 * k + 1]);
        }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) s_part[kind][sl][t][cg * 8 + k] = acc[k];
    }
  }
  __syncthreads();
  uint16_t* out = static_cast<uint16_t*>(kind ? a.cv : a.ck);
  for (int i = t7; i < a.n_tokens * r; i += 128) {
    const int t = i / r, col = i - t * r;
    float v = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < kSlices; ++s2) v += s_part[kind][s2][t][col];
    const int64_t p = a.pos + t;
    const int64_t at = kind ? bh * a.cap * r + ((p >> 3) * r + col) * 8 + (p & 7) : (bh * a.cap + p) * r + col;
    out[at] = f32_to_bf16(v);
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
  // about two resident workgroups per compute unit, each looping over tiles
  const int64_t tiles = (a.n_tokens + kTile - 1) / kTile;
  const int64_t units = (int64_t)a.hkv * a.batch;
  int64_t per_unit = (512 + units - 1) / units;
  if (per_unit > tiles) per_unit = tiles;
  if (per_unit < 1) per_unit = 1;
  const dim3 grid((unsigned)per_unit, a.hkv, a.batch);
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

#define LRKV_PAIR_CASE(D, NB)                                                            \
  case (D * 16 + NB):                                                                    \
    hipLaunchKernelGGL((compress_pair_bf16_kernel<D, NB>), grid, dim3(256), 0, s, k, v); \
    break;

hipError_t launch_compress_pair_bf16(const CompressArgs& k, const CompressArgs& v, hipStream_t s) {
  if (k.n_tokens != v.n_tokens || k.batch != v.batch || k.hkv != v.hkv || k.d != v.d) return hipErrorInvalidValue;
  const int64_t tiles = (k.n_tokens + kTile - 1) / kTile;
  const int64_t units = (int64_t)k.hkv * k.batch;
  int64_t per_unit = (512 + units - 1) / units;
  if (per_unit > tiles) per_unit = tiles;
  if (per_unit < 1) per_unit = 1;
  const dim3 grid((unsigned)per_unit, k.hkv, k.batch);
  const int nb = ((k.rank > v.rank ? k.rank : v.rank) + 15) / 16;
  switch (k.d * 16 + nb) {
    LRKV_PAIR_CASE(64, 1) LRKV_PAIR_CASE(64, 2) LRKV_PAIR_CASE(64, 3) LRKV_PAIR_CASE(64, 4)
    LRKV_PAIR_CASE(128, 1) LRKV_PAIR_CASE(128, 2) LRKV_PAIR_CASE(128, 3) LRKV_PAIR_CASE(128, 4)
    LRKV_PAIR_CASE(128, 5) LRKV_PAIR_CASE(128, 6) LRKV_PAIR_CASE(128, 7) LRKV_PAIR_CASE(128, 8)
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_compress_kv_small_bf16(const CompressKvArgs& a, hipStream_t s) {
  const dim3 grid(a.hkv, a.batch);
  if (a.d == 128) hipLaunchKernelGGL(compress_kv_small_kernel<128>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(compress_kv_small_kernel<64>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_compress_f32(const CompressArgs& a, hipStream_t s) {
  const int64_t total = a.n_tokens * a.rank;
  const dim3 grid((unsigned)((total + 255) / 256), a.hkv, a.batch);
  hipLaunchKernelGGL(compress_f32_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lrkv
