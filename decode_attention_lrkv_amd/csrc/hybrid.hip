// Hybrid compress: tokens whose key or value is poorly reconstructed from
// its stored low-rank coefficients stay full rank in a side list; the others
// are appended to the low-rank caches (gfx950).
//
// Three launches, all deterministic (no order-dependent atomics):
//   select  per 64-token tile: c = round(x B) on the matrix cores, x_hat = c B^T
//           on the matrix cores, ||x - x_hat||^2 > tau^2 ||x||^2 in float32 for
//           K and for V; a token is flagged when either is; per-tile counts.
//   scan    per (b, kv head): exclusive prefix of the tile counts gives every
//           tile's first low-rank row and first side-list row; the counters
//           advance (clamped at the capacities, with an overflow flag).
//   write   per tile: recompute c, place each token at its tile offset plus its
//           rank among the tile's tokens of the same kind (a wave ballot).
#include "lrkv_device.h"
#include "lrkv_internal.h"

namespace lrkv {

namespace {

constexpr int kPad = 8;
constexpr int kMaxRank = 128;

enum Mode { kSelect = 0, kWrite = 1 };

template <int D>
__global__ __launch_bounds__(256) void hybrid_tile_kernel(HybridArgs a, int mode) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n16 = lane & 15;
  const int grp = lane >> 4;
  const int tile = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int64_t bh = (int64_t)b * a.hkv + h;
  const int64_t t_base = (int64_t)tile * kHybridTile;
  const int64_t rem = a.n_tokens - t_base;
  const int nt = rem < kHybridTile ? (int)rem : kHybridTile;
  const int64_t n_slots = (int64_t)a.n_tiles * kHybridTile;

  __shared__ uint16_t s_bt[kMaxRank][D + kPad];   // basis, transposed: [coefficient][dim]
  __shared__ uint16_t s_x[kHybridTile][D + kPad];  // the tile's key or value rows
  __shared__ uint16_t s_c[kHybridTile][kMaxRank + kPad];
  __shared__ int s_flag[kHybridTile];
  __shared__ int s_rank[kHybridTile];
  __shared__ int s_sel[kHybridTile];

  int64_t lr_off = 0, side_off = 0;
  if (mode == kWrite) {
    if (tid < kHybridTile) {
      const int f = tid < nt ? a.ws_flags[bh * n_slots + t_base + tid] : 0;
      const uint64_t mask = __ballot(f);
      const uint64_t below = mask & ((1ull << tid) - 1ull);
      const int n_side_before = __popcll(below);
      s_flag[tid] = f;
      s_rank[tid] = f ? n_side_before : tid - n_side_before;
    }
    lr_off = a.ws_offsets[(bh * a.n_tiles + tile) * 2 + 0];
    side_off = a.ws_offsets[(bh * a.n_tiles + tile) * 2 + 1];
  } else {
    if (tid < kHybridTile) s_sel[tid] = 0;
  }
  for (int i = tid; i < kHybridTile * (kMaxRank + kPad); i += 256) (&s_c[0][0])[i] = 0;

  for (int which = 0; which < 2; ++which) {
    const int r = which ? a.rv : a.rk;
    const uint16_t* basis = static_cast<const uint16_t*>(which ? a.bv : a.bk) + (int64_t)h * D * r;
    const uint16_t* x = static_cast<const uint16_t*>(which ? a.v : a.k);
    __syncthreads();
    for (int i = tid; i < D * kMaxRank; i += 256) {
      const int c = i / D, dd = i - c * D;
      s_bt[c][dd] = c < r ? basis[dd * r + c] : (uint16_t)0;
    }
    for (int i = tid; i < kHybridTile * (D / 8); i += 256) {
      const int tl = i / (D / 8), k8 = (i - tl * (D / 8)) * 8;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (tl < nt) v = *reinterpret_cast<const u32x4*>(x + ((b * a.n_tokens + t_base + tl) * a.hkv + h) * D + k8);
      *reinterpret_cast<u32x4*>(&s_x[tl][k8]) = v;
    }
    __syncthreads();

    // c = x B for the wave's 16 tokens; columns >= r come out zero.
    const int nbr = (r + 15) / 16;
    f32x4 acc1[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc1[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      const int k = 32 * c + 8 * grp;
      const u32x4 xa = *reinterpret_cast<const u32x4*>(&s_x[16 * wave + n16][k]);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        if (nb < nbr) acc1[nb] = mfma_16x16x32(xa, *reinterpret_cast<const u32x4*>(&s_bt[16 * nb + n16][k]), acc1[nb]);
    }

    if (mode == kSelect) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        if (nb < nbr)
#pragma unroll
          for (int i = 0; i < 4; ++i) s_c[16 * wave + 4 * grp + i][16 * nb + n16] = f32_to_bf16(acc1[nb][i]);
      __syncthreads();
      // x_hat = c B^T, one 16-dim block at a time; residual and norm per token
      const int kc2 = (r + 31) / 32;
      float e2[4] = {0.f, 0.f, 0.f, 0.f}, n2[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        f32x4 acc2 = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int c = 0; c < kc2; ++c) {
          const int k = 32 * c + 8 * grp;
          const u32x4 ca = *reinterpret_cast<const u32x4*>(&s_c[16 * wave + n16][k]);
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            w[e] = (uint32_t)s_bt[k + 2 * e][16 * db + n16] | ((uint32_t)s_bt[k + 2 * e + 1][16 * db + n16] << 16);
          acc2 = mfma_16x16x32(ca, u32x4{w[0], w[1], w[2], w[3]}, acc2);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float xv = bf16_to_f32(s_x[16 * wave + 4 * grp + i][16 * db + n16]);
          const float res = xv - acc2[i];
          e2[i] = fmaf(res, res, e2[i]);
          n2[i] = fmaf(xv, xv, n2[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          e2[i] += __shfl_xor(e2[i], o);
          n2[i] += __shfl_xor(n2[i], o);
        }
        if (n16 == 0 && e2[i] > a.tau2 * n2[i]) s_sel[16 * wave + 4 * grp + i] = 1;
      }
    } else {
      // low-rank tokens: coefficients to row (keys) or octet (values) layout
      uint16_t* out = static_cast<uint16_t*>(which ? a.cv : a.ck);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int col = 16 * nb + n16;
        if (nb < nbr && col < r) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tl = 16 * wave + 4 * grp + i;
            if (tl < nt && !s_flag[tl]) {
              const int64_t p = lr_off + s_rank[tl];
              if (p < a.cap) {
                const int64_t idx = which ? bh * a.cap * r + ((p >> 3) * r + col) * 8 + (p & 7)
                                          : (bh * a.cap + p) * r + col;
                out[idx] = f32_to_bf16(acc1[nb][i]);
              }
            }
          }
        }
      }
      // full-rank tokens: copy the rows bit for bit into the side list
      uint16_t* side = static_cast<uint16_t*>(which ? a.v_side : a.k_side);
      for (int i = tid; i < kHybridTile * D; i += 256) {
        const int tl = i / D, dd = i - tl * D;
        if (tl < nt && s_flag[tl]) {
          const int64_t p = side_off + s_rank[tl];
          if (p < a.side_cap) {
            const int64_t idx = which ? bh * a.side_cap * D + ((p >> 3) * D + dd) * 8 + (p & 7)
                                      : (bh * a.side_cap + p) * D + dd;
            side[idx] = s_x[tl][dd];
          }
        }
      }
    }
  }

  __syncthreads();
  if (mode == kSelect) {
    if (tid < kHybridTile) {
      const int f = tid < nt ? s_sel[tid] : 0;
      a.ws_flags[bh * n_slots + t_base + tid] = (uint8_t)f;
      if (a.flags && tid < nt) a.flags[bh * a.n_tokens + t_base + tid] = (uint8_t)f;
      const uint64_t mask = __ballot(f);
      if (tid == 0) a.ws_counts[bh * a.n_tiles + tile] = __popcll(mask);
    }
  } else if (tid < nt && s_flag[tid]) {
    const int64_t p = side_off + s_rank[tid];
    if (p < a.side_cap) a.side_idx[bh * a.side_cap + p] = (int32_t)(a.pos + t_base + tid);
  }
}

// Exclusive scan of the per-tile counts of one (b, kv head); advances the counters.
__global__ __launch_bounds__(256) void hybrid_scan_kernel(HybridArgs a) {
  const int tid = threadIdx.x;
  const int64_t bh = (int64_t)blockIdx.y * a.hkv + blockIdx.x;
  const int n = a.n_tiles;
  const int seg = (n + 255) / 256;
  const int j0 = tid * seg;
  const int j1 = j0 + seg < n ? j0 + seg : n;
  const int32_t* cnt = a.ws_counts + bh * n;
  const int64_t lr_base = a.n_lr[bh];
  const int64_t side_base = a.n_side[bh];

  __shared__ int64_t s_scan[256];
  int64_t local = 0;
  for (int j = j0; j < j1; ++j) local += cnt[j];
  s_scan[tid] = local;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int64_t v = tid >= o ? s_scan[tid - o] : 0;
    __syncthreads();
    s_scan[tid] += v;
    __syncthreads();
  }
  int64_t run = s_scan[tid] - local;   // flagged tokens before this thread's first tile
  for (int j = j0; j < j1; ++j) {
    a.ws_offsets[(bh * n + j) * 2 + 0] = (int32_t)(lr_base + (int64_t)j * kHybridTile - run);
    a.ws_offsets[(bh * n + j) * 2 + 1] = (int32_t)(side_base + run);
    run += cnt[j];
  }
  if (tid == 255) {
    const int64_t flagged = s_scan[255];
    int64_t new_side = side_base + flagged;
    int64_t new_lr = lr_base + (a.n_tokens - flagged);
    bool over = false;
    if (new_side > a.side_cap) { new_side = a.side_cap; over = true; }
    if (new_lr > a.cap) { new_lr = a.cap; over = true; }
    a.n_side[bh] = (int32_t)new_side;
    a.n_lr[bh] = (int32_t)new_lr;
    if (over) *a.overflow = 1;
  }
}

}  // namespace

hipError_t launch_hybrid_bf16(const HybridArgs& a, hipStream_t s) {
  const dim3 grid(a.n_tiles, a.hkv, a.batch);
  if (a.d == 128) hipLaunchKernelGGL(hybrid_tile_kernel<128>, grid, dim3(256), 0, s, a, (int)kSelect);
  else hipLaunchKernelGGL(hybrid_tile_kernel<64>, grid, dim3(256), 0, s, a, (int)kSelect);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(hybrid_scan_kernel, dim3(a.hkv, a.batch), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.d == 128) hipLaunchKernelGGL(hybrid_tile_kernel<128>, grid, dim3(256), 0, s, a, (int)kWrite);
  else hipLaunchKernelGGL(hybrid_tile_kernel<64>, grid, dim3(256), 0, s, a, (int)kWrite);
  return hipGetLastError();
}

}  // namespace lrkv
