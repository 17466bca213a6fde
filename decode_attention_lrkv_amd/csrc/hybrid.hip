// Hybrid compress: tokens whose key or value is poorly reconstructed from
// its stored low-rank coefficients stay full rank in a side list; the others
// are appended to the low-rank caches (gfx950).
//
// Three launches, all deterministic (no order-dependent atomics):
//   select  c = round(x B) and x_hat = c B^T on the matrix cores, then
//           ||x - x_hat||^2 > tau^2 ||x||^2 in float32, for K and for V; a token
//           is flagged when either is.  Per 16-token sub-tile: flags and count.
//   scan    per (b, kv head): exclusive prefix of the sub-tile counts gives every
//           sub-tile's first low-rank row and first side-list row; the counters
//           advance (clamped at the capacities, with an overflow flag).
//   write   recompute c; each token goes to its sub-tile's offset plus its rank
//           among the sub-tile's tokens of the same kind (a wave ballot).
// Select and write are persistent: a workgroup stages both bases in LDS once
// and its waves walk 16-token sub-tiles of one (b, kv head), each wave
// loading the next sub-tile's rows while it works on the current one.
#include "lrkv_device.h"
#include "lrkv_internal.h"

namespace lrkv {

namespace {

constexpr int kPad = 8;
constexpr int kMaxRank = 128;
constexpr int kWavesH = 8;                 // waves per hybrid workgroup
constexpr int kThreadsH = 64 * kWavesH;

// Both bases of kv head h, transposed ([coefficient][dim]); rows >= rank are zero.
template <int D>
__device__ void stage_bases(const HybridArgs& a, int h, uint16_t (*s_bt)[kMaxRank][D + kPad]) {
  const int tid = threadIdx.x;
  for (int kind = 0; kind < 2; ++kind) {
    const int r = kind ? a.rv : a.rk;
    const uint16_t* bs = static_cast<const uint16_t*>(kind ? a.bv : a.bk) + (int64_t)h * D * r;
    const int n = D * (r / 8);
    // piece i = (8-column group, head_dim row): consecutive lanes take consecutive
    // rows, so the transposed 2-byte LDS writes land in distinct banks
    for (int i0 = 0; i0 < n; i0 += 4 * kThreadsH) {
      u32x4 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + tid + kThreadsH * u;
        if (i < n) w[u] = *reinterpret_cast<const u32x4*>(bs + (i % D) * r + (i / D) * 8);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + tid + kThreadsH * u;
        if (i < n) {
          const int dd = i % D, c = (i / D) * 8;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s_bt[kind][c + 2 * e][dd] = (uint16_t)(w[u][e] & 0xFFFFu);
            s_bt[kind][c + 2 * e + 1][dd] = (uint16_t)(w[u][e] >> 16);
          }
        }
      }
    }
    for (int i = tid; i < (kMaxRank - r) * D; i += kThreadsH) s_bt[kind][r + i / D][i % D] = 0;
  }
}

// Rows of one 16-token sub-tile as matrix-core A operands: lane (n16, grp)
// holds token n16's elements 32c + 8 grp .. +7.
template <int D>
__device__ __forceinline__ void load_rows(const HybridArgs& a, int b, int h, int kind, int64_t sub, int n16,
                                          int grp, u32x4 (&xa)[D / 32]) {
  const int64_t tok = sub * kHybridTile + n16;
  const bool valid = tok < a.n_tokens;
  const uint16_t* x = static_cast<const uint16_t*>(kind ? a.v : a.k) + ((b * a.n_tokens + tok) * a.hkv + h) * D;
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
    xa[c] = valid ? *reinterpret_cast<const u32x4*>(x + 32 * c + 8 * grp) : u32x4{0u, 0u, 0u, 0u};
}

// c = x B for the sub-tile: acc[nb] lane (n16, grp) register i is coefficient
// 16 nb + n16 of token 4 grp + i.
template <int D>
__device__ __forceinline__ void coeffs(const u32x4 (&xa)[D / 32], const uint16_t (*bt)[D + kPad], int nbr, int n16,
                                       int grp, f32x4 (&acc)[8]) {
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    const int k = 32 * c + 8 * grp;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
      if (nb < nbr) acc[nb] = mfma_16x16x32(xa[c], *reinterpret_cast<const u32x4*>(&bt[16 * nb + n16][k]), acc[nb]);
  }
}

template <int D>
__global__ __launch_bounds__(kThreadsH) void hybrid_select_kernel(HybridArgs a) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n16 = lane & 15, grp = lane >> 4;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * a.hkv + h;
  const int64_t n_slots = (int64_t)a.n_tiles * kHybridTile;

  __shared__ __attribute__((aligned(16))) uint16_t s_bt[2][kMaxRank][D + kPad];
  __shared__ __attribute__((aligned(16))) uint16_t s_x[kWavesH][kHybridTile][D + kPad];
  __shared__ __attribute__((aligned(16))) uint16_t s_c[kWavesH][kHybridTile][kMaxRank + kPad];
  stage_bases<D>(a, h, s_bt);
  __syncthreads();

  const int64_t stride = (int64_t)gridDim.x * kWavesH;
  int64_t sub = (int64_t)blockIdx.x * kWavesH + wave;
  u32x4 xa[D / 32], xn[D / 32];
  if (sub < a.n_tiles) load_rows<D>(a, b, h, 0, sub, n16, grp, xa);
  for (; sub < a.n_tiles; sub += stride) {
    bool sel[4] = {false, false, false, false};
    for (int kind = 0; kind < 2; ++kind) {
      // rows of the next item: this sub-tile's values, or the next sub-tile's keys
      if (kind == 0) load_rows<D>(a, b, h, 1, sub, n16, grp, xn);
      else if (sub + stride < a.n_tiles) load_rows<D>(a, b, h, 0, sub + stride, n16, grp, xn);
      const int r = kind ? a.rv : a.rk;
      const int nbr = (r + 15) / 16, kc2 = (r + 31) / 32;
      const uint16_t (*bt)[D + kPad] = s_bt[kind];
#pragma unroll
      for (int c = 0; c < D / 32; ++c) *reinterpret_cast<u32x4*>(&s_x[wave][n16][32 * c + 8 * grp]) = xa[c];
      f32x4 acc1[8];
      coeffs<D>(xa, bt, nbr, n16, grp, acc1);
      // the stored coefficients, zero past the rank up to the reconstruction's k range
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        if (nb < 2 * kc2)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            s_c[wave][4 * grp + i][16 * nb + n16] = nb < nbr ? f32_to_bf16(acc1[nb][i]) : (uint16_t)0;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // x_hat = c B^T one 16-dim block at a time; residual and norm per token
      float e2[4] = {0.f, 0.f, 0.f, 0.f}, n2[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        f32x4 acc2 = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int c = 0; c < kc2; ++c) {
          const int k = 32 * c + 8 * grp;
          const u32x4 ca = *reinterpret_cast<const u32x4*>(&s_c[wave][n16][k]);
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            w[e] = (uint32_t)bt[k + 2 * e][16 * db + n16] | ((uint32_t)bt[k + 2 * e + 1][16 * db + n16] << 16);
          acc2 = mfma_16x16x32(ca, u32x4{w[0], w[1], w[2], w[3]}, acc2);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float xv = bf16_to_f32(s_x[wave][4 * grp + i][16 * db + n16]);
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
        sel[i] = sel[i] || (e2[i] > a.tau2 * n2[i]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();   // s_x and s_c are rewritten by the next item
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int c = 0; c < D / 32; ++c) xa[c] = xn[c];
    }
    // lanes (n16 = 0, grp) hold the flags of tokens 4 grp + i
    int count = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t tok = sub * kHybridTile + 4 * grp + i;
      const bool f = sel[i] && tok < a.n_tokens;
      if (n16 == 0 && tok < a.n_tokens) {
        a.ws_flags[bh * n_slots + tok] = (uint8_t)f;
        if (a.flags) a.flags[bh * a.n_tokens + tok] = (uint8_t)f;
      }
      count += __popcll(__ballot(n16 == 0 && f));
    }
    if (lane == 0) a.ws_counts[bh * a.n_tiles + sub] = count;
  }
}

template <int D>
__global__ __launch_bounds__(kThreadsH) void hybrid_write_kernel(HybridArgs a) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n16 = lane & 15, grp = lane >> 4;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * a.hkv + h;
  const int64_t n_slots = (int64_t)a.n_tiles * kHybridTile;

  __shared__ __attribute__((aligned(16))) uint16_t s_bt[2][kMaxRank][D + kPad];
  stage_bases<D>(a, h, s_bt);
  __syncthreads();

  const int64_t stride = (int64_t)gridDim.x * kWavesH;
  int64_t sub = (int64_t)blockIdx.x * kWavesH + wave;
  u32x4 xa[D / 32], xn[D / 32];
  if (sub < a.n_tiles) load_rows<D>(a, b, h, 0, sub, n16, grp, xa);
  for (; sub < a.n_tiles; sub += stride) {
    // flags of this sub-tile's tokens and each token's rank within its kind
    const int64_t tok_lane = sub * kHybridTile + n16;
    const bool f_lane = tok_lane < a.n_tokens && a.ws_flags[bh * n_slots + tok_lane];
    const uint32_t side_mask = (uint32_t)(__ballot(grp == 0 && f_lane) & 0xFFFFu);
    const int nt = (int)((a.n_tokens - sub * kHybridTile) < kHybridTile ? (a.n_tokens - sub * kHybridTile) : kHybridTile);
    const int64_t lr_off = a.ws_offsets[(bh * a.n_tiles + sub) * 2 + 0];
    const int64_t side_off = a.ws_offsets[(bh * a.n_tiles + sub) * 2 + 1];
    for (int kind = 0; kind < 2; ++kind) {
      if (kind == 0) load_rows<D>(a, b, h, 1, sub, n16, grp, xn);
      else if (sub + stride < a.n_tiles) load_rows<D>(a, b, h, 0, sub + stride, n16, grp, xn);
      const int r = kind ? a.rv : a.rk;
      const int nbr = (r + 15) / 16;
      f32x4 acc1[8];
      coeffs<D>(xa, s_bt[kind], nbr, n16, grp, acc1);
      // low-rank tokens: coefficients to the row (keys) or octet (values) layout
      uint16_t* out = static_cast<uint16_t*>(kind ? a.cv : a.ck);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tl = 4 * grp + i;
        if (tl < nt && !((side_mask >> tl) & 1u)) {
          const int64_t p = lr_off + tl - __popc(side_mask & ((1u << tl) - 1u));
          if (p < a.cap) {
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
              const int col = 16 * nb + n16;
              if (nb < nbr && col < r) {
                const int64_t idx = kind ? bh * a.cap * r + ((p >> 3) * r + col) * 8 + (p & 7)
                                         : (bh * a.cap + p) * r + col;
                out[idx] = f32_to_bf16(acc1[nb][i]);
              }
            }
          }
        }
      }
      // full-rank tokens: their rows, bit for bit, into the side list
      if (f_lane && n16 < nt) {
        const int64_t p = side_off + __popc(side_mask & ((1u << n16) - 1u));
        if (p < a.side_cap) {
          uint16_t* side = static_cast<uint16_t*>(kind ? a.v_side : a.k_side);
#pragma unroll
          for (int c = 0; c < D / 32; ++c) {
            const int col = 32 * c + 8 * grp;
            if (!kind) {
              *reinterpret_cast<u32x4*>(side + (bh * a.side_cap + p) * D + col) = xa[c];
            } else {
              uint16_t* q = side + bh * a.side_cap * D + (p & 7);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                q[((p >> 3) * D + col + 2 * e) * 8] = (uint16_t)(xa[c][e] & 0xFFFFu);
                q[((p >> 3) * D + col + 2 * e + 1) * 8] = (uint16_t)(xa[c][e] >> 16);
              }
            }
          }
          if (kind == 0 && grp == 0) a.side_idx[bh * a.side_cap + p] = (int32_t)(a.pos + tok_lane);
        }
      }
#pragma unroll
      for (int c = 0; c < D / 32; ++c) xa[c] = xn[c];
    }
  }
}

// Exclusive scan of the per-sub-tile counts of one (b, kv head); advances the counters.
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
  int64_t run = s_scan[tid] - local;   // flagged tokens before this thread's first sub-tile
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

// Persistent grid: about `target` workgroups in all, none without work.
dim3 persistent_grid(const HybridArgs& a, int target) {
  const int64_t units = (int64_t)a.hkv * a.batch;
  int64_t per_unit = (target + units - 1) / units;
  const int64_t max_per_unit = (a.n_tiles + kWavesH - 1) / kWavesH;
  if (per_unit > max_per_unit) per_unit = max_per_unit;
  if (per_unit < 1) per_unit = 1;
  return dim3((unsigned)per_unit, a.hkv, a.batch);
}

}  // namespace

hipError_t launch_hybrid_bf16(const HybridArgs& a, hipStream_t s) {
  const dim3 gs = persistent_grid(a, 256), gw = persistent_grid(a, 512);
  if (a.d == 128) hipLaunchKernelGGL(hybrid_select_kernel<128>, gs, dim3(kThreadsH), 0, s, a);
  else hipLaunchKernelGGL(hybrid_select_kernel<64>, gs, dim3(kThreadsH), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(hybrid_scan_kernel, dim3(a.hkv, a.batch), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.d == 128) hipLaunchKernelGGL(hybrid_write_kernel<128>, gw, dim3(kThreadsH), 0, s, a);
  else hipLaunchKernelGGL(hybrid_write_kernel<64>, gw, dim3(kThreadsH), 0, s, a);
  return hipGetLastError();
}

}  // namespace lrkv
