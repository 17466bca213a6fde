// Hybrid compress: tokens whose key or value is poorly reconstructed from
// its stored low-rank coefficients stay full rank in a side list; the others
// are appended to the low-rank caches (gfx950).
//
// Three launches, all deterministic (no order-dependent atomics):
//   select  c = x B and x_hat = round(c) B^T on the matrix cores, then
//           ||x - x_hat||^2 > tau^2 ||x||^2 in float32, for K and for V; a token
//           is flagged when either is.  Per 16-token sub-tile: flags and count.
//           The squared residual is evaluated as ||x||^2 - 2 <c, round(c)> +
//           ||x_hat||^2 (equal to it in exact arithmetic, since <x, x_hat> =
//           <x B, round(c)>), which keeps every operand in registers.
//   scan    per (b, kv head): exclusive prefix of the sub-tile counts gives every
//           sub-tile's first low-rank row and first side-list row; the counters
//           advance (clamped at the capacities, with an overflow flag).
//   write   recompute c; each token goes to its sub-tile's offset plus its rank
//           among the sub-tile's tokens of the same kind (a wave ballot).
// Select and write are persistent: a workgroup stages the bases in LDS once
// (sized to the ranks) and each of its waves walks a contiguous run of
// 16-token sub-tiles of one (b, kv head), loading the next two sub-tiles' key
// and value rows (and, in write, their flags and offsets) while it works on
// the current one.  Contiguous runs keep the partial writes of a value octet or a
// flag line that straddles two sub-tiles inside one L2.
#include <type_traits>

#include "lrkv_device.h"
#include "lrkv_internal.h"

namespace lrkv {

namespace {

constexpr int kWavesH = 4;                 // waves per hybrid workgroup
constexpr int kThreadsH = 64 * kWavesH;

// LDS layout of one workgroup, in bfloat16 elements: both bases transposed
// ([coefficient][dim], 16 NB rows each, unpadded in the swizzled layout of
// lds_swz, read 16 bytes per lane from 16 consecutive rows without bank
// conflicts) and, for select, as stored ([dim][coefficient], 32 ceil(NB/2)
// columns each, read 8 bytes per lane, pitch of 2 x odd dwords); rows and
// columns past a rank are zero.  Without row padding the bases and the write
// kernel's rings of two workgroups fit one compute unit's LDS.
struct HybridLds {
  int rows, cols_n, pitch_n;
  int off_t[2], off_n[2];
  int elems_t, elems_select;
};

__host__ __device__ inline HybridLds hybrid_lds(int d, int nb) {
  HybridLds L;
  L.rows = 16 * nb;
  L.cols_n = 32 * ((nb + 1) / 2);
  L.pitch_n = L.cols_n + 4;
  L.off_t[0] = 0;
  L.off_t[1] = L.rows * d;
  L.elems_t = 2 * L.rows * d;
  L.off_n[0] = L.elems_t;
  L.off_n[1] = L.elems_t + d * L.pitch_n;
  L.elems_select = L.elems_t + 2 * d * L.pitch_n;
  return L;
}

template <int D>
__device__ void stage_transposed(const HybridArgs& a, const HybridLds& L, int h, uint16_t* smem) {
  const int tid = threadIdx.x;
  for (int kind = 0; kind < 2; ++kind) {
    const int r = kind ? a.rv : a.rk;
    const uint16_t* bs = static_cast<const uint16_t*>(kind ? a.bv : a.bk) + (int64_t)h * D * r;
    uint16_t* st = smem + L.off_t[kind];
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
            st[lds_swz<D>(c + 2 * e, dd)] = (uint16_t)(w[u][e] & 0xFFFFu);
            st[lds_swz<D>(c + 2 * e + 1, dd)] = (uint16_t)(w[u][e] >> 16);
          }
        }
      }
    }
    for (int i = tid; i < (L.rows - r) * D; i += kThreadsH) st[lds_swz<D>(r + i / D, i % D)] = 0;
  }
}

template <int D>
__device__ void stage_natural(const HybridArgs& a, const HybridLds& L, int h, uint16_t* smem) {
  const int tid = threadIdx.x;
  for (int kind = 0; kind < 2; ++kind) {
    const int r = kind ? a.rv : a.rk;
    const uint16_t* bs = static_cast<const uint16_t*>(kind ? a.bv : a.bk) + (int64_t)h * D * r;
    uint16_t* sn = smem + L.off_n[kind];
    const int pieces = L.cols_n / 8;   // 8-coefficient pieces per row
    for (int i = tid; i < D * pieces; i += kThreadsH) {
      const int row = i / pieces, c = (i % pieces) * 8;
      const u32x4 w = c < r ? *reinterpret_cast<const u32x4*>(bs + row * r + c) : u32x4{0u, 0u, 0u, 0u};
      uint32_t* dst = reinterpret_cast<uint32_t*>(sn + row * L.pitch_n + c);   // 8-byte aligned
      *reinterpret_cast<uint2*>(dst) = uint2{w[0], w[1]};
      *reinterpret_cast<uint2*>(dst + 2) = uint2{w[2], w[3]};
    }
  }
}

// Rows of one 16-token sub-tile as matrix-core operands: lane (n16, grp)
// holds token n16's elements 32c + 8 grp .. +7.  Tokens past the end, and
// every lane when `live` is false, read zero (buffer range), so the number
// of loads never depends on the data.
template <int D>
__device__ __forceinline__ void load_rows(const HybridArgs& a, int b, int h, int kind, int64_t sub, bool live,
                                          int n16, int grp, u32x4 (&xa)[D / 32]) {
  const int64_t t0 = sub * kHybridTile;
  const int64_t left = a.n_tokens - t0;
  const int nt = left < kHybridTile ? (int)left : kHybridTile;
  const uint16_t* x = static_cast<const uint16_t*>(kind ? a.v : a.k) + ((b * a.n_tokens + t0) * a.hkv + h) * D;
  const uint32_t bytes = live && nt > 0 ? (uint32_t)(((nt - 1) * a.hkv + 1) * D * 2) : 0u;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(x, bytes);
  const uint32_t voff = (uint32_t)((n16 * a.hkv * D + 8 * grp) * 2);
#pragma unroll
  for (int c = 0; c < D / 32; ++c) xa[c] = buf_load16(rs, voff + 64 * c);
}

// This lane's element offsets of its transposed-basis operands (row
// 16 nb + n16, dims 32 c + 8 grp .. + 7), computed once per kernel.  The
// swizzle of a row depends on the row's line modulo 16 only, so blocks nb and
// nb + P (P = 1 for 128-element rows, 2 for 64-element rows, whose 16-row
// block fills 8 lines) differ by a constant, which the loop adds as an
// immediate to one of P x D/32 live addresses.
template <int D, int NB>
struct BasisOffsets {
  static constexpr int P = D == 64 ? 2 : 1;
  static constexpr int kStep = P * 16 * D;
  int o[P][D / 32];
  __device__ __forceinline__ BasisOffsets(int n16, int grp) {
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int c = 0; c < D / 32; ++c) o[p][c] = lds_swz<D>(16 * p + n16, 32 * c + 8 * grp);
  }
  __device__ __forceinline__ int at(int nb, int c) const { return o[nb % P][c] + (nb / P) * kStep; }
};

// c^T = B^T x^T for the sub-tile (transposed basis as the row operand, the
// token rows as loaded as the column operand): acc[nb] lane (n16, grp)
// register i is coefficient 16 nb + 4 grp + i of token n16.
template <int D, int NB>
__device__ __forceinline__ void coeffs_t(const u32x4 (&xa)[D / 32], const uint16_t* bt, const BasisOffsets<D, NB>& bo,
                                         f32x4 (&acc)[NB]) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      acc[nb] = mfma_16x16x32(*reinterpret_cast<const u32x4*>(bt + bo.at(nb, c)), xa[c], acc[nb]);
  }
}

// Two waves per SIMD: the LDS of two workgroups (both bases twice) fills a compute unit.
template <int D, int NB>
__global__ __launch_bounds__(kThreadsH) __attribute__((amdgpu_waves_per_eu(2, 2)))
void hybrid_select_kernel(HybridArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int n16 = lane & 15, grp = lane >> 4;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * a.hkv + h;
  const int64_t n_slots = (int64_t)a.n_tiles * kHybridTile;
  const HybridLds L = hybrid_lds(D, NB);
  constexpr int KK = (NB + 1) / 2;

  stage_transposed<D>(a, L, h, smem);
  stage_natural<D>(a, L, h, smem);
  __syncthreads();
  const BasisOffsets<D, NB> bo(n16, grp);

  const int64_t n_waves = (int64_t)gridDim.x * kWavesH;
  const int64_t per_wave = (a.n_tiles + n_waves - 1) / n_waves;
  int64_t sub = ((int64_t)blockIdx.x * kWavesH + wave) * per_wave;
  const int64_t sub_end = sub + per_wave < a.n_tiles ? sub + per_wave : a.n_tiles;
  const __amdgpu_buffer_rsrc_t rs_wsf = make_rsrc(a.ws_flags + bh * n_slots, (uint32_t)n_slots);
  const __amdgpu_buffer_rsrc_t rs_flags =
      make_rsrc(a.flags ? a.flags + bh * a.n_tokens : a.ws_flags, a.flags ? (uint32_t)a.n_tokens : 0u);
  const __amdgpu_buffer_rsrc_t rs_cnt = make_rsrc(a.ws_counts + bh * a.n_tiles, (uint32_t)(a.n_tiles * 4));

  // ||x - x_hat||^2 > tau^2 ||x||^2 for token n16 of two sub-tiles, one kind.
  // The two sub-tiles share every basis operand read from LDS (the basis is
  // the row operand of both products), so each read feeds two matrix-core
  // operations and the two dependency chains interleave.
  auto flagged2 = [&](const u32x4 (&xa)[2][D / 32], int kind, bool (&fl)[2]) {
    const uint16_t* bt = smem + L.off_t[kind];
    f32x4 acc1[2][NB];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc1[t][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const u32x4 bop = *reinterpret_cast<const u32x4*>(bt + bo.at(nb, c));
        acc1[0][nb] = mfma_16x16x32(bop, xa[0][c], acc1[0][nb]);
        acc1[1][nb] = mfma_16x16x32(bop, xa[1][c], acc1[1][nb]);
      }
    }
    // stored coefficients round(c), packed as the column operand of x_hat^T = B round(c)^T:
    // k-slots 0..3 of block kk are coefficients 32 kk + 4 grp + 0..3, slots 4..7 are 32 kk + 16 + 4 grp + 0..3
    float cc[2] = {0.f, 0.f};
    uint32_t cw[2][2 * KK][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int nb = 0; nb < 2 * KK; ++nb) {
        uint16_t tb[4] = {0, 0, 0, 0};
        if (nb < NB) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            tb[i] = f32_to_bf16(acc1[t][nb < NB ? nb : 0][i]);
            cc[t] = fmaf(acc1[t][nb < NB ? nb : 0][i], bf16_to_f32(tb[i]), cc[t]);
          }
        }
        cw[t][nb][0] = (uint32_t)tb[0] | ((uint32_t)tb[1] << 16);
        cw[t][nb][1] = (uint32_t)tb[2] | ((uint32_t)tb[3] << 16);
      }
    __builtin_amdgcn_sched_barrier(0);
    const uint16_t* bn = smem + L.off_n[kind];
    float xh2[2] = {0.f, 0.f};
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      f32x4 acc2[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const uint16_t* row = bn + (16 * db + n16) * L.pitch_n + 32 * kk + 4 * grp;
        const uint2 lo = *reinterpret_cast<const uint2*>(row);
        const uint2 hi = *reinterpret_cast<const uint2*>(row + 16);
        const u32x4 aop = u32x4{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc2[t] = mfma_16x16x32(
              aop, u32x4{cw[t][2 * kk][0], cw[t][2 * kk][1], cw[t][2 * kk + 1][0], cw[t][2 * kk + 1][1]}, acc2[t]);
      }
      // lane (n16, grp) register i: x_hat of token n16 at dim 16 db + 4 grp + i
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) xh2[t] = fmaf(acc2[t][i], acc2[t][i], xh2[t]);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float n2 = 0.f;
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = bf16_lo(xa[t][c][e]), hi = bf16_hi(xa[t][c][e]);
          n2 = fmaf(lo, lo, n2);
          n2 = fmaf(hi, hi, n2);
        }
      float ct = cc[t], xt = xh2[t];
#pragma unroll
      for (int o = 16; o < 64; o <<= 1) {
        ct += __shfl_xor(ct, o);
        xt += __shfl_xor(xt, o);
        n2 += __shfl_xor(n2, o);
      }
      const float e2 = n2 - 2.f * ct + xt;
      fl[t] = e2 > a.tau2 * n2;
    }
  };

  // keys and values of two pairs of consecutive sub-tiles: one pair streams
  // in while the other is tested.  The buffers rotate statically (the loop is
  // unrolled by two pairs), so no register copy waits for a load in flight; a
  // sub-tile past the wave's run reads zero and writes nothing.
  struct Rows2 {
    u32x4 k[2][D / 32], v[2][D / 32];
  };
  auto fetch2 = [&](Rows2& r, int64_t s) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bool live = s + t < sub_end;
      load_rows<D>(a, b, h, 0, live ? s + t : sub, live, n16, grp, r.k[t]);
      load_rows<D>(a, b, h, 1, live ? s + t : sub, live, n16, grp, r.v[t]);
    }
  };
  auto test2 = [&](const Rows2& r, int64_t s) {
    __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead and the two kinds apart
    bool fk[2], fv[2];
    flagged2(r.k, 0, fk);
    __builtin_amdgcn_sched_barrier(0);
    flagged2(r.v, 1, fv);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t st = s + t;
      const bool live = st < sub_end;
      const int64_t tok = st * kHybridTile + n16;
      const bool f = (fk[t] || fv[t]) && tok < a.n_tokens;
      const uint32_t slot = grp == 0 && live ? (uint32_t)tok : kOob;
      buf_store1(rs_wsf, slot, (uint8_t)f);
      buf_store1(rs_flags, slot, (uint8_t)f);
      const int count = __popcll(__ballot(grp == 0 && f));
      buf_store4(rs_cnt, lane == 0 && live ? (uint32_t)(st * 4) : kOob, (uint32_t)count);
    }
  };
  // The pairs of the run are taken last to first: the write kernel walks the
  // run first to last, so the rows it reads first are the ones read here
  // last, still in the last-level cache.  A pair index below zero reads
  // nothing (sub_end is past the run).
  const int64_t n_pairs = sub < sub_end ? (sub_end - sub + 1) / 2 : 0;
  auto pair_at = [&](int64_t j) { return j >= 0 ? sub + 2 * j : sub_end; };
  Rows2 ra, rb;
  if (n_pairs > 0) fetch2(ra, pair_at(n_pairs - 1));
  for (int64_t j = n_pairs - 1; j >= 0; j -= 2) {
    fetch2(rb, pair_at(j - 1));
    test2(ra, pair_at(j));
    if (j - 1 < 0) break;
    fetch2(ra, pair_at(j - 2));
    test2(rb, pair_at(j - 1));
  }
}

// Per-wave LDS rings of the write kernel: value octet rows (8 consecutive
// cache rows x all columns) being assembled, for the low-rank cache and for
// the side list.  Slots 0..2 hold rows o % 3 (at most three rows are open at
// once, since a sub-tile adds at most 16 rows); slot 3 holds the wave's first
// row when the wave's run starts inside it (that row is shared with the
// previous wave and is written slot by slot at the end).
template <int D, int NB>
struct WriteRings {
  static constexpr int kLrRow = 16 * NB * 8;       // elements per ring row
  static constexpr int kSideRow = D * 8;
  static constexpr int kPerWave = 4 * kLrRow + 4 * kSideRow;
};

template <int D, int NB>
size_t write_lds_bytes(const HybridLds& L) {
  return 2 * ((size_t)L.elems_t + (size_t)kWavesH * WriteRings<D, NB>::kPerWave);
}

// Octet row o of a ring: flush its columns col0 + 64 j with 16-byte stores
// (offset kOob when the row is not to be written).
template <int COLS>
__device__ __forceinline__ void flush_row(__amdgpu_buffer_rsrc_t rs, const uint16_t* ring_row, int64_t o, bool ok,
                                          int cols, int lane) {
#pragma unroll
  for (int j = 0; j < (COLS + 63) / 64; ++j) {
    const int col = lane + 64 * j;
    const int cc = col < COLS ? col : 0;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ring_row + cc * 8);
    buf_store16(rs, ok && col < cols ? (uint32_t)((o * cols + col) * 16) : kOob, v);
  }
}

// Slots [s0, s1) of octet row o, 2 bytes at a time (rows shared with another wave).
template <int COLS>
__device__ void flush_row_part(__amdgpu_buffer_rsrc_t rs, const uint16_t* ring_row, int64_t o, int s0, int s1,
                               int cols, int lane) {
  for (int j = 0; j < (COLS + 63) / 64; ++j) {
    const int col = lane + 64 * j;
    if (col >= cols) continue;
    for (int sl = s0; sl < s1; ++sl)
      buf_store2(rs, (uint32_t)(((o * cols + col) * 8 + sl) * 2), ring_row[col * 8 + sl]);
  }
}

// Two waves per SIMD: the bases and the rings of two workgroups fill a compute
// unit's LDS (exactly, at head_dim 128 and ranks up to 64: 80 KB each).
template <int D, int NB>
__global__ __launch_bounds__(kThreadsH) __attribute__((amdgpu_waves_per_eu(2, 2)))
void hybrid_write_kernel(HybridArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  using R = WriteRings<D, NB>;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int n16 = lane & 15, grp = lane >> 4;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * a.hkv + h;
  const int64_t n_slots = (int64_t)a.n_tiles * kHybridTile;
  const HybridLds L = hybrid_lds(D, NB);
  const int rk = a.rk, rv = a.rv;
  uint16_t* ring_lr = smem + L.elems_t + wave * R::kPerWave;
  uint16_t* ring_side = ring_lr + 4 * R::kLrRow;

  stage_transposed<D>(a, L, h, smem);
  __syncthreads();
  const BasisOffsets<D, NB> bo(n16, grp);

  const int64_t n_waves = (int64_t)gridDim.x * kWavesH;
  const int64_t per_wave = (a.n_tiles + n_waves - 1) / n_waves;
  const int64_t sub_begin = ((int64_t)blockIdx.x * kWavesH + wave) * per_wave;
  const int64_t sub_end = sub_begin + per_wave < a.n_tiles ? sub_begin + per_wave : a.n_tiles;
  if (sub_begin >= sub_end) return;   // no barrier follows
  const __amdgpu_buffer_rsrc_t rs_wsf = make_rsrc(a.ws_flags + bh * n_slots, (uint32_t)n_slots);
  const __amdgpu_buffer_rsrc_t rs_off = make_rsrc(a.ws_offsets + bh * a.n_tiles * 2, (uint32_t)(a.n_tiles * 8));
  const __amdgpu_buffer_rsrc_t rs_ck =
      make_rsrc(static_cast<uint16_t*>(a.ck) + bh * a.cap * rk, (uint32_t)(a.cap * rk * 2));
  const __amdgpu_buffer_rsrc_t rs_cv =
      make_rsrc(static_cast<uint16_t*>(a.cv) + bh * a.cap * rv, (uint32_t)(a.cap * rv * 2));
  const __amdgpu_buffer_rsrc_t rs_ks =
      make_rsrc(static_cast<uint16_t*>(a.k_side) + bh * a.side_cap * D, (uint32_t)(a.side_cap * D * 2));
  const __amdgpu_buffer_rsrc_t rs_vs =
      make_rsrc(static_cast<uint16_t*>(a.v_side) + bh * a.side_cap * D, (uint32_t)(a.side_cap * D * 2));
  const __amdgpu_buffer_rsrc_t rs_idx = make_rsrc(a.side_idx + bh * a.side_cap, (uint32_t)(a.side_cap * 4));

  // keys, values, token n16's flag and the sub-tile's (low-rank row, side row)
  // of three consecutive sub-tiles: two stream in while one is written (a
  // static rotation, as in the select kernel)
  struct Rows {
    u32x4 k[D / 32], v[D / 32];
    uint32_t fl;
    u32x2 off;
  };
  auto fetch = [&](Rows& r, int64_t s) {
    const bool live = s < sub_end;
    load_rows<D>(a, b, h, 0, live ? s : sub_begin, live, n16, grp, r.k);
    load_rows<D>(a, b, h, 1, live ? s : sub_begin, live, n16, grp, r.v);
    r.fl = buf_load1(rs_wsf, live ? (uint32_t)(s * kHybridTile + n16) : kOob);
    r.off = buf_load8(rs_off, live ? (uint32_t)(s * 8) : kOob);
  };
  Rows r0, r1, r2;
  fetch(r0, sub_begin);
  fetch(r1, sub_begin + 1);

  // the run's first rows; when they start inside an octet row, that row is shared
  const int64_t p0_lr = (int32_t)r0.off[0], p0_side = (int32_t)r0.off[1];
  const int64_t first_lr = (p0_lr & 7) ? (p0_lr >> 3) : -1;
  const int64_t first_side = (p0_side & 7) ? (p0_side >> 3) : -1;
  auto lr_row = [&](int64_t o) { return ring_lr + (o == first_lr ? 3 : (int)(o % 3)) * R::kLrRow; };
  auto side_row = [&](int64_t o) { return ring_side + (o == first_side ? 3 : (int)(o % 3)) * R::kSideRow; };
  int64_t lr_end = p0_lr, side_end = p0_side;

  auto place = [&](const Rows& r, int64_t sub) {
    __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the phases below
    const int64_t tok = sub * kHybridTile + n16;
    const int64_t left = a.n_tokens - sub * kHybridTile;
    const int nt = left < kHybridTile ? (int)left : kHybridTile;
    const bool f_lane = r.fl != 0u;
    const uint32_t side_mask = (uint32_t)(__ballot(grp == 0 && f_lane) & 0xFFFFu);
    const uint32_t below = side_mask & ((1u << n16) - 1u);
    const int64_t lr_off = (int32_t)r.off[0], side_off = (int32_t)r.off[1];
    const int64_t p_lr = lr_off + n16 - __popc(below);
    const int64_t p_side = side_off + __popc(below);
    const bool lr_ok = n16 < nt && !f_lane && p_lr < a.cap;
    const bool side_ok = f_lane && p_side < a.side_cap;
    const int n_side_sub = __popc(side_mask);
    const int64_t lr_next = lr_off + nt - n_side_sub, side_next = side_off + n_side_sub;

    f32x4 acc[NB];
    // keys: coefficients 16 nb + 4 grp + 0..3 of token n16, one 8-byte store per block
    coeffs_t(r.k, smem + L.off_t[0], bo, acc);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = 16 * nb + 4 * grp;
      const uint32_t voff = lr_ok && col < rk ? (uint32_t)((p_lr * rk + col) * 2) : kOob;
      buf_store8(rs_ck, voff, u32x2{pack_bf16(acc[nb][0], acc[nb][1]), pack_bf16(acc[nb][2], acc[nb][3])});
    }
    __builtin_amdgcn_sched_barrier(0);
    // values: into the octet rows being assembled
    coeffs_t(r.v, smem + L.off_t[1], bo, acc);
    if (lr_ok) {
      uint16_t* rr = lr_row(p_lr >> 3) + (p_lr & 7);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int col = 16 * nb + 4 * grp + i;
          if (col < rv) rr[col * 8] = f32_to_bf16(acc[nb][i]);
        }
    }
    // selected tokens: value elements into the side list's octet rows
    if (side_mask) {
      if (side_ok) {
        uint16_t* rr = side_row(p_side >> 3) + (p_side & 7);
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            rr[(32 * c + 8 * grp + e) * 8] = (uint16_t)(e & 1 ? r.v[c][e >> 1] >> 16 : r.v[c][e >> 1] & 0xFFFFu);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    __builtin_amdgcn_sched_barrier(0);
    // rows completed by this sub-tile (at most two of each list), whole rows only
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int64_t o = (lr_off >> 3) + k;
      flush_row<16 * NB>(rs_cv, lr_row(o), o, o < (lr_next >> 3) && o != first_lr, rv, lane);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int64_t o = (side_off >> 3) + k;
      flush_row<D>(rs_vs, side_row(o), o, o < (side_next >> 3) && o != first_side, D, lane);
    }
    // selected tokens: key rows (bit for bit) and indices
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
      buf_store16(rs_ks, side_ok ? (uint32_t)((p_side * D + 32 * c + 8 * grp) * 2) : kOob, r.k[c]);
    buf_store4(rs_idx, side_ok && grp == 0 ? (uint32_t)(p_side * 4) : kOob, (uint32_t)(a.pos + tok));
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");   // ring reads before the next sub-tile's writes
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    lr_end = lr_next;
    side_end = side_next;
  };

  for (int64_t s3 = sub_begin; s3 < sub_end; s3 += 3) {
    fetch(r2, s3 + 2);
    place(r0, s3);
    if (s3 + 1 >= sub_end) break;
    fetch(r0, s3 + 3);
    place(r1, s3 + 1);
    if (s3 + 2 >= sub_end) break;
    fetch(r1, s3 + 4);
    place(r2, s3 + 2);
  }

  // the run's shared rows: its first row (when it started inside one) and its
  // last, unfinished row, written slot by slot
  auto finish = [&](const uint16_t* first_ring, int64_t first, int64_t p0, int64_t end, __amdgpu_buffer_rsrc_t rs,
                    int cols, auto row_of, auto cols_tag) {
    constexpr int COLS = decltype(cols_tag)::value;
    if (first >= 0) {
      const int64_t stop = end < 8 * (first + 1) ? end : 8 * (first + 1);
      if (stop > p0) flush_row_part<COLS>(rs, first_ring, first, (int)(p0 & 7), (int)(stop - 8 * first), cols, lane);
    }
    const int64_t last = end >> 3;
    if ((end & 7) && last != first) flush_row_part<COLS>(rs, row_of(last), last, 0, (int)(end & 7), cols, lane);
  };
  const int64_t lr_stop = lr_end < a.cap ? lr_end : a.cap;
  const int64_t side_stop = side_end < a.side_cap ? side_end : a.side_cap;
  finish(ring_lr + 3 * R::kLrRow, first_lr, p0_lr, lr_stop, rs_cv, rv, lr_row,
         std::integral_constant<int, 16 * NB>{});
  finish(ring_side + 3 * R::kSideRow, first_side, p0_side, side_stop, rs_vs, D, side_row,
         std::integral_constant<int, D>{});
}

// Exclusive scan of the per-sub-tile counts of one (b, kv head); advances the
// counters.  Rounds of 8192 counts: lane l of wave w holds the 32 consecutive
// counts [w * 2048 + 32 l, + 32) of the round in registers (all loads in
// flight at once), takes their running sum, and one scan over the lanes and
// one over the four wave totals give each lane its base; the lane then writes
// its 32 (low-rank row, side row) pairs.  Counts past n_tiles read zero and
// their offsets are dropped (buffer bounds).
__global__ __launch_bounds__(256) void hybrid_scan_kernel(HybridArgs a) {
  constexpr int kPer = 32;                       // counts per lane per round
  constexpr int kWaveSpan = 64 * kPer;
  constexpr int kRound = kWavesH * kWaveSpan;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int64_t bh = (int64_t)blockIdx.y * a.hkv + blockIdx.x;
  const int n = a.n_tiles;
  const __amdgpu_buffer_rsrc_t rs_cnt = make_rsrc(a.ws_counts + bh * n, (uint32_t)n * 4u);
  const __amdgpu_buffer_rsrc_t rs_off = make_rsrc(a.ws_offsets + bh * n * 2, (uint32_t)n * 8u);
  const int64_t lr_base = a.n_lr[bh];
  const int64_t side_base = a.n_side[bh];
  __shared__ int32_t s_tot[kWavesH];

  int64_t carry = 0;                             // flagged tokens before this round
  for (int r0 = 0; r0 < n; r0 += kRound) {
    const int j0 = r0 + wave * kWaveSpan + kPer * lane;   // this lane's first sub-tile
    uint32_t c[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) c[k] = buf_load4(rs_cnt, (uint32_t)(j0 + k) * 4u);
    int32_t lane_sum = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) lane_sum += (int32_t)c[k];
    int32_t incl = lane_sum;                     // inclusive scan over the lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) s_tot[wave] = incl;
    __syncthreads();
    int64_t base = carry + (incl - lane_sum), round_total = 0;
#pragma unroll
    for (int w = 0; w < kWavesH; ++w) {
      if (w < wave) base += s_tot[w];
      round_total += s_tot[w];
    }
    __syncthreads();                             // s_tot is rewritten next round
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int64_t j = j0 + k;                  // base = flagged tokens before sub-tile j
      buf_store8(rs_off, (uint32_t)j * 8u,
                 u32x2{(uint32_t)(int32_t)(lr_base + j * kHybridTile - base), (uint32_t)(int32_t)(side_base + base)});
      base += (int32_t)c[k];
    }
    carry += round_total;
  }
  if (tid == 0) {
    const int64_t flagged = carry;
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

// Persistent grid: one round of resident workgroups, none without work.
template <typename K>
hipError_t launch_persistent(K kernel, const HybridArgs& a, size_t lds_bytes, hipStream_t s) {
  const void* fn = reinterpret_cast<const void*>(kernel);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreadsH, lds_bytes);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  const int64_t units = (int64_t)a.hkv * a.batch;
  const int64_t target = (int64_t)(a.cus > 0 ? a.cus : 256) * per_cu;
  int64_t per_unit = (target + units - 1) / units;
  const int64_t max_per_unit = (a.n_tiles + kWavesH - 1) / kWavesH;
  if (per_unit > max_per_unit) per_unit = max_per_unit;
  if (per_unit < 1) per_unit = 1;
  hipLaunchKernelGGL(kernel, dim3((unsigned)per_unit, a.hkv, a.batch), dim3(kThreadsH), lds_bytes, s, a);
  return hipGetLastError();
}

template <int D, int NB>
hipError_t launch_hybrid_nb(const HybridArgs& a, hipStream_t s) {
  hipError_t e = launch_persistent(hybrid_select_kernel<D, NB>, a, 2 * (size_t)hybrid_lds(D, NB).elems_select, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(hybrid_scan_kernel, dim3(a.hkv, a.batch), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_persistent(hybrid_write_kernel<D, NB>, a, write_lds_bytes<D, NB>(hybrid_lds(D, NB)), s);
}

}  // namespace

hipError_t launch_hybrid_bf16(const HybridArgs& a, hipStream_t s) {
  const int nb = ((a.rk > a.rv ? a.rk : a.rv) + 15) / 16;
  if (a.d == 64) {
    switch (nb) {
      case 1: return launch_hybrid_nb<64, 1>(a, s);
      case 2: return launch_hybrid_nb<64, 2>(a, s);
      case 3: return launch_hybrid_nb<64, 3>(a, s);
      case 4: return launch_hybrid_nb<64, 4>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (a.d != 128) return hipErrorInvalidValue;
  switch (nb) {
    case 1: return launch_hybrid_nb<128, 1>(a, s);
    case 2: return launch_hybrid_nb<128, 2>(a, s);
    case 3: return launch_hybrid_nb<128, 3>(a, s);
    case 4: return launch_hybrid_nb<128, 4>(a, s);
    case 5: return launch_hybrid_nb<128, 5>(a, s);
    case 6: return launch_hybrid_nb<128, 6>(a, s);
    case 7: return launch_hybrid_nb<128, 7>(a, s);
    case 8: return launch_hybrid_nb<128, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lrkv
