// Split-K decode attention over a low-rank KV cache (gfx950).
//
// One wave attends one split (a run of 32-token chunks) of one (batch, kv
// head) for all g query heads of that kv head, so every coefficient row is
// read from HBM once per kv head.  Per chunk:
//   scores  s = C_K q'             matrix cores, tokens as rows, heads as columns
//   softmax running max / sum per head, rescaling the accumulator
//   acc    += P C_V                matrix cores, heads as rows, value columns as columns
// q' = q B_K * scale * log2(e) is folded once per workgroup.  The value cache's
// octet layout makes each lane's 16-byte load exactly the 8 consecutive tokens
// of one column that a matrix-core operand wants, and the key tiles load their
// tokens in the order that leaves each lane's scores in the k-slots of the
// value product, so no data moves between lanes inside the loop.  bfloat16
// operands that must keep float32 accuracy (q' and the weights p) are split
// into a high and a low bfloat16 part: the two products sum to float32
// precision.  A second kernel merges the splits by log-sum-exp and lifts the
// latent accumulator through B_V^T.
#include "lrkv_device.h"
#include "lrkv_internal.h"

namespace lrkv {

namespace {

constexpr int kWaves = 4;

// ----------------------------------------------------------------------------
// bfloat16 split kernel (matrix cores)
// ----------------------------------------------------------------------------
// KC: 32-wide k chunks covering r_K;  VB: 16-wide column blocks covering r_V.
// FOLD false: keys are full-rank rows (hybrid side list), q' = q * scale.
template <int KC, int VB, bool FOLD>
__global__ __launch_bounds__(256) void split_bf16_kernel(SplitArgs a) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n16 = lane & 15;     // matrix row/column index this lane supplies
  const int grp = lane >> 4;     // k-slot group
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int split = blockIdx.x * kWaves + wave;
  const int g = a.g;
  const int rk = a.rk, rv = a.rv, d = a.d;
  const int64_t bh = (int64_t)b * a.hkv + h;

  __shared__ float s_q[8 * 128];          // q rows of this kv head's query heads
  __shared__ float s_qf[8 * 128];         // folded queries q' [g][rk]
  __shared__ float s_acc[kWaves][16][VB * 16];

  const uint16_t* q = static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.hq + (int64_t)h * g) * d;
  for (int i = tid; i < g * d; i += 256) s_q[i] = bf16_to_f32(q[i]);
  __syncthreads();
  if (FOLD) {
    const uint16_t* bk = static_cast<const uint16_t*>(a.basis_k) + (int64_t)h * d * rk;
    for (int i = tid; i < g * rk; i += 256) {
      const int j = i / rk, k = i - j * rk;
      float acc = 0.f;
      for (int e = 0; e < d; ++e) acc = fmaf(s_q[j * d + e], bf16_to_f32(bk[e * rk + k]), acc);
      s_qf[i] = acc * a.qscale;
    }
  } else {
    for (int i = tid; i < g * d; i += 256) s_qf[i] = s_q[i] * a.qscale;
  }
  __syncthreads();

  // Query operand of the score product: column n16 is head n16 (high part in
  // the first MFMA, low part in the second); columns g..2g-1 repeat the heads
  // so that lanes g..2g-1 also see full scores; other columns are zero.
  const int head = n16 < g ? n16 : (n16 < 2 * g ? n16 - g : -1);
  u32x4 bq_hi[KC], bq_lo[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = 32 * c + 8 * grp + e;
      v[e] = (head >= 0 && k < rk) ? s_qf[head * rk + k] : 0.f;
    }
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hi[e] = pack_bf16(v[2 * e], v[2 * e + 1]);
      lo[e] = pack_bf16(v[2 * e] - bf16_lo(hi[e]), v[2 * e + 1] - bf16_hi(hi[e]));
    }
    bq_hi[c] = u32x4{hi[0], hi[1], hi[2], hi[3]};
    bq_lo[c] = u32x4{lo[0], lo[1], lo[2], lo[3]};
  }

  int64_t n_end = a.n_static;
  if (a.n_dev) {
    n_end = a.n_dev[bh];
    if (n_end > a.cap) n_end = a.cap;
    if (n_end < 0) n_end = 0;
  }
  const int64_t n_chunks = (n_end + kChunk - 1) / kChunk;
  const int64_t c_begin = (int64_t)split * a.chunks_per_split;
  int64_t c_end = c_begin + a.chunks_per_split;
  if (c_end > n_chunks) c_end = n_chunks;

  const uint16_t* ck = static_cast<const uint16_t*>(a.ck) + bh * a.cap * rk;
  const uint16_t* cv = static_cast<const uint16_t*>(a.cv) + bh * a.cap * rv;

  f32x4 acc[VB];
#pragma unroll
  for (int i = 0; i < VB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  // This lane takes the high (rows < g) or low (rows g..2g-1) part of p.
  const bool take_hi = n16 < g;
  const bool p_row = n16 < 2 * g;

  for (int64_t chunk = c_begin; chunk < c_end; ++chunk) {
    const int64_t t0 = chunk * kChunk;
    // --- key tiles: tile T, row m holds token t0 + 8*(m/4) + 4*T + m%4
    u32x4 kt[2][KC];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      const int64_t tok = t0 + 8 * (n16 >> 2) + 4 * T + (n16 & 3);
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const int col = 32 * c + 8 * grp;
        kt[T][c] = (tok < n_end && col < rk)
                       ? *reinterpret_cast<const u32x4*>(ck + tok * rk + col)
                       : u32x4{0u, 0u, 0u, 0u};
      }
    }
    // --- value octets: column 16*vb + n16, tokens t0 + 8*grp .. +7
    u32x4 vt[VB];
    const int64_t oct_tok = t0 + 8 * grp;
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
      const int col = 16 * vb + n16;
      vt[vb] = (oct_tok < n_end && col < rv)
                   ? *reinterpret_cast<const u32x4*>(cv + ((oct_tok >> 3) * rv + col) * 8)
                   : u32x4{0u, 0u, 0u, 0u};
    }
    if (t0 + kChunk > n_end) {
      // tail chunk: zero value elements past the end (they may hold anything)
      const int64_t nv = n_end - oct_tok;
      if (nv < 8) {
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            uint32_t m = 0u;
            if (2 * w < nv) m |= 0x0000FFFFu;
            if (2 * w + 1 < nv) m |= 0xFFFF0000u;
            vt[vb][w] &= m;
          }
        }
      }
    }

    // --- scores
    f32x4 st[2];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        s = mfma_16x16x32(kt[T][c], bq_hi[c], s);
        s = mfma_16x16x32(kt[T][c], bq_lo[c], s);
      }
      st[T] = s;
    }
    // lane (n16, grp) now holds, for head(n16), tokens t0 + 8*grp + 4*T + i
    float sv[8];
    float cmax = -INFINITY;
#pragma unroll
    for (int T = 0; T < 2; ++T) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t tok = oct_tok + 4 * T + i;
        const float s = tok < n_end ? st[T][i] : -INFINITY;
        sv[4 * T + i] = s;
        cmax = fmaxf(cmax, s);
      }
    }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = exp2_fast(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
    uint32_t pw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = exp2_fast(sv[2 * e] - m_new);
      const float p1 = exp2_fast(sv[2 * e + 1] - m_new);
      psum += p0 + p1;
      const uint32_t hi = pack_bf16(p0, p1);
      const uint32_t lo = pack_bf16(p0 - bf16_lo(hi), p1 - bf16_hi(hi));
      pw[e] = p_row ? (take_hi ? hi : lo) : 0u;
    }
    l_run = l_run * alpha + psum;
    const u32x4 pop = u32x4{pw[0], pw[1], pw[2], pw[3]};

    // rescale the accumulator rows 4*grp + i by the alpha of their head
    float ar[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * grp + i);
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[vb][i] *= ar[i];
      acc[vb] = mfma_16x16x32(pop, vt[vb], acc[vb]);
    }
  }

  // --- epilogue: rows j (high part) + rows g + j (low part) are head j
#pragma unroll
  for (int vb = 0; vb < VB; ++vb)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_acc[wave][4 * grp + i][16 * vb + n16] = acc[vb][i];
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  __syncthreads();
  if (split < a.n_splits) {
    const int64_t row0 = ((int64_t)b * a.hq + (int64_t)h * g) * a.n_splits + split;
    for (int i = lane; i < g * rv; i += 64) {
      const int j = i / rv, c = i - j * rv;
      a.part_acc[(row0 + (int64_t)j * a.n_splits) * rv + c] = s_acc[wave][j][c] + s_acc[wave][g + j][c];
    }
    if (lane < g) {
      a.part_ml[(row0 + (int64_t)lane * a.n_splits) * 2 + 0] = m_run;
      a.part_ml[(row0 + (int64_t)lane * a.n_splits) * 2 + 1] = l_tot;
    }
  }
}

// ----------------------------------------------------------------------------
// float32 split kernel (vector ALU): 64-token tiles, one token per lane for the
// scores, one value column per lane for the accumulation.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void split_f32_kernel(SplitArgs a) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int split = blockIdx.x * kWaves + wave;
  const int g = a.g;
  const int rk = a.rk, rv = a.rv, d = a.d;
  const int64_t bh = (int64_t)b * a.hkv + h;
  const bool fold = a.basis_k != nullptr;
  const int rq = fold ? rk : d;

  __shared__ float s_q[8 * 128];
  __shared__ float s_qf[8 * 128];
  __shared__ float s_p[kWaves][8][64];

  const float* q = static_cast<const float*>(a.q) + ((int64_t)b * a.hq + (int64_t)h * g) * d;
  for (int i = tid; i < g * d; i += 256) s_q[i] = q[i];
  __syncthreads();
  if (fold) {
    const float* bk = static_cast<const float*>(a.basis_k) + (int64_t)h * d * rk;
    for (int i = tid; i < g * rk; i += 256) {
      const int j = i / rk, k = i - j * rk;
      float acc = 0.f;
      for (int e = 0; e < d; ++e) acc = fmaf(s_q[j * d + e], bk[e * rk + k], acc);
      s_qf[i] = acc * a.qscale;
    }
  } else {
    for (int i = tid; i < g * d; i += 256) s_qf[i] = s_q[i] * a.qscale;
  }
  __syncthreads();

  int64_t n_end = a.n_static;
  if (a.n_dev) {
    n_end = a.n_dev[bh];
    if (n_end > a.cap) n_end = a.cap;
    if (n_end < 0) n_end = 0;
  }
  const int64_t n_chunks = (n_end + kChunk - 1) / kChunk;
  const int64_t c_begin = (int64_t)split * a.chunks_per_split;
  int64_t c_end = c_begin + a.chunks_per_split;
  if (c_end > n_chunks) c_end = n_chunks;
  const int64_t t_begin = c_begin * kChunk;
  int64_t t_end = c_end * kChunk;
  if (t_end > n_end) t_end = n_end;

  const float* ck = static_cast<const float*>(a.ck) + bh * a.cap * rk;
  const float* cv = static_cast<const float*>(a.cv) + bh * a.cap * rv;

  float m_run[8], l_run[8], acc[8][2];
#pragma unroll
  for (int j = 0; j < 8; ++j) { m_run[j] = -INFINITY; l_run[j] = 0.f; acc[j][0] = acc[j][1] = 0.f; }

  for (int64_t t0 = t_begin; t0 < t_end; t0 += 64) {
    const int64_t tok = t0 + lane;
    const bool valid = tok < t_end;
    float s[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] = 0.f;
    if (valid) {
      const float* row = ck + tok * rk;
      for (int k = 0; k < rk; k += 4) {
        const float4 c4 = *reinterpret_cast<const float4*>(row + k);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (j < g) {
            const float* qq = s_qf + j * rq + k;
            s[j] = fmaf(c4.x, qq[0], fmaf(c4.y, qq[1], fmaf(c4.z, qq[2], fmaf(c4.w, qq[3], s[j]))));
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < g) {
        const float sj = valid ? s[j] : -INFINITY;
        const float m_new = fmaxf(m_run[j], wave_max(sj));
        const float alpha = exp2_fast(m_run[j] - m_new);
        const float p = valid ? exp2_fast(sj - m_new) : 0.f;
        l_run[j] = l_run[j] * alpha + wave_sum(p);
        m_run[j] = m_new;
        acc[j][0] *= alpha;
        acc[j][1] *= alpha;
        s_p[wave][j][lane] = p;
      }
    }
    __builtin_amdgcn_wave_barrier();
    const int nt = (int)((t_end - t0) < 64 ? (t_end - t0) : 64);
    for (int ci = 0; ci < 2; ++ci) {
      const int c = lane + 64 * ci;
      if (c < rv) {
        for (int t = 0; t < nt; ++t) {
          const int64_t tt = t0 + t;
          const float v = cv[((tt >> 3) * rv + c) * 8 + (tt & 7)];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (j < g) acc[j][ci] = fmaf(s_p[wave][j][t], v, acc[j][ci]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  if (split < a.n_splits) {
    const int64_t row0 = ((int64_t)b * a.hq + (int64_t)h * g) * a.n_splits + split;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < g) {
        for (int ci = 0; ci < 2; ++ci) {
          const int c = lane + 64 * ci;
          if (c < rv) a.part_acc[(row0 + (int64_t)j * a.n_splits) * rv + c] = acc[j][ci];
        }
        if (lane == 0) {
          a.part_ml[(row0 + (int64_t)j * a.n_splits) * 2 + 0] = m_run[j];
          a.part_ml[(row0 + (int64_t)j * a.n_splits) * 2 + 1] = l_run[j];
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// merge + lift: one workgroup per (batch, query head)
// ----------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ float load_f(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_f<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
template <>
__device__ __forceinline__ float load_f<float>(const float* p, int64_t i) { return p[i]; }

template <typename T>
__device__ __forceinline__ void store_f(T* p, int64_t i, float v);
template <>
__device__ __forceinline__ void store_f<uint16_t>(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
template <>
__device__ __forceinline__ void store_f<float>(float* p, int64_t i, float v) { p[i] = v; }

__device__ __forceinline__ float block_max_128(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = fmaxf(red[0], red[1]);
  __syncthreads();
  return v;
}

__device__ __forceinline__ float block_sum_128(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = red[0] + red[1];
  __syncthreads();
  return v;
}

template <typename T>
__global__ __launch_bounds__(128) void merge_kernel(MergeArgs a) {
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int h = hq / a.g;
  const int tid = threadIdx.x;
  const int S = a.n_splits, SS = a.n_side_splits;
  const int64_t row = (int64_t)b * a.hq + hq;

  __shared__ float s_w[kMaxSplits];
  __shared__ float s_acc[128];
  __shared__ float s_red[2];

  const float* ml = a.part_ml + row * S * 2;
  const float* sml = a.side_ml ? a.side_ml + row * SS * 2 : nullptr;
  float m = -INFINITY;
  for (int s = tid; s < S; s += 128) m = fmaxf(m, ml[2 * s]);
  for (int s = tid; s < SS; s += 128) m = fmaxf(m, sml[2 * s]);
  const float M = block_max_128(m, s_red);
  float l = 0.f;
  for (int s = tid; s < S + SS; s += 128) {
    const float ms = s < S ? ml[2 * s] : sml[2 * (s - S)];
    const float ls = s < S ? ml[2 * s + 1] : sml[2 * (s - S) + 1];
    const float w = (ms == -INFINITY) ? 0.f : exp2_fast(ms - M);
    s_w[s] = w;
    l = fmaf(w, ls, l);
  }
  const float L = block_sum_128(l, s_red);   // also orders the s_w writes
  const float inv = L > 0.f ? 1.f / L : 0.f;

  if (tid < a.rv) {
    const float* pa = a.part_acc + row * (int64_t)S * a.racc + tid;
    float acc = 0.f;
    for (int s = 0; s < S; ++s) acc = fmaf(s_w[s], pa[(int64_t)s * a.racc], acc);
    s_acc[tid] = acc * inv;
  }
  __syncthreads();
  if (tid < a.d) {
    const T* bv = static_cast<const T*>(a.basis_v) + ((int64_t)h * a.d + tid) * a.rv;
    float o = 0.f;
    for (int c = 0; c < a.rv; ++c) o = fmaf(load_f(bv, c), s_acc[c], o);
    if (SS > 0) {
      const float* sa = a.side_acc + row * (int64_t)SS * a.d + tid;
      float os = 0.f;
      for (int s = 0; s < SS; ++s) os = fmaf(s_w[S + s], sa[(int64_t)s * a.d], os);
      o = fmaf(os, inv, o);
    }
    store_f(static_cast<T*>(a.out), row * a.d + tid, o);
  }
  if (tid == 0 && a.lse) a.lse[row] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

}  // namespace

#define LRKV_SPLIT_CASE(KC, VB)                                                          \
  case (KC * 16 + VB):                                                                   \
    hipLaunchKernelGGL((split_bf16_kernel<KC, VB, true>), grid, dim3(256), 0, s, a);     \
    break;

hipError_t launch_split_bf16(const SplitArgs& a, hipStream_t s) {
  const dim3 grid((a.n_splits + kWaves - 1) / kWaves, a.hkv, a.batch);
  const int kc = (a.rk + 31) / 32, vb = (a.rv + 15) / 16;
  if (a.basis_k == nullptr) {
    if (a.d == 128) hipLaunchKernelGGL((split_bf16_kernel<4, 8, false>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((split_bf16_kernel<2, 4, false>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  switch (kc * 16 + vb) {
    LRKV_SPLIT_CASE(1, 1) LRKV_SPLIT_CASE(1, 2) LRKV_SPLIT_CASE(1, 3) LRKV_SPLIT_CASE(1, 4)
    LRKV_SPLIT_CASE(1, 5) LRKV_SPLIT_CASE(1, 6) LRKV_SPLIT_CASE(1, 7) LRKV_SPLIT_CASE(1, 8)
    LRKV_SPLIT_CASE(2, 1) LRKV_SPLIT_CASE(2, 2) LRKV_SPLIT_CASE(2, 3) LRKV_SPLIT_CASE(2, 4)
    LRKV_SPLIT_CASE(2, 5) LRKV_SPLIT_CASE(2, 6) LRKV_SPLIT_CASE(2, 7) LRKV_SPLIT_CASE(2, 8)
    LRKV_SPLIT_CASE(3, 1) LRKV_SPLIT_CASE(3, 2) LRKV_SPLIT_CASE(3, 3) LRKV_SPLIT_CASE(3, 4)
    LRKV_SPLIT_CASE(3, 5) LRKV_SPLIT_CASE(3, 6) LRKV_SPLIT_CASE(3, 7) LRKV_SPLIT_CASE(3, 8)
    LRKV_SPLIT_CASE(4, 1) LRKV_SPLIT_CASE(4, 2) LRKV_SPLIT_CASE(4, 3) LRKV_SPLIT_CASE(4, 4)
    LRKV_SPLIT_CASE(4, 5) LRKV_SPLIT_CASE(4, 6) LRKV_SPLIT_CASE(4, 7) LRKV_SPLIT_CASE(4, 8)
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_split_f32(const SplitArgs& a, hipStream_t s) {
  const dim3 grid((a.n_splits + kWaves - 1) / kWaves, a.hkv, a.batch);
  hipLaunchKernelGGL(split_f32_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, bool bf16, hipStream_t s) {
  const dim3 grid(a.hq, a.batch);
  if (bf16) hipLaunchKernelGGL(merge_kernel<uint16_t>, grid, dim3(128), 0, s, a);
  else hipLaunchKernelGGL(merge_kernel<float>, grid, dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace lrkv
