// Launchers of the split-K decode attention over a low-rank KV cache
// (gfx950): the latent-query, hybrid-cache and float32 attention kernels and
// the merge kernel.  The low-rank attention kernel of the plain and step
// calls is instantiated in decode_split.hip.
#include "decode_body.h"

namespace lrkv {

namespace {

// Latent queries and outputs (projections that absorb the bases): no fold,
// no lift; q is [B, Hq, r_K] and each partial is r_V wide.
template <int KC, int VB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void split_bf16_latent_kernel(SplitArgs a) {
  __shared__ SplitSmem sm;
  split_bf16_body<KC, VB, false, kStages<KC, VB>, false, true>(a, blockIdx.x, blockIdx.x, sm);
}

// Hybrid cache in one launch: the gridDim.x workgroups of each (b, kv head)
// are divided between the low-rank rows and the full-rank side list (r = d,
// no fold and no lift, single-buffered so that both fit two waves per SIMD)
// in proportion to the bytes each list holds, from the counts on the device;
// within a list, the workgroups take runs of chunks that differ by at most
// one chunk (the stream is shared fairly between compute units, so the
// workgroup with the most bytes ends last), which their four waves take in
// turn.  Every workgroup writes partial blockIdx.x.
// With lr.merge_cnt the last workgroup of each (b, kv head) merges the
// partials in this launch (merge_in_launch), so that no second launch is
// needed.
template <int KC, int VB, int SKC, int SVB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void split_bf16_hybrid_kernel(SplitArgs lr, SplitArgs side) {
  __shared__ SplitSmem sm;
  const int64_t bh = (int64_t)blockIdx.z * lr.hkv + blockIdx.y;
  // the two lists' lengths, read once as scalars and handed to the body as
  // static lengths (the body reads no count of its own); a cache holds fewer
  // than 2^31 tokens, so 32-bit arithmetic suffices for the division
  // Every argument either list reads is loaded here, before the counts are
  // waited for (left alone, the compiler sinks each argument load into the
  // branch that first uses it, and the prologue waits for one round trip
  // after another).
  asm volatile("" ::"s"(lr.q), "s"(lr.basis_k), "s"(lr.ck), "s"(lr.cv), "s"(lr.basis_v), "s"(lr.part_o),
               "s"(lr.part_ml), "s"(side.ck), "s"(side.cv), "s"(lr.cap), "s"(side.cap));
  asm volatile("" ::"s"(lr.rk), "s"(lr.rv), "s"(lr.d), "s"(lr.g), "s"(lr.hq), "s"(lr.n_parts), "s"(lr.qscale));
  // (both counts' loads issued before either is used: one round trip)
  const int32_t* cnt_lr = lr.n_dev;
  const int32_t* cnt_side = side.n_dev;
  const int raw_lr = __builtin_amdgcn_readfirstlane(cnt_lr[bh]);
  const int raw_side = __builtin_amdgcn_readfirstlane(cnt_side[bh]);
  auto clamp = [](int n, int64_t cap) { return n < 0 ? 0 : (n > cap ? (int)cap : n); };
  const int n_lr = clamp(raw_lr, lr.cap), n_side = clamp(raw_side, side.cap);
  const int ch_lr = (n_lr + kChunk - 1) / kChunk;
  const int ch_side = (n_side + kChunk - 1) / kChunk;
  const int P = gridDim.x;
  int p_side = 0;
  if (ch_side > 0) {
    if (ch_lr == 0) {
      p_side = P;
    } else {
      // round(P * bytes_side / (bytes_lr + bytes_side)) in double (exact
      // enough for these ranges, and without a 64-bit integer division)
      const double w_lr = (double)ch_lr * (lr.rk + lr.rv), w_side = (double)ch_side * (2 * lr.d);
      p_side = (int)floor(P * w_side / (w_lr + w_side) + 0.5);
      p_side = p_side < 1 ? 1 : (p_side > P - 1 ? P - 1 : p_side);
    }
  }
  const int p_lr = P - p_side;
  const int x = blockIdx.x;
  if (x < p_lr) {
    SplitArgs a = lr;
    a.n_dev = nullptr;
    a.n_ctx_b = nullptr;   // (no per-sequence lengths, append, final outputs or
    a.k_new = nullptr;     // fixed-size runs here: known to the compiler, so their
    a.out = nullptr;       // branches and argument loads drop out)
    a.chunks_per_split = 0;
    a.n_static = n_lr;
    a.list_wgs = p_lr;
    split_bf16_body<KC, VB, true, kStages<KC, VB>, false, true, true>(a, x, x, sm);
  } else {
    // the side list's own fields; the rest as the low-rank list's
    SplitArgs a = lr;
    a.basis_k = nullptr;
    a.basis_v = nullptr;
    a.ck = side.ck;
    a.cv = side.cv;
    a.cap = side.cap;
    a.rk = a.rv = lr.d;
    a.n_dev = nullptr;
    a.n_ctx_b = nullptr;
    a.k_new = nullptr;
    a.out = nullptr;
    a.chunks_per_split = 0;
    a.n_static = n_side;
    a.list_wgs = p_side;
    split_bf16_body<SKC, SVB, false, 1, false, false, true>(a, x - p_lr, x, sm);
  }
  if (lr.merge_cnt != nullptr) merge_in_launch(lr, bh, P);
}

// ----------------------------------------------------------------------------
// float32 attention kernel (vector ALU): 64-token tiles, one token per lane for
// the scores, one value column per lane for the accumulation.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void split_f32_kernel(SplitArgs a) {
  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = tid & 63;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int split = blockIdx.x * kWaves + wave;
  const int g = a.g;
  const int rk = a.rk, rv = a.rv, d = a.d;
  const int64_t bh = (int64_t)b * a.hkv + h;
  const bool fold = a.basis_k != nullptr;
  const int qw = fold ? d : rk;   // q row width: d for the fold, else already r_K wide

  __shared__ float s_q[8 * 128];
  __shared__ float s_qf[8 * 128];
  __shared__ float s_p[kWaves][8][64];
  __shared__ float s_ml[kWaves][8][2];
  __shared__ __attribute__((aligned(16))) float s_acc[kWaves][16][128];   // rows 0..g-1 used

  const float* q = static_cast<const float*>(a.q) + ((int64_t)b * a.hq + (int64_t)h * g) * qw;
  for (int i = tid; i < g * qw; i += 256) s_q[i] = q[i];
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
    for (int i = tid; i < g * rk; i += 256) s_qf[i] = s_q[i] * a.qscale;
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
            const float* qq = s_qf + j * rk + k;
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

#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < g) {
      for (int ci = 0; ci < 2; ++ci) {
        const int c = lane + 64 * ci;
        if (c < rv) s_acc[wave][j][c] = acc[j][ci];
      }
      if (lane == 0) {
        s_ml[wave][j][0] = m_run[j];
        s_ml[wave][j][1] = l_run[j];
      }
    }
  }
  __syncthreads();
  workgroup_partial<float>(a, b, h, blockIdx.x, &s_acc[0][0][0], 128, s_ml, nullptr, s_qf);
}

// ----------------------------------------------------------------------------
// merge kernel of the two-phase interface: one workgroup per (batch, kv head)
// ----------------------------------------------------------------------------
// (one workgroup per unit is far below a full chip, so occupancy is not a
// concern: the register budget of two waves per SIMD lets every load of a
// batch of partials issue before the first use)
template <typename T>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void merge_kernel(MergeArgs a) {
  merge_unit<T>(a, blockIdx.x);
}

}  // namespace

#define LRKV_LATENT_CASE(KC, VB)                                                         \
  case (KC * 16 + VB):                                                                   \
    hipLaunchKernelGGL((split_bf16_latent_kernel<KC, VB>), grid, dim3(256), 0, s, a);    \
    break;

hipError_t launch_split_bf16_latent(const SplitArgs& a, hipStream_t s) {
  const dim3 grid(a.n_parts, a.hkv, a.batch);
  const int kc = (a.rk + 31) / 32, vb = (a.rv + 15) / 16;
  if (a.basis_k != nullptr || a.basis_v != nullptr || a.k_new != nullptr) return hipErrorInvalidValue;
  switch (kc * 16 + vb) {
    LRKV_LATENT_CASE(1, 1) LRKV_LATENT_CASE(1, 2) LRKV_LATENT_CASE(1, 3) LRKV_LATENT_CASE(1, 4)
    LRKV_LATENT_CASE(1, 5) LRKV_LATENT_CASE(1, 6) LRKV_LATENT_CASE(1, 7) LRKV_LATENT_CASE(1, 8)
    LRKV_LATENT_CASE(2, 1) LRKV_LATENT_CASE(2, 2) LRKV_LATENT_CASE(2, 3) LRKV_LATENT_CASE(2, 4)
    LRKV_LATENT_CASE(2, 5) LRKV_LATENT_CASE(2, 6) LRKV_LATENT_CASE(2, 7) LRKV_LATENT_CASE(2, 8)
    LRKV_LATENT_CASE(3, 1) LRKV_LATENT_CASE(3, 2) LRKV_LATENT_CASE(3, 3) LRKV_LATENT_CASE(3, 4)
    LRKV_LATENT_CASE(3, 5) LRKV_LATENT_CASE(3, 6) LRKV_LATENT_CASE(3, 7) LRKV_LATENT_CASE(3, 8)
    LRKV_LATENT_CASE(4, 1) LRKV_LATENT_CASE(4, 2) LRKV_LATENT_CASE(4, 3) LRKV_LATENT_CASE(4, 4)
    LRKV_LATENT_CASE(4, 5) LRKV_LATENT_CASE(4, 6) LRKV_LATENT_CASE(4, 7) LRKV_LATENT_CASE(4, 8)
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

#define LRKV_HYB_CASE(KC, VB, SKC, SVB)                                                              \
  case (KC * 16 + VB):                                                                               \
    hipLaunchKernelGGL((split_bf16_hybrid_kernel<KC, VB, SKC, SVB>), grid, dim3(256), 0, s, lr, side); \
    break;

hipError_t launch_split_bf16_hybrid(const SplitArgs& lr, const SplitArgs& side, int wgs_per_unit, hipStream_t s) {
  const dim3 grid(wgs_per_unit, lr.hkv, lr.batch);
  if (wgs_per_unit < 1 || lr.n_parts != wgs_per_unit || lr.n_dev == nullptr || side.n_dev == nullptr)
    return hipErrorInvalidValue;
  const int kc = (lr.rk + 31) / 32, vb = (lr.rv + 15) / 16;
  if (lr.basis_k == nullptr || lr.basis_v == nullptr || side.basis_k != nullptr || side.basis_v != nullptr ||
      side.rk != lr.d || side.rv != lr.d)
    return hipErrorInvalidValue;
  if (lr.d == 64) {
    switch (kc * 16 + vb) {
      LRKV_HYB_CASE(1, 1, 2, 4) LRKV_HYB_CASE(1, 2, 2, 4) LRKV_HYB_CASE(1, 3, 2, 4) LRKV_HYB_CASE(1, 4, 2, 4)
      LRKV_HYB_CASE(2, 1, 2, 4) LRKV_HYB_CASE(2, 2, 2, 4) LRKV_HYB_CASE(2, 3, 2, 4) LRKV_HYB_CASE(2, 4, 2, 4)
      default:
        return hipErrorInvalidValue;
    }
  } else {
    switch (kc * 16 + vb) {
      LRKV_HYB_CASE(1, 1, 4, 8) LRKV_HYB_CASE(1, 2, 4, 8) LRKV_HYB_CASE(1, 3, 4, 8) LRKV_HYB_CASE(1, 4, 4, 8)
      LRKV_HYB_CASE(1, 5, 4, 8) LRKV_HYB_CASE(1, 6, 4, 8) LRKV_HYB_CASE(1, 7, 4, 8) LRKV_HYB_CASE(1, 8, 4, 8)
      LRKV_HYB_CASE(2, 1, 4, 8) LRKV_HYB_CASE(2, 2, 4, 8) LRKV_HYB_CASE(2, 3, 4, 8) LRKV_HYB_CASE(2, 4, 4, 8)
      LRKV_HYB_CASE(2, 5, 4, 8) LRKV_HYB_CASE(2, 6, 4, 8) LRKV_HYB_CASE(2, 7, 4, 8) LRKV_HYB_CASE(2, 8, 4, 8)
      LRKV_HYB_CASE(3, 1, 4, 8) LRKV_HYB_CASE(3, 2, 4, 8) LRKV_HYB_CASE(3, 3, 4, 8) LRKV_HYB_CASE(3, 4, 4, 8)
      LRKV_HYB_CASE(3, 5, 4, 8) LRKV_HYB_CASE(3, 6, 4, 8) LRKV_HYB_CASE(3, 7, 4, 8) LRKV_HYB_CASE(3, 8, 4, 8)
      LRKV_HYB_CASE(4, 1, 4, 8) LRKV_HYB_CASE(4, 2, 4, 8) LRKV_HYB_CASE(4, 3, 4, 8) LRKV_HYB_CASE(4, 4, 4, 8)
      LRKV_HYB_CASE(4, 5, 4, 8) LRKV_HYB_CASE(4, 6, 4, 8) LRKV_HYB_CASE(4, 7, 4, 8) LRKV_HYB_CASE(4, 8, 4, 8)
      default:
        return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

hipError_t launch_split_f32(const SplitArgs& a, hipStream_t s) {
  const dim3 grid((a.n_splits + kWaves - 1) / kWaves, a.hkv, a.batch);
  hipLaunchKernelGGL(split_f32_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, bool bf16, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.batch * a.hkv));
  if (bf16) hipLaunchKernelGGL(merge_kernel<uint16_t>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(merge_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lrkv
