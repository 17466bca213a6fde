// Device code of the split-K decode attention kernels (gfx950), shared by
// decode.hip and decode_split.hip.
//
// Split-K decode attention over a low-rank KV cache (gfx950).
//
// Launch 1, the attention kernel: one workgroup attends a run of 32-token
// chunks of one (batch, kv head) for all g query heads of that kv head, so
// every coefficient row is read from HBM once per kv head; its four waves
// take the run's chunks in turn (wave w: chunks w, w + 4, ...), so that they
// read one dense window of the cache together.  Per chunk:
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
// precision.  At the end the workgroup's four waves are merged in LDS and the
// merged latent accumulator is lifted through B_V^T, so each workgroup leaves
// one head_dim-wide partial (running max, sum, unnormalised output) per query
// head.  When one workgroup covers a (batch, kv head) it writes the final
// output and lse itself instead, and there is no second launch.
// Launch 2, the merge kernel: log-sum-exp combination of those partials
// (and of the full-rank side list's partials in the hybrid cache).
// Variants: a decode step's appended token is compressed and attended inside
// launch 1 (with the basis, or a separate key encoder); latent queries and
// outputs (projections that absorb the bases) skip the fold and the lift.
#pragma once

#include "lrkv_device.h"
#include "lrkv_internal.h"

namespace lrkv {

namespace {

constexpr int kWaves = 4;
// the fold's operand row that carries an appended key (query heads take rows < g <= 8)
constexpr int kAppRow = 15;

template <typename T>
__device__ __forceinline__ float load_f(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_f<float>(const float* p, int64_t i) { return p[i]; }

// A partial result.  DEVICE: a device-scope store (written through to memory,
// sc1), for a partial that another workgroup of the same launch merges.
template <bool DEVICE = false>
__device__ __forceinline__ void store_partial(float* p, float v) {
  if (DEVICE) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}

template <typename T>
__device__ __forceinline__ void store_f(T* p, int64_t i, float v);
template <>
__device__ __forceinline__ void store_f<uint16_t>(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
template <>
__device__ __forceinline__ void store_f<float>(float* p, int64_t i, float v) { p[i] = v; }

// ----------------------------------------------------------------------------
// workgroup epilogue shared by the attention kernels
// ----------------------------------------------------------------------------
// In LDS on entry: wave w's unnormalised latent accumulator of head j at
// s_acc[(w * 16 + j) * acc_ld + c] (c < rv), and s_ml[w][j] = {running max
// (log2 units), sum}.  The four waves are merged (M = max_w m_w,
// acc = sum_w 2^(m_w - M) acc_w, likewise the sum), the result is lifted
// through B_V^T (or taken as is when the values are full rank, basis_v null)
// and written as this workgroup's partial.
// s_bv: B_V already staged in LDS with row pitch rv + 16 / sizeof(T), or
// null to read it from memory.
template <typename T>
__device__ void workgroup_partial(const SplitArgs& a, int b, int h, int part, const float* s_acc, int acc_ld,
                                  const float (*s_ml)[8][2], const T* s_bv, float* s_merged) {
  const int tid = threadIdx.x;
  const int g = a.g, rv = a.rv, d = a.d;
  constexpr int kVec = 16 / sizeof(T);
  const int ldb = rv + kVec;
  const bool lift = a.basis_v != nullptr;
  __shared__ float s_w[kWaves][8];
  __shared__ float s_mm[8][2];
  const T* bv = lift ? static_cast<const T*>(a.basis_v) + (int64_t)h * d * rv : nullptr;

  if (tid < g) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_ml[w][tid][0]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float m = s_ml[w][tid][0];
      const float wt = m == -INFINITY ? 0.f : exp2_fast(m - M);
      s_w[w][tid] = wt;
      L = fmaf(wt, s_ml[w][tid][1], L);
    }
    s_mm[tid][0] = M;
    s_mm[tid][1] = L;
  }
  __syncthreads();
  for (int i = tid; i < g * rv; i += 256) {
    const int j = i / rv, c = i - j * rv;
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) acc = fmaf(s_w[w][j], s_acc[(w * 16 + j) * acc_ld + c], acc);
    s_merged[j * 128 + c] = acc;
  }
  __syncthreads();
  const int64_t row0 = (int64_t)b * a.hq + (int64_t)h * g;
  float* po = a.part_o;
  if (lift) {
    for (int i = tid; i < g * d; i += 256) {
      const int j = i / d, dd = i - j * d;
      const T* br = s_bv ? s_bv + dd * ldb : bv + (int64_t)dd * rv;
      const float* ac = s_merged + j * 128;
      float o = 0.f;
      for (int c = 0; c < rv; ++c) o = fmaf(load_f(br, c), ac[c], o);
      store_partial(po + ((row0 + j) * a.n_parts + part) * d + dd, o);
    }
  } else {
    for (int i = tid; i < g * rv; i += 256) {
      const int j = i / rv, c = i - j * rv;
      store_partial(po + ((row0 + j) * a.n_parts + part) * rv + c, s_merged[j * 128 + c]);
    }
  }
  if (tid < g) {
    store_partial(a.part_ml + ((row0 + tid) * a.n_parts + part) * 2 + 0, s_mm[tid][0]);
    store_partial(a.part_ml + ((row0 + tid) * a.n_parts + part) * 2 + 1, s_mm[tid][1]);
  }
}

// ----------------------------------------------------------------------------
// log-sum-exp merge of the partials of one (batch, kv head)
// ----------------------------------------------------------------------------
//   M = max_s m_s,  L = sum_s 2^(m_s - M) l_s,
//   out = sum_s 2^(m_s - M) o_s / L,  lse = (M + log2 L) ln 2
// over the n_parts partials of each of the unit's g query heads; partials of
// workgroups that saw no token have m_s = -inf and weigh nothing.  Wave w
// takes heads w, w + 4.  Lane (grp, col) of a wave folds float4 column col of
// partials grp, grp + 64 / (d / 4), ... into a running (max, sum, output),
// sixteen partials at a time: their loads are issued together, the batch's
// maximum is taken first, the running state is rescaled to it once and the
// partials are added with their weights in ascending order (so no step waits
// for the previous step's maximum).  The lane groups are then combined
// pairwise (the lower lane's state first, so that both lanes of a pair
// compute the same bits).
struct MergeState {
  float m, l;
  f32x4 o;
};

__device__ __forceinline__ MergeState merge_two(const MergeState& a, const MergeState& b) {
  const float M = fmaxf(a.m, b.m);
  const float wa = a.m == -INFINITY ? 0.f : exp2_fast(a.m - M);
  const float wb = b.m == -INFINITY ? 0.f : exp2_fast(b.m - M);
  MergeState r;
  r.m = M;
  r.l = fmaf(b.l, wb, a.l * wa);
#pragma unroll
  for (int e = 0; e < 4; ++e) r.o[e] = fmaf(b.o[e], wb, a.o[e] * wa);
  return r;
}

template <typename T, bool DEVICE = false>
__device__ void merge_unit(const MergeArgs& a, int64_t unit) {
  constexpr int kU = 16;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int S = a.n_parts, d = a.d, g = a.g;
  // d / 4 float4 columns, rounded up to a power of two lanes (a latent
  // output's width r_V need not be one); lanes past the width compute
  // unused values and store nothing
  int cols = 1;
  while (cols < d / 4) cols <<= 1;
  const int groups = 64 / cols;
  const int col = lane % cols, grp = lane / cols;
  for (int j = wave; j < g; j += kWaves) {
    const int64_t row = unit * g + j;
    const __amdgpu_buffer_rsrc_t rs_ml = make_rsrc(a.part_ml + row * S * 2, (uint32_t)(S * 8));
    const __amdgpu_buffer_rsrc_t rs_o = make_rsrc(a.part_o + row * S * d, (uint32_t)(S * d * 4));
    MergeState st{-INFINITY, 0.f, f32x4{0.f, 0.f, 0.f, 0.f}};
    for (int s0 = grp; s0 < S; s0 += groups * kU) {
      u32x2 ml[kU];
      u32x4 ov[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t s = (uint32_t)(s0 + u * groups);
        ml[u] = DEVICE ? buf_load8_device(rs_ml, s * 8) : buf_load8(rs_ml, s * 8);
        ov[u] = DEVICE ? buf_load16_device(rs_o, (s * d + 4 * col) * 4) : buf_load16(rs_o, (s * d + 4 * col) * 4);
      }
      // the batch's maximum first, then every partial's weight at once (no
      // step waits for the previous one's maximum), in ascending order.  An
      // empty partial (max -inf, or past the count) is skipped by a select,
      // whatever its output words hold (an appended token's slot has none);
      // no branch depends on the maxima, so every load of the batch issues
      // before the first use
      float mb = st.m;
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (s0 + u * groups < S) mb = fmaxf(mb, __uint_as_float(ml[u][0]));
      const float sc = st.m == -INFINITY ? 0.f : exp2_fast(st.m - mb);
      st.l *= sc;
#pragma unroll
      for (int e = 0; e < 4; ++e) st.o[e] *= sc;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const float ms = __uint_as_float(ml[u][0]);
        const bool live = s0 + u * groups < S && ms != -INFINITY;
        const float w = live ? exp2_fast(ms - mb) : 0.f;
        st.l = live ? fmaf(w, __uint_as_float(ml[u][1]), st.l) : st.l;
#pragma unroll
        for (int e = 0; e < 4; ++e) st.o[e] = live ? fmaf(w, __uint_as_float(ov[u][e]), st.o[e]) : st.o[e];
      }
      st.m = mb;
    }
    for (int off = cols; off < 64; off <<= 1) {
      MergeState other;
      other.m = __shfl_xor(st.m, off);
      other.l = __shfl_xor(st.l, off);
#pragma unroll
      for (int e = 0; e < 4; ++e) other.o[e] = __shfl_xor(st.o[e], off);
      st = (lane & off) ? merge_two(other, st) : merge_two(st, other);
    }
    const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
    if (grp == 0 && 4 * col < d) {
#pragma unroll
      for (int e = 0; e < 4; ++e) store_f(static_cast<T*>(a.out), row * d + 4 * col + e, st.o[e] * inv);
    }
    if (lane == 0 && a.lse) a.lse[row] = st.l > 0.f ? (st.m + __log2f(st.l)) * kLn2 : -INFINITY;
  }
}

// Merge in the attention launch (a.merge_cnt set; the partials were stored
// with device scope, sc1, written through to memory): each wave waits for
// its own stores, the workgroup barrier follows, and one thread counts the
// workgroup's arrival on its unit's counter with a device-scope atomic.  The
// workgroup that arrives last of `arrivals` merges the unit's a.n_parts
// partials with device-scope loads (no stale line of another XCD's L2 is
// returned) into a.merge_out / a.merge_lse and sets the counter back to zero
// for the next launch.  No fence is needed: the stores are complete at the
// coherence point before the count, and the loads read from there.
__device__ __forceinline__ void merge_in_launch(const SplitArgs& a, int64_t bh, int arrivals) {
  __shared__ uint32_t s_last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(a.merge_cnt + bh, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (uint32_t)(arrivals - 1);
  __syncthreads();
  if (!s_last) return;
  MergeArgs m{};
  m.part_o = a.part_o; m.part_ml = a.part_ml; m.n_parts = a.n_parts;
  m.d = a.d; m.g = a.g; m.hq = a.hq; m.hkv = a.hkv; m.batch = a.batch;
  m.out = a.merge_out; m.lse = a.merge_lse;
  merge_unit<uint16_t, true>(m, bh);
  // every workgroup of the unit has counted: the counter is free for the next launch
  if (threadIdx.x == 0) __hip_atomic_store(a.merge_cnt + bh, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ----------------------------------------------------------------------------
// bfloat16 attention kernel (matrix cores)
// ----------------------------------------------------------------------------
// KC: 32-wide k chunks covering r_K;  VB: 16-wide column blocks covering r_V.
// FOLD false: keys are full-rank rows (hybrid side list), q' = q * scale.
// STAGES: chunks in flight per wave, held in registers (2, or 1 where the
// operands are too wide for two waves per SIMD).
//
// Each chunk is read through buffer resources based at the chunk and sized to
// its valid tokens: rows past the context, and lanes pointed past the end on
// purpose (columns beyond the rank), read as zero without a branch.  The rows
// are read once, so the loads are non-temporal (they do not fill the caches).
// Chunks are double-buffered in registers: the loads of chunk i+1 are in
// flight while chunk i is scored and accumulated.
template <int KC, int VB>
struct Chunk {
  u32x4 k[2][KC];
  u32x4 v[VB];
};

// LDS of one attention workgroup: the prologue's B_K and the waves'
// accumulator rows share `raw`; B_V is staged in the prologue, so that its
// load overlaps the fold and the stream instead of delaying the epilogue.
struct SplitSmem {
  static constexpr int kRawBytes = 128 * (128 + 8) * 2;   // >= kWaves * 16 * 128 * 4
  __attribute__((aligned(16))) unsigned char raw[kRawBytes];
  __attribute__((aligned(16))) uint16_t bv[128 * (128 + 8)];   // B_V for the lift, pitch rv + 8
  float q[8 * 128];
  float qf[8 * 128];
  float ml[kWaves][8][2];
};

// wg: this workgroup's index among the workgroups attending this list of
// this (b, kv head); part: the partial it writes.  append: this workgroup
// also compresses the appended token (after the fold, while its first chunk
// streams in), stores its cache rows and adds the token as one more term of
// the workgroup's merge, so the token's own partial slot, a.n_parts - 1, is
// left empty.  ENC: the appended key has a separate encoder (a.enc_k).
// EARLY (two stages only): both register buffers are loaded before the fold,
// so that two chunks per wave stream in during the prologue instead of one.
template <int KC, int VB, bool FOLD, int STAGES, bool ENC = false, bool EARLY = false, bool DEVICE_PARTIAL = false>
__device__ __forceinline__ void split_bf16_body(const SplitArgs& a, int wg, int part, SplitSmem& sm,
                                                bool append = false) {
  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = tid & 63;
  const int n16 = lane & 15;     // matrix row/column index this lane supplies
  const int grp = lane >> 4;     // k-slot group
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int g = a.g;
  const int rk = a.rk, rv = a.rv, d = a.d;
  const int64_t bh = (int64_t)b * a.hkv + h;

  static_assert(kWaves * 16 * VB * 16 * 4 <= SplitSmem::kRawBytes, "accumulator rows exceed LDS");
  float* s_q = sm.q;
  float* s_qf = sm.qf;
  float (*s_ml)[8][2] = sm.ml;
  uint16_t* s_bk = reinterpret_cast<uint16_t*>(sm.raw);
  float (*s_acc)[16][VB * 16] = reinterpret_cast<float (*)[16][VB * 16]>(sm.raw);

  // lengths on the device are the same for the whole workgroup: read as
  // scalars, so that the buffer resources built from them stay scalar
  int64_t n_end = a.n_static;
  if (a.n_dev) {
    n_end = __builtin_amdgcn_readfirstlane(a.n_dev[bh]);
    if (n_end > a.cap) n_end = a.cap;
    if (n_end < 0) n_end = 0;
  }
  // the appended token's row (decode step), and whether this workgroup owns
  // the token's partial slot (it marks the slot empty even when a device
  // length outside [1, cap] leaves nothing to append)
  int64_t append_row = a.append_row;
  const bool tok_slot = append;
  int64_t cps = a.chunks_per_split;
  if (a.n_ctx_b) {
    const int64_t total = __builtin_amdgcn_readfirstlane(a.n_ctx_b[b]);
    const bool ok = total >= 1 && total <= a.cap;
    n_end = ok ? (a.k_new ? total - 1 : total) : 0;
    append_row = total - 1;
    append = append && ok;
    // the host planned n_splits splits (ceil(n_splits / kWaves) attention
    // workgroups) for a length bound; ceil(chunks / n_splits) chunks per
    // split needs at most n_splits splits for any length, and is the host's
    // own plan when the length is the bound
    cps = ((n_end + kChunk - 1) / kChunk + a.n_splits - 1) / a.n_splits;
  }
  // The workgroup owns kWaves * cps consecutive chunks and its waves take
  // them in turn: wave w reads chunks w, w + kWaves, ...  Four waves reading
  // adjacent chunks keep the workgroup's loads in one dense window of the
  // cache (measured: 1.4 % faster than one contiguous run per wave with ranks
  // 32/96, where every per-wave run starts at a multiple of 128 KB).  The
  // online softmax does not depend on the order.
  // With a.list_wgs the workgroups' runs differ by at most one chunk (the
  // per-workgroup bytes, which set when a workgroup's stream ends, are even).
  const int64_t n_chunks = (n_end + kChunk - 1) / kChunk;
  const int64_t w_begin = a.list_wgs > 0 ? n_chunks * wg / a.list_wgs : (int64_t)wg * kWaves * cps;
  const int64_t c_begin = w_begin + wave;
  int64_t c_end = a.list_wgs > 0 ? n_chunks * (wg + 1) / a.list_wgs : w_begin + (int64_t)kWaves * cps;
  if (c_end > n_chunks) c_end = n_chunks;
  constexpr int64_t kStep = kWaves;

  const uint16_t* ck = static_cast<const uint16_t*>(a.ck) + bh * a.cap * rk;
  const uint16_t* cv = static_cast<const uint16_t*>(a.cv) + bh * a.cap * rv;
  // per-lane byte offsets inside a chunk; lanes past the rank point out of range
  uint32_t vo_k[2][KC], vo_v[VB];
#pragma unroll
  for (int T = 0; T < 2; ++T)
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int col = 32 * c + 8 * grp;
      const int row = 8 * (n16 >> 2) + 4 * T + (n16 & 3);   // tile T, row n16
      vo_k[T][c] = col < rk ? (uint32_t)((row * rk + col) * 2) : kOob;
    }
#pragma unroll
  for (int vb = 0; vb < VB; ++vb) {
    const int col = 16 * vb + n16;
    vo_v[vb] = col < rv ? (uint32_t)((grp * rv + col) * 16) : kOob;
  }
  // a chunk past this wave's range (EARLY's loop loads one ahead
  // unconditionally) gets an empty range: its loads read zero without
  // touching memory, and every path issues the same loads
  auto load = [&](Chunk<KC, VB>& c, int64_t chunk) {
    const int64_t t0 = chunk * kChunk;
    const int64_t left = chunk < c_end ? n_end - t0 : 0;
    const int nt = left < kChunk ? (int)left : kChunk;
    const __amdgpu_buffer_rsrc_t rs_k = make_rsrc(ck + t0 * rk, (uint32_t)(nt * rk * 2));
    const __amdgpu_buffer_rsrc_t rs_v = make_rsrc(cv + t0 * rv, (uint32_t)(((nt + 7) >> 3) * rv * 16));
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int cc = 0; cc < KC; ++cc) c.k[T][cc] = buf_load16_stream(rs_k, vo_k[T][cc]);
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) c.v[vb] = buf_load16_stream(rs_v, vo_v[vb]);
  };

  // --- fold q' = q B_K * scale * log2(e) for the g query heads of this kv head
  Chunk<KC, VB> ca, cb;
  {
    // every load of the prologue, and the first chunk's, is issued before the first wait
    // q rows are d wide for the fold; without it they are already r_K wide
    // (a latent query, or a full-rank key list with r_K = d)
    const uint16_t* q = static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.hq + (int64_t)h * g) * (FOLD ? d : rk);
    const int nq = FOLD ? 0 : g * rk / 8;           // <= 128 sixteen-byte pieces
    const u32x4 wq = tid < nq ? *reinterpret_cast<const u32x4*>(q + 8 * tid) : u32x4{0u, 0u, 0u, 0u};
    // the fold's row operand: lane (n16, grp) holds q[head n16][32 c + 8 grp .. + 7].
    // Without a separate key encoder the appended token is compressed on the
    // matrix cores too: its key is row kAppRow of this operand (the fold's
    // product then also gives c_K = k B_K) and its value row 0 of a second
    // product against the staged B_V (va).
    const bool app_mfma = FOLD && !ENC && append;
    const uint16_t* qrow = n16 < g ? q + n16 * d
                                   : (app_mfma && n16 == kAppRow ? static_cast<const uint16_t*>(a.k_new) + bh * d
                                                                  : nullptr);
    const uint16_t* vrow = app_mfma && n16 == 0 ? static_cast<const uint16_t*>(a.v_new) + bh * d : nullptr;
    u32x4 qa[4], va[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      qa[c] = (FOLD && qrow && 32 * c < d) ? *reinterpret_cast<const u32x4*>(qrow + 32 * c + 8 * grp)
                                           : u32x4{0u, 0u, 0u, 0u};
      va[c] = (vrow && 32 * c < d) ? *reinterpret_cast<const u32x4*>(vrow + 32 * c + 8 * grp) : u32x4{0u, 0u, 0u, 0u};
    }
    constexpr int kBkIter = 8;                      // d * rk / 8 <= 2048 = 8 * 256
    u32x4 wb[kBkIter];
    const uint16_t* bk = FOLD ? static_cast<const uint16_t*>(a.basis_k) + (int64_t)h * d * rk : nullptr;
    const int nb = FOLD ? d * rk / 8 : 0;
#pragma unroll
    for (int it = 0; it < kBkIter; ++it) {
      const int i = tid + 256 * it;
      if (i < nb) wb[it] = *reinterpret_cast<const u32x4*>(bk + 8 * i);
    }
    // B_V of the epilogue's lift
    const int bv_row = a.rv / 8, nbv = a.basis_v ? d * bv_row : 0;
    const uint16_t* bvs = a.basis_v ? static_cast<const uint16_t*>(a.basis_v) + (int64_t)h * d * a.rv : nullptr;
    u32x4 wv[kBkIter];
#pragma unroll
    for (int it = 0; it < kBkIter; ++it) {
      const int i = tid + 256 * it;
      if (i < nbv) wv[it] = *reinterpret_cast<const u32x4*>(bvs + 8 * i);
    }
    // with a separate key encoder: the appended token's key and value as
    // floats (into the otherwise unused s_q) for the vector-ALU compress
    const int e_new = tid & 127;
    float x_new = 0.f;
    if (ENC && append && e_new < d) {
      if (tid < 128) x_new = bf16_to_f32(static_cast<const uint16_t*>(a.k_new)[bh * d + e_new]);
      else x_new = bf16_to_f32(static_cast<const uint16_t*>(a.v_new)[bh * d + e_new]);
    }
    // the first chunk (with EARLY, the first two) streams in while the query is folded
    if (EARLY) {
      load(ca, c_begin);
      load(cb, c_begin + kStep);
    } else if (c_begin < c_end) {
      load(ca, c_begin);
    }
    if (ENC && append && e_new < d) s_q[(tid < 128 ? 0 : 128) + e_new] = x_new;
    if (tid < nq) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s_q[8 * tid + 2 * e] = bf16_lo(wq[e]);
        s_q[8 * tid + 2 * e + 1] = bf16_hi(wq[e]);
      }
    }
#pragma unroll
    for (int it = 0; it < kBkIter; ++it) {
      const int i = tid + 256 * it;
      if (i < nb) *reinterpret_cast<u32x4*>(s_bk + 8 * i) = wb[it];
    }
#pragma unroll
    for (int it = 0; it < kBkIter; ++it) {
      const int i = tid + 256 * it;
      if (i < nbv) *reinterpret_cast<u32x4*>(sm.bv + (i / bv_row) * (a.rv + 8) + (i % bv_row) * 8) = wv[it];
    }
    __syncthreads();
    if (FOLD) {
      // on the matrix cores: wave w takes the 16-column blocks w, w + 4, ... of q' = q B_K;
      // the column operand, lane (n16, grp): B_K[32 c + 8 grp + e][16 nb + n16], e < 8,
      // read transposed from the staged rows (two 8-byte reads; a column past
      // r_K reads other bytes of the staged block, and its result is not kept)
      for (int nb = wave; nb * 16 < rk; nb += kWaves) {
        const int col = 16 * nb + n16;
        f32x4 f = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (32 * c < d) {
            const uint16_t* src = s_bk + (32 * c + 8 * grp + (n16 >> 2)) * rk + 16 * nb + 4 * (n16 & 3);
            const u32x2 lo = lds_read_tr16(src);
            const u32x2 hi = lds_read_tr16(src + 4 * rk);
            f = mfma_16x16x32(qa[c], u32x4{lo[0], lo[1], hi[0], hi[1]}, f);
          }
        }
        // lane (n16, grp) register i: q' of head 4 grp + i, column col
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * grp + i < g && col < rk) s_qf[(4 * grp + i) * rk + col] = f[i] * a.qscale;
        // row kAppRow: the appended key's coefficient, rounded once, kept
        // (s_c, for its score) and stored at the appended cache row
        if (app_mfma && grp == kAppRow / 4 && col < rk) {
          const uint16_t c16 = f32_to_bf16(f[kAppRow % 4]);
          s_q[256 + col] = bf16_to_f32(c16);
          const_cast<uint16_t*>(ck)[append_row * rk + col] = c16;
        }
      }
      if (app_mfma) {
        // c_V = v B_V: wave w takes the 16-column blocks w, w + 4, ...; the
        // column operand is read transposed from the staged B_V (pitch rv + 8)
        const int ldv = rv + 8;
        for (int nb = wave; nb * 16 < rv; nb += kWaves) {
          const int col = 16 * nb + n16;
          f32x4 f = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if (32 * c < d) {
              const uint16_t* src = sm.bv + (32 * c + 8 * grp + (n16 >> 2)) * ldv + 16 * nb + 4 * (n16 & 3);
              const u32x2 lo = lds_read_tr16(src);
              const u32x2 hi = lds_read_tr16(src + 4 * ldv);
              f = mfma_16x16x32(va[c], u32x4{lo[0], lo[1], hi[0], hi[1]}, f);
            }
          }
          // row 0 (lane group 0, register 0): the value's coefficient, column col
          if (grp == 0 && col < rv) {
            const uint16_t c16 = f32_to_bf16(f[0]);
            s_q[256 + 128 + col] = bf16_to_f32(c16);
            const_cast<uint16_t*>(cv)[((append_row >> 3) * rv + col) * 8 + (append_row & 7)] = c16;
          }
        }
      }
    } else {
      for (int i = tid; i < g * rk; i += 256) s_qf[i] = s_q[i] * a.qscale;
    }
    __syncthreads();
  }

  // Query operand of the score product: column n16 is head n16 (high part in
  // the first MFMA, low part in the second); columns g..2g-1 repeat the heads
  // so that lanes g..2g-1 also see full scores; other columns are zero.
  const int head = n16 < g ? n16 : (n16 < 2 * g ? n16 - g : -1);
  u32x4 bq_hi[KC], bq_lo[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    // r_K is a multiple of 8: a lane's 8 values are all inside or all past
    // it, and read as two 16-byte pieces
    const int k0 = 32 * c + 8 * grp;
    float4 q0 = make_float4(0.f, 0.f, 0.f, 0.f), q1 = q0;
    if (head >= 0 && k0 < rk) {
      q0 = *reinterpret_cast<const float4*>(s_qf + head * rk + k0);
      q1 = *reinterpret_cast<const float4*>(s_qf + head * rk + k0 + 4);
    }
    const float v[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hi[e] = pack_bf16(v[2 * e], v[2 * e + 1]);
      lo[e] = pack_bf16(v[2 * e] - bf16_lo(hi[e]), v[2 * e + 1] - bf16_hi(hi[e]));
    }
    bq_hi[c] = u32x4{hi[0], hi[1], hi[2], hi[3]};
    bq_lo[c] = u32x4{lo[0], lo[1], lo[2], lo[3]};
  }

  if (append) {
    // With a separate key encoder: c = round(x E) for the key (threads < 128,
    // column tid) and c = round(x B_V) for the value (threads >= 128, column
    // tid - 128) on the vector ALU, stored at the appended row.  Without one
    // the prologue's matrix-core products already did this (s_c is complete
    // since its last barrier).  Then the token's score q' . c_K (log2 units),
    // kept with c_V for the epilogue.
    const int pa = a.n_parts - 1;
    const int64_t p = append_row;
    float* s_c = s_q + 256;   // past the token's key and value
    const int col = tid & 127;
    const bool kind_v = tid >= 128;
    const int r = kind_v ? rv : rk;
    if constexpr (ENC) {
      // a separate key encoder (a non-orthogonal transform) is read from
      // memory by every thread: thread (row group rg, column group cg) sums
      // x[e] E[e][8 cg .. 8 cg + 7] over rows e = rg, rg + n_rg, ... into
      // per-row-group partials in `raw` (B_K's copy there is dead after the
      // fold), which the key column threads then add up
      const int ng = rk >> 3;          // <= 16
      const int n_rg = 256 / ng;       // >= 16, so a thread takes <= 8 rows of d <= 128
      const int cg = tid % ng, rg = tid / ng;
      float* s_part = reinterpret_cast<float*>(sm.raw);
      if (rg < n_rg) {
        const uint16_t* src = static_cast<const uint16_t*>(a.enc_k) + (int64_t)h * d * rk + 8 * cg;
        float sum[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) sum[j] = 0.f;
        // two batches of four rows in flight (the attention's first chunk is
        // also in flight here, so registers are short)
        for (int i0 = 0; i0 < 8; i0 += 4) {
          u32x4 w[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = rg + n_rg * (i0 + i);
            w[i] = e < d ? *reinterpret_cast<const u32x4*>(src + (int64_t)e * rk) : u32x4{0u, 0u, 0u, 0u};
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = rg + n_rg * (i0 + i);
            const float xe = e < d ? s_q[e] : 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              sum[2 * j] = fmaf(xe, bf16_lo(w[i][j]), sum[2 * j]);
              sum[2 * j + 1] = fmaf(xe, bf16_hi(w[i][j]), sum[2 * j + 1]);
            }
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) s_part[rg * rk + 8 * cg + j] = sum[j];
      }
      __syncthreads();
    }
    if (ENC && col < r) {
      float acc = 0.f;
      if (kind_v) {
        // four partial sums: the token's compress is on this workgroup's critical path
        float p4[4] = {0.f, 0.f, 0.f, 0.f};
        for (int e = 0; e < d; e += 4)
#pragma unroll
          for (int u = 0; u < 4; ++u) p4[u] = fmaf(s_q[128 + e + u], bf16_to_f32(sm.bv[(e + u) * (rv + 8) + col]), p4[u]);
        acc = (p4[0] + p4[1]) + (p4[2] + p4[3]);
      } else if (ENC) {
        const float* s_part = reinterpret_cast<const float*>(sm.raw);
        const int n_rg = 256 / (rk >> 3);
        for (int i = 0; i < n_rg; ++i) acc += s_part[i * rk + col];
      } else {
        float p4[4] = {0.f, 0.f, 0.f, 0.f};
        for (int e = 0; e < d; e += 4)
#pragma unroll
          for (int u = 0; u < 4; ++u) p4[u] = fmaf(s_q[e + u], bf16_to_f32(s_bk[(e + u) * rk + col]), p4[u]);
        acc = (p4[0] + p4[1]) + (p4[2] + p4[3]);
      }
      const uint16_t c16 = f32_to_bf16(acc);
      s_c[(kind_v ? 128 : 0) + col] = bf16_to_f32(c16);
      if (kind_v)
        static_cast<uint16_t*>(const_cast<void*>(a.cv))[bh * a.cap * rv + ((p >> 3) * rv + col) * 8 + (p & 7)] = c16;
      else
        static_cast<uint16_t*>(const_cast<void*>(a.ck))[(bh * a.cap + p) * rk + col] = c16;
    }
    if (ENC) __syncthreads();
    const int64_t row0 = (int64_t)b * a.hq + (int64_t)h * g;
    if (tid < g) {
      float p4[4] = {0.f, 0.f, 0.f, 0.f};
      for (int k = 0; k < rk; k += 4)   // rk is a multiple of 8
#pragma unroll
        for (int u = 0; u < 4; ++u) p4[u] = fmaf(s_qf[tid * rk + k + u], s_c[k + u], p4[u]);
      const float s = (p4[0] + p4[1]) + (p4[2] + p4[3]);
      // the token joins this workgroup's merge in the epilogue (c_V stays in
      // s_c), before the lift; its own partial slot is marked empty
      s_q[512 + tid] = s;
      if (!a.out) {
        store_partial<DEVICE_PARTIAL>(a.part_ml + ((row0 + tid) * a.n_parts + pa) * 2 + 0, -INFINITY);
        store_partial<DEVICE_PARTIAL>(a.part_ml + ((row0 + tid) * a.n_parts + pa) * 2 + 1, 0.f);
      }
    }
  } else if (tok_slot && !a.out && tid < g) {
    // no token to append (a device length outside [1, cap]): its slot stays empty
    const int64_t row0 = (int64_t)b * a.hq + (int64_t)h * g;
    store_partial<DEVICE_PARTIAL>(a.part_ml + ((row0 + tid) * a.n_parts + a.n_parts - 1) * 2 + 0, -INFINITY);
    store_partial<DEVICE_PARTIAL>(a.part_ml + ((row0 + tid) * a.n_parts + a.n_parts - 1) * 2 + 1, 0.f);
  }


  f32x4 acc[VB];
#pragma unroll
  for (int i = 0; i < VB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  // This lane takes the high (rows < g) or low (rows g..2g-1) part of p.
  const bool take_hi = n16 < g;
  const bool p_row = n16 < 2 * g;

  auto process = [&](Chunk<KC, VB>& c, int64_t chunk) {
    const int64_t t0 = chunk * kChunk;
    const int64_t oct_tok = t0 + 8 * grp;
    const bool tail = t0 + kChunk > n_end;
    if (tail) {
      // value elements past the end may hold anything: zero them
      const int64_t nv = n_end - oct_tok;
#pragma unroll
      for (int vb = 0; vb < VB; ++vb)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t m = 0u;
          if (2 * w < nv) m |= 0x0000FFFFu;
          if (2 * w + 1 < nv) m |= 0xFFFF0000u;
          c.v[vb][w] &= m;
        }
    }
    // scores: tile T, row m is token t0 + 8*(m/4) + 4*T + m%4
    f32x4 st[2];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < KC; ++cc) {
        s = mfma_16x16x32(c.k[T][cc], bq_hi[cc], s);
        s = mfma_16x16x32(c.k[T][cc], bq_lo[cc], s);
      }
      st[T] = s;
    }
    // lane (n16, grp) now holds, for head(n16), tokens t0 + 8*grp + 4*T + i
    float sv[8];
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[4 * T + i] = st[T][i];
    if (tail) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (oct_tok + e >= n_end) sv[e] = -INFINITY;
    }
    float cmax = sv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cmax = fmaxf(cmax, sv[e]);
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
      acc[vb] = mfma_16x16x32(pop, c.v[vb], acc[vb]);
    }
  };

  if (STAGES == 2 && EARLY) {
    if (c_begin + kStep >= c_end) {
      // at most one chunk for this wave (short contexts)
      if (c_begin < c_end) process(ca, c_begin);
    } else {
      // one chunk always in flight behind the one being processed
      for (int64_t chunk = c_begin; chunk < c_end; chunk += 2 * kStep) {
        process(ca, chunk);
        load(ca, chunk + 2 * kStep);
        if (chunk + kStep >= c_end) break;
        process(cb, chunk + kStep);
        load(cb, chunk + 3 * kStep);
      }
    }
  } else if (STAGES == 2) {
    for (int64_t chunk = c_begin; chunk < c_end; chunk += 2 * kStep) {
      if (chunk + kStep < c_end) load(cb, chunk + kStep);
      process(ca, chunk);
      if (chunk + kStep >= c_end) break;
      if (chunk + 2 * kStep < c_end) load(ca, chunk + 2 * kStep);
      process(cb, chunk + kStep);
    }
  } else {
    for (int64_t chunk = c_begin; chunk < c_end; chunk += kStep) {
      process(ca, chunk);
      if (chunk + kStep < c_end) load(ca, chunk + kStep);
    }
  }

  // --- epilogue
  // 1. Head j of the wave is accumulator row j (high part of p) plus row g + j
  //    (low part).  Row r lives in lane group r / 4, register r % 4; the 2 g
  //    rows go to LDS as they are and the four-wave merge below adds each
  //    pair (high + low, the same sum a cross-lane exchange here would form),
  //    so the wave exchanges nothing between lanes.
  //    The LDS written here (s_acc over the prologue's B_K, s_ml) was last read
  //    before the fold's barrier, so no barrier is needed first.
#pragma unroll
  for (int vb = 0; vb < VB; ++vb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * grp + i < 2 * g) s_acc[wave][4 * grp + i][16 * vb + n16] = acc[vb][i];
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (lane < g) {
    s_ml[wave][lane][0] = m_run;     // -inf for a wave without tokens
    s_ml[wave][lane][1] = l_tot;
  }
  __syncthreads();
  // 2. the four waves merged: M = max_w m_w, acc = sum_w 2^(m_w - M) acc_w,
  //    likewise the sum.  The appended token of this workgroup (score in
  //    s_q[512 + j], latent value c_V in s_c) is one more term.  With final
  //    outputs the sum is inverted for the lift instead of being stored.
  float* s_merged = s_qf;   // the query operand was read before the main loop
  const bool fin = a.out != nullptr;
  const bool tok = append;
  const float* s_tok_c = s_q + 256 + 128;
  float* s_inv = s_q + 520;
  for (int i = tid; i < g * rv; i += 256) {
    const int j = i / rv, c = i - j * rv;
    float M = tok ? s_q[512 + j] : -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_ml[w][j][0]);
    float o = tok ? exp2_fast(s_q[512 + j] - M) * s_tok_c[c] : 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float m = s_ml[w][j][0];
      o = fmaf(m == -INFINITY ? 0.f : exp2_fast(m - M), s_acc[w][j][c] + s_acc[w][g + j][c], o);
    }
    s_merged[j * 128 + c] = o;
  }
  const int64_t row0 = (int64_t)b * a.hq + (int64_t)h * g;
  if (tid < g) {
    float M = tok ? s_q[512 + tid] : -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_ml[w][tid][0]);
    float L = tok ? exp2_fast(s_q[512 + tid] - M) : 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float m = s_ml[w][tid][0];
      L = fmaf(m == -INFINITY ? 0.f : exp2_fast(m - M), s_ml[w][tid][1], L);
    }
    if (fin) {
      s_inv[tid] = L > 0.f ? 1.f / L : 0.f;
      if (a.lse) a.lse[row0 + tid] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
    } else {
      store_partial<DEVICE_PARTIAL>(a.part_ml + ((row0 + tid) * a.n_parts + part) * 2 + 0, M);
      store_partial<DEVICE_PARTIAL>(a.part_ml + ((row0 + tid) * a.n_parts + part) * 2 + 1, L);
    }
  }
  __syncthreads();
  // 3. lift o = acc B_V^T on the matrix cores: wave w takes the 16-dim blocks
  //    w, w + 4, ...; the row operand is acc (head n16) split into high and
  //    low bfloat16 parts, the column operand B_V[dim][32 c + 8 grp .. + 7]
  //    straight from the staged rows.  Full-rank values (side list) are the
  //    output as they are.
  float* po = a.part_o;
  if (FOLD) {
    const int ldb = rv + 8;
    // the row operand is the same for every dim block: built once per wave,
    // over the (VB + 1) / 2 blocks of 32 coefficients that cover r_V (a
    // compile-time count, so the B_V reads below are issued together)
    constexpr int kLiftK = (VB + 1) / 2;
    u32x4 a_hi[kLiftK], a_lo[kLiftK];
#pragma unroll
    for (int c = 0; c < kLiftK; ++c) {
      const int k0 = 32 * c + 8 * grp;
      const bool kv = k0 < rv;   // rv is a multiple of 8: a lane group is all in or all out
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (kv && n16 < g) ? s_merged[n16 * 128 + k0 + e] : 0.f;
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hi[e] = pack_bf16(v[2 * e], v[2 * e + 1]);
        lo[e] = pack_bf16(v[2 * e] - bf16_lo(hi[e]), v[2 * e + 1] - bf16_hi(hi[e]));
      }
      a_hi[c] = u32x4{hi[0], hi[1], hi[2], hi[3]};
      a_lo[c] = u32x4{lo[0], lo[1], lo[2], lo[3]};
    }
    for (int nd = wave; nd * 16 < d; nd += kWaves) {
      const int dim = 16 * nd + n16;
      f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < kLiftK; ++c) {
        const int k0 = 32 * c + 8 * grp;
        const u32x4 bvw = k0 < rv ? *reinterpret_cast<const u32x4*>(sm.bv + dim * ldb + k0) : u32x4{0u, 0u, 0u, 0u};
        o = mfma_16x16x32(a_hi[c], bvw, o);
        o = mfma_16x16x32(a_lo[c], bvw, o);
      }
      // lane (n16, grp) register i: head 4 grp + i, dim
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * grp + i >= g) continue;
        if (fin)
          static_cast<uint16_t*>(a.out)[(row0 + 4 * grp + i) * d + dim] = f32_to_bf16(o[i] * s_inv[4 * grp + i]);
        else
          store_partial<DEVICE_PARTIAL>(po + ((row0 + 4 * grp + i) * a.n_parts + part) * d + dim, o[i]);
      }
    }
  } else {
    // no lift: the partial is the r_V-wide accumulator (d wide for a full-rank list)
    for (int i = tid; i < g * rv; i += 256) {
      const int j = i / rv, c = i - j * rv;
      store_partial<DEVICE_PARTIAL>(po + ((row0 + j) * a.n_parts + part) * rv + c, s_merged[j * 128 + c]);
    }
  }
}

// Chunks in flight per wave: two unless that no longer fits two waves per
// SIMD (a chunk takes 4 (2 KC + VB) registers per lane).
template <int KC, int VB>
constexpr int kStages = 2 * KC + VB < 16 ? 2 : 1;

}  // namespace

}  // namespace lrkv
