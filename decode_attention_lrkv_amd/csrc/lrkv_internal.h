// Host-side launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lrkv.h"

namespace lrkv {

// Records a printf-style message for lrkv_last_error() on this thread and returns st.
lrkv_status fail(lrkv_status st, const char* fmt, ...);

constexpr float kLog2eHost = 1.4426950408889634f;

// Tokens per decode chunk: two 16-token matrix-core tiles.
constexpr int kChunk = 32;
// Waves (splits) per attention workgroup; a workgroup leaves one partial.
constexpr int kSplitsPerPart = 4;
// Upper bound on splits per (batch, kv head) the planner uses.
constexpr int kMaxSplits = 1 << 16;

struct SplitArgs {
  const void* q;         // [B, Hq, d], or [B, Hq, rk] without a fold
  const void* basis_k;   // [Hkv, d, rk] (nullptr: no fold; q is already rk wide: a latent
                         // query, or a full-rank key list with rk = d)
  const void* ck;        // key rows [B, Hkv, cap, rk]
  const void* cv;        // value octets [B, Hkv, cap/8, rv, 8]
  const void* basis_v;   // [Hkv, d, rv] (nullptr: no lift; partials are rv wide)
  int64_t cap;
  int rk, rv, d, g, hq, hkv, batch;
  int64_t n_static;      // context length when n_dev and n_ctx_b are null
  const int32_t* n_dev;  // per-(b, h) token counts on the device, or null
  // Per-sequence context lengths on the device ([B], the appended token
  // included), or null.  A length outside [1, cap] attends nothing (out 0,
  // lse -inf) and appends nothing.  With it the host plans n_splits splits
  // for a length bound and each workgroup's run of chunks is derived on the
  // device from the length (chunks_per_split is not used).
  const int32_t* n_ctx_b;
  int chunks_per_split;
  // > 0: the list's chunks are divided as evenly as whole chunks allow over
  // this many workgroups (wg in [0, list_wgs) takes chunks
  // [wg C / list_wgs, (wg + 1) C / list_wgs) of C); chunks_per_split is not used
  int list_wgs;
  int n_splits;
  int n_parts;           // partials per (b, q head): one per attention workgroup
  float qscale;          // softmax scale * log2(e)
  float* part_o;         // [B, Hq, n_parts, d (rv without a lift)]  unnormalised outputs
  float* part_ml;        // [B, Hq, n_parts, 2]  running max (log2 units), softmax sum
  // Append (decode step): when k_new is non-null, the last workgroup of each
  // (b, kv head) compresses the new token's key and value, stores them at
  // cache row append_row (through ck / cv) and adds the token to its own
  // partial (the token's slot, n_parts - 1, is marked empty);
  // the other workgroups attend rows [0, n_static).
  const void* k_new;     // [B, Hkv, d] or null
  const void* v_new;     // [B, Hkv, d]
  const void* enc_k;     // [Hkv, d, rk] encoder of the appended key, or null: basis_k encodes
  int64_t append_row;
  // Final outputs: with one attention workgroup per (b, kv head) (and the
  // append, if any, in that workgroup) the kernel normalises and writes
  // out [B, Hq, d] and lse [B, Hq] itself, and no partials or merge are needed.
  void* out;             // or null: write partials
  float* lse;            // or null
  // Merge in the same launch (hybrid cache): when merge_cnt is non-null,
  // every workgroup counts its arrival on merge_cnt[b * hkv + h] after its
  // partial is stored, and the workgroup that arrives last merges the unit's
  // n_parts partials into merge_out / merge_lse and sets the counter back to
  // zero.  The counters must be zero when the launch starts.
  uint32_t* merge_cnt;
  void* merge_out;       // [B, Hq, d]
  float* merge_lse;      // [B, Hq] or null
};

// Log-sum-exp merge of n_parts partials per (b, q head).
struct MergeArgs {
  const float* part_o; const float* part_ml; int n_parts;
  int d, g, hq, hkv, batch;
  void* out;             // [B, Hq, d]
  float* lse;            // [B, Hq] or null
};

struct CompressArgs {
  const void* x; const void* basis; void* coeff;
  int values_layout;     // 0: row layout, 1: octet layout
  int batch, hkv, d, rank;
  int64_t n_tokens, pos, cap;
};

// Both caches of a few new tokens in one launch.
constexpr int kSmallT = 4;
struct CompressKvArgs {
  const void* xk; const void* xv; const void* bk; const void* bv; void* ck; void* cv;
  int batch, hkv, d, rk, rv;
  int64_t n_tokens, pos, cap;
};

// Oja subspace update of the bases from a chunk of tokens (all batch rows).
struct OjaArgs {
  const void* x;         // [B, T, Hkv, d] bf16; n_tokens = B * T rows per head
  float* basis;          // [Hkv, d, rank] float32, updated in place
  void* basis_bf16;      // [Hkv, d, rank] bf16 copy, or null
  int hkv, d, rank;
  int64_t n_tokens;
  float eta;
  float* ws;             // [Hkv, n_wg, d, d] the runs' partial Gram matrices
  float* ws_sum;         // [Hkv, 2 d R] S1 [d][R] then a copy of B [d][r] (R = rank padded to 16)
  int n_wg;              // gram workgroups (runs of tokens) per kv head
};
// Oja updates of at most this many tokens per head (a decode step's) run as
// a single launch that needs no workspace.
constexpr int kOjaSmallTokens = 64;
// Tokens per step of a gram workgroup.
constexpr int kOjaGramStep = 128;
// Oja workspace layout: per head and gram workgroup, the partial Gram
// matrix [d][d]; then per head S1 [d][R] (R = rank padded to whole
// 16-column blocks) and a copy of the basis before the step [d][r].
__host__ __device__ inline int64_t oja_head_floats(int d, int r_pad) { return 2 * (int64_t)d * r_pad; }
inline int oja_rank_pad(int rank) { return 16 * ((rank + 15) / 16); }
inline size_t oja_partial_floats(int hkv, int d, int n_wg) { return (size_t)hkv * n_wg * d * d; }
inline size_t oja_workspace_floats(int hkv, int d, int rank, int n_wg) {
  return oja_partial_floats(hkv, d, n_wg) + (size_t)hkv * oja_head_floats(d, oja_rank_pad(rank));
}
hipError_t launch_oja_update(const OjaArgs& a, hipStream_t s);

hipError_t launch_split_bf16(const SplitArgs& a, hipStream_t s);
// the same attention with the merge in the launch (a.merge_cnt set)
hipError_t launch_split_bf16_merged(const SplitArgs& a, hipStream_t s);
// Hybrid cache: low-rank rows (lr) and full-rank side list (side) in one
// launch of wgs_per_unit workgroups per (b, kv head), divided between the two
// lists on the device from the counts there.  Partials go to lr.part_o /
// lr.part_ml with lr.n_parts = wgs_per_unit; launch_merge combines them.
hipError_t launch_split_bf16_hybrid(const SplitArgs& lr, const SplitArgs& side, int wgs_per_unit, hipStream_t s);
hipError_t launch_compress_kv_small_bf16(const CompressKvArgs& a, hipStream_t s);
hipError_t launch_split_f32(const SplitArgs& a, hipStream_t s);
// Latent queries (basis_k and basis_v null, q [B, Hq, rk], partials rv wide).
hipError_t launch_split_bf16_latent(const SplitArgs& a, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, bool bf16, hipStream_t s);
hipError_t launch_compress_bf16(const CompressArgs& a, hipStream_t s);
// Keys and values of the same tokens in one launch (same batch, heads, d, tokens).
hipError_t launch_compress_pair_bf16(const CompressArgs& k, const CompressArgs& v, hipStream_t s);
hipError_t launch_compress_f32(const CompressArgs& a, hipStream_t s);

struct HybridArgs {
  const void* k; const void* v; const void* bk; const void* bv;
  float tau2;
  void* ck; void* cv; int32_t* n_lr;
  void* k_side; void* v_side; int32_t* side_idx; int32_t* n_side;
  uint8_t* flags; int32_t* overflow;
  int batch, hkv, d, rk, rv;
  int64_t n_tokens, pos, cap, side_cap;
  uint8_t* ws_flags;     // [B, Hkv, n_tiles * kHybridTile]
  int32_t* ws_counts;    // [B, Hkv, n_tiles] flagged tokens per sub-tile
  int32_t* ws_offsets;   // [B, Hkv, n_tiles, 2] (low-rank row, side row) of each sub-tile's first token
  int n_tiles;
  int cus;               // compute units of the device (sizes the persistent grids)
};

constexpr int kHybridTile = 16;   // tokens per hybrid compaction unit (one wave sub-tile)
hipError_t launch_hybrid_bf16(const HybridArgs& a, hipStream_t s);

}  // namespace lrkv
