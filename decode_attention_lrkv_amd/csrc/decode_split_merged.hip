// The low-rank attention kernel of the plain and step decode calls in the
// form that merges its own partials (gfx950): the partials are stored with
// device scope and the last workgroup of each (b, kv head) merges them in
// the launch (merge_in_launch), so there is no merge launch.  The host
// chooses it for launches far smaller than the chip (batch-1 decodes), where
// the second launch is a large part of a layer's time.  A translation unit
// of its own so that it compiles in parallel with the others.
#include "decode_body.h"

namespace lrkv {

namespace {

template <int KC, int VB, bool EARLY>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void split_bf16_merged_kernel(SplitArgs a) {
  __shared__ SplitSmem sm;
  split_bf16_body<KC, VB, true, kStages<KC, VB>, false, EARLY, true>(a, blockIdx.x, blockIdx.x, sm,
                                                                     a.k_new != nullptr && blockIdx.x == gridDim.x - 1);
  merge_in_launch(a, (int64_t)blockIdx.z * a.hkv + blockIdx.y, gridDim.x);
}

}  // namespace

#define LRKV_MERGED_CASE(KC, VB)                                                                   \
  case (KC * 16 + VB):                                                                             \
    if (early)                                                                                     \
      hipLaunchKernelGGL((split_bf16_merged_kernel<KC, VB, true>), grid, dim3(256), 0, s, a);      \
    else                                                                                           \
      hipLaunchKernelGGL((split_bf16_merged_kernel<KC, VB, false>), grid, dim3(256), 0, s, a);     \
    break;

hipError_t launch_split_bf16_merged(const SplitArgs& a, hipStream_t s) {
  const dim3 grid(a.k_new ? a.n_parts - 1 : a.n_parts, a.hkv, a.batch);
  const int kc = (a.rk + 31) / 32, vb = (a.rv + 15) / 16;
  // no instantiation with a separate key encoder or final outputs
  if (a.basis_k == nullptr || a.basis_v == nullptr || a.enc_k || a.out || !a.merge_cnt || !a.merge_out)
    return hipErrorInvalidValue;
  const bool early = a.chunks_per_split >= 2;
  switch (kc * 16 + vb) {
    LRKV_MERGED_CASE(1, 1) LRKV_MERGED_CASE(1, 2) LRKV_MERGED_CASE(1, 3) LRKV_MERGED_CASE(1, 4)
    LRKV_MERGED_CASE(1, 5) LRKV_MERGED_CASE(1, 6) LRKV_MERGED_CASE(1, 7) LRKV_MERGED_CASE(1, 8)
    LRKV_MERGED_CASE(2, 1) LRKV_MERGED_CASE(2, 2) LRKV_MERGED_CASE(2, 3) LRKV_MERGED_CASE(2, 4)
    LRKV_MERGED_CASE(2, 5) LRKV_MERGED_CASE(2, 6) LRKV_MERGED_CASE(2, 7) LRKV_MERGED_CASE(2, 8)
    LRKV_MERGED_CASE(3, 1) LRKV_MERGED_CASE(3, 2) LRKV_MERGED_CASE(3, 3) LRKV_MERGED_CASE(3, 4)
    LRKV_MERGED_CASE(3, 5) LRKV_MERGED_CASE(3, 6) LRKV_MERGED_CASE(3, 7) LRKV_MERGED_CASE(3, 8)
    LRKV_MERGED_CASE(4, 1) LRKV_MERGED_CASE(4, 2) LRKV_MERGED_CASE(4, 3) LRKV_MERGED_CASE(4, 4)
    LRKV_MERGED_CASE(4, 5) LRKV_MERGED_CASE(4, 6) LRKV_MERGED_CASE(4, 7) LRKV_MERGED_CASE(4, 8)
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lrkv
