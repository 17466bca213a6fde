// The low-rank attention kernel of the plain and step decode calls (gfx950),
// in every (KC, VB) instantiation, each with and without the early
// prefetch of the second chunk; a translation unit of its own so that it
// compiles in parallel with the other kernels.
#include "decode_body.h"

namespace lrkv {

namespace {

// Low-rank keys: two waves per SIMD (one round of workgroups fills the chip).
// ENC: the appended key has its own encoder (a.enc_k), a separate
// instantiation so that the plain kernel carries none of its code.
// EARLY: both chunk buffers are loaded before the fold; chosen by the host
// when every wave has at least two chunks (with one chunk per wave there is
// no second chunk to prefetch, and the smaller kernel without it runs).
template <int KC, int VB, bool ENC, bool EARLY>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void split_bf16_kernel(SplitArgs a) {
  __shared__ SplitSmem sm;
  split_bf16_body<KC, VB, true, kStages<KC, VB>, ENC, EARLY>(a, blockIdx.x, blockIdx.x, sm,
                                                             a.k_new != nullptr && blockIdx.x == gridDim.x - 1);
}

}  // namespace

#define LRKV_SPLIT_CASE(KC, VB)                                                               \
  case (KC * 16 + VB):                                                                        \
    if (a.enc_k)                                                                              \
      hipLaunchKernelGGL((split_bf16_kernel<KC, VB, true, false>), grid, dim3(256), 0, s, a);  \
    else if (early)                                                                           \
      hipLaunchKernelGGL((split_bf16_kernel<KC, VB, false, true>), grid, dim3(256), 0, s, a);  \
    else                                                                                      \
      hipLaunchKernelGGL((split_bf16_kernel<KC, VB, false, false>), grid, dim3(256), 0, s, a); \
    break;

hipError_t launch_split_bf16(const SplitArgs& a, hipStream_t s) {
  // one workgroup per partial; with k_new set, the last workgroup of each
  // (b, kv head) also appends (adding the token to its own partial), and the
  // token's slot is the extra last one, left empty
  const dim3 grid(a.k_new ? a.n_parts - 1 : a.n_parts, a.hkv, a.batch);
  const int kc = (a.rk + 31) / 32, vb = (a.rv + 15) / 16;
  if (a.basis_k == nullptr || a.basis_v == nullptr || (a.enc_k && !a.k_new)) return hipErrorInvalidValue;
  if (a.merge_cnt) return launch_split_bf16_merged(a, s);   // decode_split_merged.hip
  // each wave takes chunks_per_split chunks (the plan for the bound when the
  // lengths are on the device, which never gives a wave more)
  const bool early = a.chunks_per_split >= 2;
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

}  // namespace lrkv
