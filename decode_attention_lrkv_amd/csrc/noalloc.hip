// Decode step without a caller-provided workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// The workspace of lrkv_decode_step (per-workgroup partial results: running
// max, softmax sum and an unnormalised head_dim-wide output per query head)
// lives in a fixed device array of this library instead.  Each GPU holds its
// own copy at its own address; the host looks that address up once per device
// with hipGetSymbolAddress and passes it to the kernels like any workspace.
// The array keeps the last call's contents.  Its first bytes are the step's
// per-(b, kv head) arrival counters, which launches that merge their partials
// in the same launch need at zero: a device global without an initialiser is
// zero-filled when the code object loads, and every call leaves the counters
// zero, so nothing is cleared (the partials behind them need no initial
// contents).  Calls on one GPU share the array, so calls that overlap in time
// on one GPU (different streams, or different threads without ordering) race.
#include <mutex>

#include "lrkv.h"
#include "lrkv_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(8) << 20;   // 8 MiB per GPU

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch array (looked up on the first call on
// the device, with that device current), or null with *err set.
void* scratch_on_current_device(hipError_t* err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  *err = hipSuccess;
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t lrkv_decode_step_noalloc_max_bytes(void) { return kScratchBytes; }

lrkv_status lrkv_decode_step_noalloc(const void* q, const void* k_new, const void* v_new, const void* basis_k,
                                     void* coeff_k, const void* basis_v, void* coeff_v, const void* enc_k, void* out,
                                     float* lse, const lrkv_dims* dims, int64_t n_ctx, float scale, lrkv_dtype dtype,
                                     hipStream_t stream) {
  const char* fn = "lrkv_decode_step_noalloc";
  if (!dims) return lrkv::fail(LRKV_ERR_INVALID_ARGUMENT, "%s: dims is NULL", fn);
  // every argument is checked again by lrkv_decode_step; the size check comes
  // first so that an oversized call is refused before any device call
  const size_t need = lrkv_decode_step_workspace_bytes(dims, n_ctx);
  if (need == 0)
    return lrkv::fail(LRKV_ERR_INVALID_ARGUMENT, "%s: invalid dims or n_ctx = %lld", fn, (long long)n_ctx);
  if (need > kScratchBytes)
    return lrkv::fail(LRKV_ERR_WORKSPACE_TOO_SMALL,
                     "%s: these dims need %zu bytes of workspace, more than the library's fixed %zu; "
                     "use lrkv_decode_step with a workspace",
                     fn, need, kScratchBytes);
  hipError_t e = hipSuccess;
  void* ws = scratch_on_current_device(&e);
  if (!ws)
    return lrkv::fail(LRKV_ERR_DEVICE, "%s: address of the scratch array: %s", fn, hipGetErrorString(e));
  return lrkv_decode_step(q, k_new, v_new, basis_k, coeff_k, basis_v, coeff_v, enc_k, out, lse, dims, n_ctx, scale,
                          dtype, ws, kScratchBytes, stream);
}

}  // extern "C"
