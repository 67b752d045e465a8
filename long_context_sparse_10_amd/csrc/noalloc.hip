// sparse_mqa_attend_noalloc: sparse_mqa_attend for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The split-softmax partials go to a fixed
// scratch array of CSA_NOALLOC_SCRATCH_BYTES in the library's own device
// memory: one copy per GPU, held until the process ends.  Its device address
// is looked up once per device, with that device current, and kept; host code
// uses only that address.
#include <mutex>

#include "common.hpp"
#include "internal.hpp"

using namespace csa;

namespace {

constexpr int kMaxDevices = 64;

// In host code this name is a host-side stand-in, not the array's device
// address: only the lookup below may name it.
static __device__ __align__(256) unsigned char scratch[CSA_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// device address of the current device's copy of `scratch`
csa_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CSA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return CSA_ERR_LAUNCH;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return CSA_OK;
}

}  // namespace

extern "C" {

csa_status sparse_mqa_attend_noalloc(const void* q, csa_dtype q_t, const float* q_norm_w,
                                     float eps, int rope_dims, float rope_theta,
                                     const int32_t* q_pos, const void* kv, csa_dtype kv_t,
                                     int Nmax, const int32_t* idx, int k, const void* win,
                                     int win_len, int n_win, const float* sink, float scale,
                                     int B, int Tq, int nh, int c, void* out, csa_dtype out_t,
                                     hipStream_t stream) {
  if (idx == nullptr) return CSA_ERR_INVALID;
  AttendArgs a{q, q_t, q_norm_w, eps, rope_dims, rope_theta, q_pos, kv, kv_t, Nmax, idx, k,
               nullptr, 0, win, win_len, n_win, sink, scale, B, Tq, nh, c, out, out_t, kDense};
  const csa_status st = check_attend(a);
  if (st != CSA_OK) return st;
  // the partials of this call (bytes of sparse_mqa_attend's workspace)
  if (attend_workspace(a) > CSA_NOALLOC_SCRATCH_BYTES) return CSA_ERR_WORKSPACE;
  // set-up on every call, so that an empty call (B == 0) before a graph
  // capture does it outside the capture
  void* ws = nullptr;
  const csa_status sa = scratch_address(&ws);
  if (sa != CSA_OK) return sa;
  if (a.B == 0 || a.Tq == 0) return CSA_OK;
  return launch_attend(a, ws, stream) == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}

}  // extern "C"
