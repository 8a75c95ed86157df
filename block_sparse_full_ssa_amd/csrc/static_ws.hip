// ssa_attn_fwd_noalloc: the layer forward for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, hosts
// that forbid allocation).  It runs exactly the kernels of ssa_attn_fwd; the
// workspace those kernels use comes from a file-scope device array instead
// of a caller buffer.
//
// Each device that the library runs on holds its own copy of the array, at
// its own address, until the process ends.  The address is looked up once
// per device, with that device current, on the first call there that needs
// workspace; host code then passes that device address to the kernels (the
// array's name on the host is only a stand-in for the symbol).  Nothing in
// the forward's workspace has to start at zero: every word is written before
// it is read within one call.  All calls on one device share the array, so
// calls that overlap in time on one device (different streams or threads)
// race on it.

#include <mutex>

#include "ssa.h"
#include "internal.h"

namespace ssa {
namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(16) << 20;   // 16 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace ssa

extern "C" {

size_t ssa_noalloc_scratch_bytes(void) { return ssa::kScratchBytes; }

ssa_status_t ssa_attn_fwd_noalloc(const ssa_shape_t* shape, int32_t mode, const void* q, const void* k,
                                  const void* v, const int32_t* sel, void* h_full, void* h_sparse,
                                  float* lse_full, float* lse_sparse, float* delta, float* losses,
                                  void* stream) {
  // an invalid shape or mode sizes to 0 here and is reported by ssa_attn_fwd
  const size_t need = ssa_workspace_size(shape, mode, SSA_OP_FWD);
  if (need > ssa::kScratchBytes) {
    char msg[200];
    snprintf(msg, sizeof(msg),
             "this layer needs %zu bytes of workspace; ssa_attn_fwd_noalloc holds %zu (use ssa_attn_fwd)", need,
             ssa::kScratchBytes);
    ssa::set_last_error(msg);
    return SSA_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = ssa::scratch_address(&ws);
    if (e != hipSuccess) {
      char msg[200];
      snprintf(msg, sizeof(msg), "device address of the static workspace: %s", hipGetErrorString(e));
      ssa::set_last_error(msg);
      return SSA_ERR_HIP;
    }
  }
  ssa::TimingPause no_events;     // the timing hooks would create HIP events
  return ssa_attn_fwd(shape, mode, q, k, v, sel, h_full, h_sparse, lse_full, lse_sparse, delta, losses, ws,
                      need > 0 ? ssa::kScratchBytes : 0, stream);
}

}  // extern "C"
