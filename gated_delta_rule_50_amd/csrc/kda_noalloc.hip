// Allocation-free prefill entry point: kda_chunk_fwd with its workspace in a
// file-scope device array instead of caller memory, for callers that cannot
// allocate (code under HIP graph capture, serving loops, harnesses that
// forbid hipMalloc). Same kernels, same arguments otherwise.
//
// The array `scratch` exists once per GPU the library runs on, for the life
// of the process. In host code its name is only a host-side stand-in: the
// device address comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that address is ever passed to a kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "kda.h"

namespace {

static __device__ __align__(256) uint8_t scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch`, or NULL on a HIP error.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" kda_status kda_chunk_fwd_noalloc(
    const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
    const void* h0, const int32_t* cu_seqlens, int32_t n_seqs, int64_t total_tokens,
    int32_t heads, int32_t dk, int32_t dv, kda_io_dtype io, uint32_t flags, void* o,
    void* h_final, void* stream) {
  // the size check is host arithmetic only: a call beyond the array is
  // refused before any HIP call. The prefill runs over windows of chunk
  // slots sized to the workspace, so the array only has to hold one slot.
  const size_t need =
      kda_chunk_fwd_workspace_min_bytes(n_seqs, total_tokens, heads, dk, dv, io);
  if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_SCRATCH;
  void* ws = scratch_ptr();
  if (ws == nullptr) return KDA_ERR_HIP;
  return kda_chunk_fwd(q, k, v, log_alpha, beta, h0, cu_seqlens, n_seqs, total_tokens, heads,
                       dk, dv, io, flags, o, h_final, ws, (size_t)KDA_NOALLOC_SCRATCH_BYTES,
                       stream);
}
