// Debug check of the operator's input preconditions for gfx950.
//
// The compute entry points take the gate in log space with alpha in (0, 1]
// ("Kimi Linear" review, section "The KDA State Update Equation": a decay
// per channel in [0, 1]; the gate arrives as its natural logarithm, so it
// must be finite and <= 0), finite q, k, v and beta, and a packed layout
// with cu_seqlens rising from 0 to T. The device cannot report a violation
// synchronously, so these are documented rather than checked; this pass
// checks them on request and ORs one bit per kind of violation into a word
// in device memory.
//
// Bandwidth bound: one read of q, k, v, log alpha and beta as 16-byte
// vectors, a grid-stride loop, one ballot per wave and at most one atomic OR
// per wave that found something.
#include <algorithm>

#include "kda_device.h"

namespace kda {

namespace {

constexpr int kCheckThreads = 256;
constexpr int kCheckBlocks = 2048;   // eight waves per SIMD over 256 CUs

// Flag bits (the values of KDA_BAD_* in kda.h).
constexpr int32_t kBadQKV = 1, kBadGate = 2, kBadBeta = 4, kBadCu = 8;

__device__ __forceinline__ bool finite_f(float x) { return __builtin_isfinite(x); }

__device__ __forceinline__ bool finite8(const bf16* p) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
  bool ok = true;
#pragma unroll
  for (int e = 0; e < 8; ++e) ok &= finite_f((float)v[e]);
  return ok;
}
__device__ __forceinline__ bool finite8(const float* p) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  return finite_f(a.x) && finite_f(a.y) && finite_f(a.z) && finite_f(a.w) && finite_f(b.x) &&
         finite_f(b.y) && finite_f(b.z) && finite_f(b.w);
}
// Eight gates, each finite and <= 0 (NaN fails the comparison; -inf, which
// is alpha = 0, fails the finiteness test).
__device__ __forceinline__ bool gates_ok8(const float* p) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  bool ok = true;
#pragma unroll
  for (int e = 0; e < 8; ++e) ok = ok && x[e] <= 0.f && finite_f(x[e]);
  return ok;
}

__global__ void clear_flags_kernel(int32_t* flags) { flags[0] = 0; }

// n8: number of 8-element groups of q (= of k, v, log alpha); nb: beta
// elements. Block 0 also checks cu_seqlens (n_seqs + 1 entries).
template <class IO>
__global__ __launch_bounds__(kCheckThreads) void check_inputs_kernel(
    const IO* __restrict__ q, const IO* __restrict__ k, const IO* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, int32_t n_seqs, int64_t T, int64_t n8, int64_t nb,
    int32_t* flags) {
  int32_t bad = 0;
  const int64_t stride = (int64_t)gridDim.x * kCheckThreads;
  for (int64_t i = (int64_t)blockIdx.x * kCheckThreads + threadIdx.x; i < n8; i += stride) {
    if (!(finite8(q + 8 * i) && finite8(k + 8 * i) && finite8(v + 8 * i))) bad |= kBadQKV;
    if (!gates_ok8(log_alpha + 8 * i)) bad |= kBadGate;
  }
  for (int64_t i = (int64_t)blockIdx.x * kCheckThreads + threadIdx.x; i < nb; i += stride)
    if (!finite_f(beta[i])) bad |= kBadBeta;
  if (cu != nullptr && blockIdx.x == 0) {
    for (int n = threadIdx.x; n <= n_seqs; n += kCheckThreads) {
      const int64_t c = cu[n];
      if ((n == 0 && c != 0) || (n == n_seqs && c != T) || c < 0 || c > T ||
          (n < n_seqs && (int64_t)cu[n + 1] < c))
        bad |= kBadCu;
    }
  }
  // one atomic per wave that found anything
#pragma unroll
  for (int bit = 0; bit < 4; ++bit) {
    const int32_t m = 1 << bit;
    if (__builtin_amdgcn_ballot_w64((bad & m) != 0) != 0 && (threadIdx.x & 63) == 0)
      atomicOr(flags, m);
  }
}

}  // namespace

hipError_t launch_check_inputs(bool bf16_io, const void* q, const void* k, const void* v,
                               const float* log_alpha, const float* beta, const int32_t* cu,
                               int32_t n_seqs, int64_t T, int32_t H, int32_t* flags,
                               hipStream_t stream) {
  clear_flags_kernel<<<1, 1, 0, stream>>>(flags);
  const int64_t n8 = T * H * (kD / 8), nb = T * H;
  const int64_t need = (std::max<int64_t>(n8, nb) + kCheckThreads - 1) / kCheckThreads;
  const unsigned blocks = (unsigned)std::max<int64_t>(1, std::min<int64_t>(kCheckBlocks, need));
  if (bf16_io)
    check_inputs_kernel<bf16><<<blocks, kCheckThreads, 0, stream>>>(
        (const bf16*)q, (const bf16*)k, (const bf16*)v, log_alpha, beta, cu, n_seqs, T, n8, nb,
        flags);
  else
    check_inputs_kernel<float><<<blocks, kCheckThreads, 0, stream>>>(
        (const float*)q, (const float*)k, (const float*)v, log_alpha, beta, cu, n_seqs, T, n8,
        nb, flags);
  return hipGetLastError();
}

}  // namespace kda
