// Output epilogue for gfx950: head-wise RMSNorm times a sigmoid gate.
//
//   y = sigmoid(g) * o / sqrt(mean_j o_j^2 + eps) * w
// per (token, head) row of d_v = 128 channels ("Kimi Linear" review,
// section "Neural Parameterization", output gate equation: a head-wise
// RMSNorm and a data-dependent sigmoid gate before the output projection;
// the "L2 Deep Distill" page fuses the two as FusedRMSNormGated).
//
// Bandwidth bound (three 128-channel rows moved per row of output, a few
// flops per element). Sixteen lanes own one row, eight channels each
// (16-byte bf16 accesses); the row's sum of squares is a DPP sum over the
// lanes of one 16-lane DPP row, so a row never leaves its lane group and a
// 256-thread block covers 16 rows.
#include <algorithm>

#include "kda_device.h"

namespace kda {

namespace {

__device__ __forceinline__ float dpp_sum16(float x) {
  // rotate by 8 and 4 inside the 16-lane row, then the two quad swaps
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));
  return x;
}

__device__ __forceinline__ void store8_io(bf16* p, const float* x) {
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (bf16)x[e];
  *reinterpret_cast<bf16x8*>(p) = v;
}
__device__ __forceinline__ void store8_io(float* p, const float* x) {
  reinterpret_cast<float4*>(p)[0] = float4{x[0], x[1], x[2], x[3]};
  reinterpret_cast<float4*>(p)[1] = float4{x[4], x[5], x[6], x[7]};
}

}  // namespace

// o and y may be the same buffer: every element is read and written by the
// same lane, the read first. Groups of 16 rows are strided over the grid, so
// the launch stays within the 32-bit grid size for any row count.
template <class IO>
__global__ __launch_bounds__(256) void rmsnorm_gate_kernel(const IO* o, const IO* __restrict__ g,
                                                           const float* __restrict__ w,
                                                           float eps, int64_t rows, IO* y) {
  const int c0 = (threadIdx.x & 15) * 8;
  float wv[8];
  if (w != nullptr) {
    const float4 a = *reinterpret_cast<const float4*>(w + c0);
    const float4 b = *reinterpret_cast<const float4*>(w + c0 + 4);
    wv[0] = a.x; wv[1] = a.y; wv[2] = a.z; wv[3] = a.w;
    wv[4] = b.x; wv[5] = b.y; wv[6] = b.z; wv[7] = b.w;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) wv[e] = 1.f;
  }
  const int64_t stride = (int64_t)gridDim.x * 16;
  for (int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4); row < rows; row += stride) {
    // whole 16-lane groups run the same iterations
    const int64_t base = row * kD + c0;
    float x[8], gv[8];
    load8(o + base, x);
    load8(g + base, gv);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
    ss = dpp_sum16(ss);
    // hardware reciprocal and reciprocal square root (about 1 ulp each, far
    // below the output's rounding): correctly rounded divisions would double
    // the kernel's instruction count
    const float r = __builtin_amdgcn_rsqf(ss * (1.f / kD) + eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sg = __builtin_amdgcn_rcpf(1.f + exp_f(-gv[e]));
      x[e] = x[e] * r * wv[e] * sg;
    }
    store8_io(y + base, x);
  }
}

hipError_t launch_rmsnorm_gate(bool bf16_io, const void* o, const void* g, const float* w,
                               float eps, int64_t rows, void* y, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  // one group of 16 rows per block up to 8192 blocks (32 k waves, far more
  // than the 256 CUs hold at once), then grid-stride: the grid stays small
  // for any row count
  constexpr int64_t kMaxBlocks = 8192;
  const int64_t blocks = std::min((rows + 15) / 16, kMaxBlocks);
  if (bf16_io)
    rmsnorm_gate_kernel<bf16><<<(unsigned)blocks, 256, 0, stream>>>(
        (const bf16*)o, (const bf16*)g, w, eps, rows, (bf16*)y);
  else
    rmsnorm_gate_kernel<float><<<(unsigned)blocks, 256, 0, stream>>>(
        (const float*)o, (const float*)g, w, eps, rows, (float*)y);
  return hipGetLastError();
}

}  // namespace kda
