// Achievable-rate probes for the roofline figures: what this GPU's memory
// system and matrix/vector units deliver to plain kernels, measured beside
// the operator's own kernels so their fractions can be read against both the
// published peaks and these measured ceilings.
//
//   kdab_read   streams a buffer in (16-byte loads, grid-stride)
//   kdab_copy   copies one buffer to another
//   kdab_rmw    updates a buffer in place (the decode step's access shape)
//   kdab_mfma   loops v_mfma_f32_16x16x32_bf16 on register operands
//   kdab_valu   loops fp32 FMAs on register operands (no packed forms)
//
// Every kernel keeps its accesses inside [buf, buf + bytes); the compute
// loops touch memory only through one store per lane into `sink` (256
// floats) under a condition the data never meets, which keeps the compiler
// from removing the loop. Returns 0, or -1 for arguments outside the stated
// ranges, or the HIP error code of the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;   // 16-byte accesses in flight per lane

template <bool NT>
__device__ __forceinline__ f4 ld(const f4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT>
__device__ __forceinline__ void st(f4* p, f4 x) {
  if constexpr (NT) __builtin_nontemporal_store(x, p);
  else *p = x;
}

__global__ __launch_bounds__(kThreads) void read_kernel(const f4* __restrict__ a, int64_t n4,
                                                        float* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t i = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; i < n4; i += stride) {
    f4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      x[u] = i + u * kThreads < n4 ? ld<true>(a + i + u * kThreads) : f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc += x[u];
  }
  if (acc.x == -1.2345e30f) sink[threadIdx.x] = acc.y;
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void copy_kernel(const f4* __restrict__ a,
                                                        f4* __restrict__ b, int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
  for (int64_t i = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; i < n4; i += stride) {
    f4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (i + u * kThreads < n4) x[u] = ld<NT>(a + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (i + u * kThreads < n4) st<NT>(b + i + u * kThreads, x[u]);
  }
}

__global__ __launch_bounds__(kThreads) void rmw_kernel(f4* __restrict__ a, int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
  for (int64_t i = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; i < n4; i += stride) {
    f4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (i + u * kThreads < n4) x[u] = ld<true>(a + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (i + u * kThreads < n4) st<true>(a + i + u * kThreads, x[u] * 0.5f + 0.25f);
  }
}

// Eight independent accumulators per wave cover the MFMA latency.
__global__ __launch_bounds__(kThreads) void mfma_kernel(int64_t iters, float seed,
                                                        float* __restrict__ sink) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(seed * (threadIdx.x + e));
    b[e] = (__bf16)(seed * (threadIdx.x - e));
  }
  floatx4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if (s == -1.2345e30f) sink[threadIdx.x] = s;
}

// Thirty-two independent FMA chains per lane.
constexpr int kChains = 32;
__global__ __launch_bounds__(kThreads) void valu_kernel(int64_t iters, float seed,
                                                        float* __restrict__ sink) {
  float x[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) x[j] = seed * (threadIdx.x + j);
  const float m = 1.f - seed, c = seed * 1e-3f;   // registers, not literals
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) x[j] = __builtin_fmaf(x[j], m, c);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j) s += x[j];
  if (s == -1.2345e30f) sink[threadIdx.x] = s;
}

bool bad_buffer(const void* p, int64_t bytes) {
  return p == nullptr || bytes <= 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(p) & 15);
}
bool bad_grid(int grid) { return grid < 1 || grid > (1 << 20); }
int status() { return (int)hipGetLastError(); }

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, buffer 16-byte aligned) once.
int kdab_read(const void* buf, int64_t bytes, float* sink, int grid, hipStream_t stream) {
  if (bad_buffer(buf, bytes) || sink == nullptr || bad_grid(grid)) return -1;
  read_kernel<<<grid, kThreads, 0, stream>>>(static_cast<const f4*>(buf), bytes / 16, sink);
  return status();
}

// Copies `bytes` from src to dst (non-overlapping); nontemporal != 0 uses
// streaming loads and stores.
int kdab_copy(const void* src, void* dst, int64_t bytes, int nontemporal, int grid,
              hipStream_t stream) {
  if (bad_buffer(src, bytes) || bad_buffer(dst, bytes) || bad_grid(grid)) return -1;
  const char* s = static_cast<const char*>(src);
  const char* d = static_cast<const char*>(dst);
  if (s < d + bytes && d < s + bytes) return -1;
  if (nontemporal)
    copy_kernel<true><<<grid, kThreads, 0, stream>>>(static_cast<const f4*>(src),
                                                     static_cast<f4*>(dst), bytes / 16);
  else
    copy_kernel<false><<<grid, kThreads, 0, stream>>>(static_cast<const f4*>(src),
                                                      static_cast<f4*>(dst), bytes / 16);
  return status();
}

// Reads and rewrites `bytes` in place with streaming accesses.
int kdab_rmw(void* buf, int64_t bytes, int grid, hipStream_t stream) {
  if (bad_buffer(buf, bytes) || bad_grid(grid)) return -1;
  rmw_kernel<<<grid, kThreads, 0, stream>>>(static_cast<f4*>(buf), bytes / 16);
  return status();
}

// grid workgroups of four waves, each wave issuing 8 * iters MFMAs of
// 16 x 16 x 32 (16,384 flops each).
int kdab_mfma(float* sink, int64_t iters, int grid, hipStream_t stream) {
  if (sink == nullptr || iters < 1 || bad_grid(grid)) return -1;
  mfma_kernel<<<grid, kThreads, 0, stream>>>(iters, 1e-3f, sink);
  return status();
}

// grid workgroups of 256 lanes, each lane issuing 32 * iters fp32 FMAs.
int kdab_valu(float* sink, int64_t iters, int grid, hipStream_t stream) {
  if (sink == nullptr || iters < 1 || bad_grid(grid)) return -1;
  valu_kernel<<<grid, kThreads, 0, stream>>>(iters, 1e-3f, sink);
  return status();
}

}  // extern "C"
