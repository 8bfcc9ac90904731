// Device-side helpers for the gfx950 KDA kernels: element types, MFMA
// wrappers and the fragment conventions shared by the prefill kernels.
//
// Matrix-core conventions (CDNA 16x16 MFMA, wave64). For an output tile
// D (16 x 16) += A (16 x K) * B (K x 16):
//   * a lane l = r + 16 g (r < 16, g < 4) supplies, for one 32-wide slice of
//     K, eight A values from row r and eight B values from column r, both at
//     the same eight k positions. Which eight k positions a lane group g
//     covers only has to agree between A and B; the kernels use two orders:
//       standard  k = 8 g + e                      (e < 8)
//       split     k = 4 g + e (e < 4), 16 + 4 g + (e - 4) (e >= 4)
//     The split order is what two stacked 16-row accumulator tiles already
//     hold per lane, so an accumulator pair feeds the next product as a B
//     operand without a trip through LDS.
//   * the accumulator gives lane l the four values D[4 g + e][r], e < 4.
// bf16 operands use one v_mfma_f32_16x16x32_bf16 per 32-wide slice; fp32
// operands use eight v_mfma_f32_16x16x4_f32, one per slot e.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;     // head dimension d_k = d_v
constexpr int kC = 64;      // chunk length
constexpr int kWave = 64;   // wavefront size

// Operand fragment: eight K-slots of one lane.
template <class E>
struct Frag;
template <>
struct Frag<bf16> {
  bf16x8 v;
  __device__ void set(int e, float x) { v[e] = (bf16)x; }
  __device__ float get(int e) const { return (float)v[e]; }
};
template <>
struct Frag<float> {
  float v[8];
  __device__ void set(int e, float x) { v[e] = x; }
  __device__ float get(int e) const { return v[e]; }
};

__device__ __forceinline__ floatx4 mma(floatx4 acc, const Frag<bf16>& a,
                                       const Frag<bf16>& b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mma(floatx4 acc, const Frag<float>& a,
                                       const Frag<float>& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// One 16x16x4 fp32 step, for the small fp32 products of the UT transform.
__device__ __forceinline__ floatx4 mma4(floatx4 acc, float a, float b) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

// Operand fragment of a K = 16 product: lane (r, g) supplies A[r][4 g + e]
// and B[4 g + e][r], e < 4. This is also the accumulator layout, so an
// accumulator tile of X is a ready B operand (and an A operand of X^T) for a
// product that contracts over X's rows.
template <class E>
struct Frag16;
template <>
struct Frag16<bf16> {
  bf16x4 v;
  __device__ void set(int e, float x) { v[e] = (bf16)x; }
  __device__ float get(int e) const { return (float)v[e]; }
};
template <>
struct Frag16<float> {
  float v[4];
  __device__ void set(int e, float x) { v[e] = x; }
  __device__ float get(int e) const { return v[e]; }
};

__device__ __forceinline__ floatx4 mma16(floatx4 acc, const Frag16<bf16>& a,
                                         const Frag16<bf16>& b) {
  typedef short short4_t __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, a.v),
                                                   __builtin_bit_cast(short4_t, b.v), acc, 0,
                                                   0, 0);
}
__device__ __forceinline__ floatx4 mma16(floatx4 acc, const Frag16<float>& a,
                                         const Frag16<float>& b) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], acc, 0, 0, 0);
  return acc;
}

// 16 x 16 fp32 product C = A B from accumulator tiles: `at` holds A^T and
// `b` holds B in the accumulator layout; C comes back in that layout.
__device__ __forceinline__ floatx4 mm16(floatx4 at, floatx4 b) {
  floatx4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(at[s], b[s], c, 0, 0, 0);
  return c;
}

template <class E>
__device__ __forceinline__ Frag16<E> frag16(floatx4 x) {
  Frag16<E> f;
#pragma unroll
  for (int e = 0; e < 4; ++e) f.set(e, x[e]);
  return f;
}

// Two K = 16 fragments as the two halves of a split-order K = 32 fragment.
__device__ __forceinline__ Frag<bf16> join(const Frag16<bf16>& lo, const Frag16<bf16>& hi) {
  Frag<bf16> f;
  f.v = __builtin_shufflevector(lo.v, hi.v, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
__device__ __forceinline__ Frag<float> join(const Frag16<float>& lo, const Frag16<float>& hi) {
  Frag<float> f;
#pragma unroll
  for (int e = 0; e < 4; ++e) { f.v[e] = lo.v[e]; f.v[4 + e] = hi.v[e]; }
  return f;
}

// Four consecutive I/O elements, kept in their I/O type.
__device__ __forceinline__ Frag16<bf16> ld16(const bf16* p) {
  Frag16<bf16> f;
  f.v = *reinterpret_cast<const bf16x4*>(p);
  return f;
}
__device__ __forceinline__ Frag16<float> ld16(const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  Frag16<float> f;
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  return f;
}
__device__ __forceinline__ void st16(bf16* p, const Frag16<bf16>& f) {
  *reinterpret_cast<bf16x4*>(p) = f.v;
}
__device__ __forceinline__ void st16(float* p, const Frag16<float>& f) {
  *reinterpret_cast<float4*>(p) = float4{f.v[0], f.v[1], f.v[2], f.v[3]};
}


// Cross-lane sums inside a wave (results in every lane).
// Sum over lanes l and l ^ 16: permlane16_swap with both operands x gives
// each lane x from its own 16-lane row and from the partner row.
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Sum over lanes l and l ^ 32 (permlane32_swap, same construction).
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The pages' L2Norm of q and k: x / sqrt(sum_c x_c^2 + kL2NormEps).
constexpr float kL2NormEps = 1e-6f;

// e^x through the hardware base-2 exponential.
__device__ __forceinline__ float exp_f(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// I/O element conversions.
__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <class T>
__device__ __forceinline__ T from_f(float x);
template <>
__device__ __forceinline__ float from_f<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }

// Loads 8 consecutive I/O elements as floats (16 B for bf16, 32 B for fp32).
__device__ __forceinline__ void load8(const bf16* p, float* out) {
  bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = (float)v[e];
}
__device__ __forceinline__ void load8(const float* p, float* out) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}
// Loads 4 consecutive I/O elements as floats.
__device__ __forceinline__ void load4(const bf16* p, float* out) {
  bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = (float)v[e];
}
__device__ __forceinline__ void load4(const float* p, float* out) {
  float4 a = *reinterpret_cast<const float4*>(p);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
}

// Stores a fragment's eight elements contiguously (LDS rows).
__device__ __forceinline__ void store8(bf16* p, const Frag<bf16>& f) {
  *reinterpret_cast<bf16x8*>(p) = f.v;
}
__device__ __forceinline__ void store8(float* p, const Frag<float>& f) {
  reinterpret_cast<float4*>(p)[0] = float4{f.v[0], f.v[1], f.v[2], f.v[3]};
  reinterpret_cast<float4*>(p)[1] = float4{f.v[4], f.v[5], f.v[6], f.v[7]};
}

// Fragment stores / loads in the lane-major workspace layout.
__device__ __forceinline__ void store_frag(bf16* base, int lane, const Frag<bf16>& f) {
  *reinterpret_cast<bf16x8*>(base + lane * 8) = f.v;
}
__device__ __forceinline__ void store_frag(float* base, int lane, const Frag<float>& f) {
  float4* p = reinterpret_cast<float4*>(base + lane * 8);
  p[0] = float4{f.v[0], f.v[1], f.v[2], f.v[3]};
  p[1] = float4{f.v[4], f.v[5], f.v[6], f.v[7]};
}
// Writes four accumulator values into slots 4*half .. 4*half+3 of a lane's
// fragment record (the other half belongs to another wave).
__device__ __forceinline__ void store_half_frag(bf16* base, int lane, int half, floatx4 x) {
  bf16x4 v;
  v[0] = (bf16)x[0]; v[1] = (bf16)x[1]; v[2] = (bf16)x[2]; v[3] = (bf16)x[3];
  *reinterpret_cast<bf16x4*>(base + lane * 8 + 4 * half) = v;
}
__device__ __forceinline__ void store_half_frag(float* base, int lane, int half, floatx4 x) {
  *reinterpret_cast<float4*>(base + lane * 8 + 4 * half) = float4{x[0], x[1], x[2], x[3]};
}
__device__ __forceinline__ void load_frag(const bf16* base, int lane, Frag<bf16>& f) {
  f.v = *reinterpret_cast<const bf16x8*>(base + lane * 8);
}
__device__ __forceinline__ void load_frag(const float* base, int lane, Frag<float>& f) {
  const float4* p = reinterpret_cast<const float4*>(base + lane * 8);
  float4 a = p[0], b = p[1];
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
__device__ __forceinline__ void store_c4(bf16* base, int lane, floatx4 x) {
  bf16x4 v;
  v[0] = (bf16)x[0]; v[1] = (bf16)x[1]; v[2] = (bf16)x[2]; v[3] = (bf16)x[3];
  *reinterpret_cast<bf16x4*>(base + lane * 4) = v;
}
__device__ __forceinline__ void store_c4(float* base, int lane, floatx4 x) {
  *reinterpret_cast<float4*>(base + lane * 4) = float4{x[0], x[1], x[2], x[3]};
}
// Four consecutive I/O elements from an accumulator (8 B bf16, 16 B fp32).
__device__ __forceinline__ void store4_io(bf16* p, floatx4 x) {
  bf16x4 v;
  v[0] = (bf16)x[0]; v[1] = (bf16)x[1]; v[2] = (bf16)x[2]; v[3] = (bf16)x[3];
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void store4_io(float* p, floatx4 x) {
  *reinterpret_cast<float4*>(p) = float4{x[0], x[1], x[2], x[3]};
}
__device__ __forceinline__ floatx4 load_c4(const bf16* base, int lane) {
  bf16x4 v = *reinterpret_cast<const bf16x4*>(base + lane * 4);
  return floatx4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ floatx4 load_c4(const float* base, int lane) {
  float4 v = *reinterpret_cast<const float4*>(base + lane * 4);
  return floatx4{v.x, v.y, v.z, v.w};
}

// Split-order K index of slot e for lane group g inside a 32-wide slice.
__device__ __forceinline__ int split_k(int g, int e) {
  return e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4);
}

// Per-(chunk, head) intermediate block: element counts and offsets (in E).
constexpr int kXAElems = 8 * 4 * kWave * 8;   // [-W ; Qt] A-fragments
constexpr int kKTElems = 8 * 2 * kWave * 8;   // K'^T A-fragments
constexpr int kUCElems = 8 * 8 * kWave * 4;   // [U ; Ut] C-fragments
constexpr int kGCFloats = kD;                 // gamma_C
template <class E>
struct Inter {
  static constexpr size_t kXA = 0;
  static constexpr size_t kKT = kXA + kXAElems;
  static constexpr size_t kUC = kKT + kKTElems;
  static constexpr size_t kBytes = (kUC + kUCElems) * sizeof(E) + kGCFloats * sizeof(float);
  static constexpr size_t kGCByte = (kUC + kUCElems) * sizeof(E);
};

}  // namespace kda
