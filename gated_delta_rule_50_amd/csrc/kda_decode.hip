// Single-token recurrent decode step for gfx950.
//
// Per (sequence, head) the step is the recurrence in the form of the review's
// "Online Learning Interpretation" ("Kimi Linear: An Expressive, Efficient
// Attention Architecture", paper-graph-ui review):
//   S~ = Diag(alpha) S,  e = S~^T k,  S <- S~ + beta k (v - e)^T,  o = S^T q.
// The readout on the updated state expands to
//   o = S~^T q + beta (q . k) (v - e),
// so both column reductions (e and S~^T q) come from ONE pass over S and the
// state is read once and written once. Decode is bandwidth bound: 64 KiB of
// fp32 state in and out per (sequence, head) against a few hundred bytes of
// token inputs.
//
// Layout: one 256-thread workgroup per (sequence, head). Thread t owns the
// column quad j = 4 (t % 32) .. +3 and the 16 rows c = t / 32 + 8 i, so every
// wave reads and writes two full 512-byte rows per instruction (16-byte
// accesses, fully coalesced). Partial sums over the eight row groups meet in
// LDS.
#include "kda_device.h"

namespace kda {

template <class IO>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const IO* __restrict__ q, const IO* __restrict__ k, const IO* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    float* __restrict__ S, IO* __restrict__ o) {
  const int64_t p = blockIdx.x;  // (sequence, head) pair
  const int t = threadIdx.x;
  const int jq = t & 31;         // column quad
  const int rg = t >> 5;         // row group: rows rg + 8 i

  __shared__ float s_k[kD], s_q[kD], s_a[kD], s_v[kD];
  __shared__ float4 s_pe[8][32], s_pp[8][32];
  __shared__ float s_qk[8];

  float4* Sp = reinterpret_cast<float4*>(S + p * (kD * kD));
  float4 s[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) s[i] = Sp[(rg + 8 * i) * 32 + jq];

  if (t < kD) {
    s_k[t] = to_f(k[p * kD + t]);
    s_q[t] = to_f(q[p * kD + t]);
    s_a[t] = expf(log_alpha[p * kD + t]);
  } else {
    s_v[t - kD] = to_f(v[p * kD + t - kD]);
  }
  __syncthreads();

  float4 pe = {0.f, 0.f, 0.f, 0.f}, pp = {0.f, 0.f, 0.f, 0.f};
  float qk = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = rg + 8 * i;
    const float a = s_a[c];
    const float ka = s_k[c] * a, qa = s_q[c] * a;
    pe.x += ka * s[i].x; pe.y += ka * s[i].y; pe.z += ka * s[i].z; pe.w += ka * s[i].w;
    pp.x += qa * s[i].x; pp.y += qa * s[i].y; pp.z += qa * s[i].z; pp.w += qa * s[i].w;
    qk += s_q[c] * s_k[c];
  }
  s_pe[rg][jq] = pe;
  s_pp[rg][jq] = pp;
  if (jq == 0) s_qk[rg] = qk;
  __syncthreads();

  float4 e = {0.f, 0.f, 0.f, 0.f}, pr = {0.f, 0.f, 0.f, 0.f};
  float qkt = 0.f;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const float4 a = s_pe[r][jq], b = s_pp[r][jq];
    e.x += a.x; e.y += a.y; e.z += a.z; e.w += a.w;
    pr.x += b.x; pr.y += b.y; pr.z += b.z; pr.w += b.w;
    qkt += s_qk[r];
  }
  const float b = beta[p];
  // d_j = beta (v_j - e_j): the correction written along k
  float4 d;
  d.x = b * (s_v[4 * jq + 0] - e.x);
  d.y = b * (s_v[4 * jq + 1] - e.y);
  d.z = b * (s_v[4 * jq + 2] - e.z);
  d.w = b * (s_v[4 * jq + 3] - e.w);

#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = rg + 8 * i;
    const float a = s_a[c], kc = s_k[c];
    float4 x;
    x.x = a * s[i].x + kc * d.x;
    x.y = a * s[i].y + kc * d.y;
    x.z = a * s[i].z + kc * d.z;
    x.w = a * s[i].w + kc * d.w;
    Sp[(rg + 8 * i) * 32 + jq] = x;
  }
  if (rg == 0) {
    IO* op = o + p * kD + 4 * jq;
    op[0] = from_f<IO>(pr.x + qkt * d.x);
    op[1] = from_f<IO>(pr.y + qkt * d.y);
    op[2] = from_f<IO>(pr.z + qkt * d.z);
    op[3] = from_f<IO>(pr.w + qkt * d.w);
  }
}

hipError_t launch_decode_step(bool bf16_io, const void* q, const void* k, const void* v,
                              const float* log_alpha, const float* beta, float* S,
                              void* o, int64_t pairs, hipStream_t stream) {
  if (pairs == 0) return hipSuccess;
  dim3 grid((unsigned)pairs), block(256);
  if (bf16_io)
    decode_step_kernel<bf16><<<grid, block, 0, stream>>>(
        (const bf16*)q, (const bf16*)k, (const bf16*)v, log_alpha, beta, S, (bf16*)o);
  else
    decode_step_kernel<float><<<grid, block, 0, stream>>>(
        (const float*)q, (const float*)k, (const float*)v, log_alpha, beta, S, (float*)o);
  return hipGetLastError();
}

}  // namespace kda
