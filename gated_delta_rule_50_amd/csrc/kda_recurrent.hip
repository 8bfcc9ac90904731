// Fused multi-token recurrent forward for gfx950.
//
// Runs the recurrence token by token (the review's "Online Learning
// Interpretation" form of Eq. 1, "Kimi Linear: An Expressive, Efficient
// Attention Architecture", paper-graph-ui review):
//   S~ = Diag(alpha_t) S,  e = S~^T k_t,  S <- S~ + beta_t k_t (v_t - e)^T,
//   o_t = S^T q_t = S~^T q_t + beta_t (q_t . k_t) (v_t - e)
// over every token of a sequence with the state held in registers: the state
// is read from HBM once before the first token and written once after the
// last, so a call over L tokens moves the state's bytes once, not L times.
// Over several tokens the decay is not applied to the state each token: with
// S = Diag(G) S^ and G the channel-wise product of the alphas so far,
//   e = S^^T (G alpha_t * k),  S^ <- S^ + (k / (G alpha_t)) (v - e)^T beta,
// so a token costs three FMAs per state value instead of a multiply and
// three FMAs. G is folded into S^ (S^ <- G alpha_t * S^, G <- 1) whenever a
// channel's G alpha_t would fall below 2^-40, and once at the end.
// This is the path the review's "FLOPs Accounting and Inference Strategy"
// section gives short inputs (the recurrent kernel for generation); the
// serving note of the "L2 Deep Distill" page routes q_len <= 64 to it. The
// single-token decode step is this kernel with one token per sequence.
//
// Optional pieces (both from the pages' serving notes):
//  * q and k normalised to unit L2 norm inside the kernel (q <- q / ||q||,
//    with ||x|| = sqrt(sum x^2 + 1e-6)), as the pages fuse it into the
//    operator;
//  * a bfloat16 state in HBM (1 MB per layer at 32 heads), widened to fp32 in
//    registers and rounded to nearest even once when written back.
//
// Layout: one wave (one 64-lane workgroup) per (sequence, head, 32-column
// slice of the value dimension). Lane l owns value columns
// 32 w + 4 (l % 8) .. +3 and key rows 16 (l / 8) .. +15 of that slice, 64
// fp32 state values. Both column reductions of a token (e and S~^T q) are
// sums over the eight lanes that share a column quad (lane bits 3..5), done
// with cross-lane moves inside the wave as a reduce-scatter (each lane ends
// with one column's sums) and a gather of the four corrections, so a token
// needs no workgroup barrier. The per-token vectors (alpha k, alpha q,
// alpha, k) go through a wave-private LDS row so each lane can read its 16
// rows with four 16-byte reads. A decode step on bf16 states uses 64-column
// slices instead (lane: 16 rows more, the four lanes of a quad reduce), so
// each state row piece of a wave is a whole 128-byte line.
#include "kda_device.h"

namespace kda {

namespace {

constexpr int kRowPitch = 20;                  // LDS floats per 16-row group (bank spread)
// The token loop keeps S = Diag(G) S^ with G the decay accumulated since the
// last fold; it folds G into S^ before G of any channel would drop below
// this (so k / G stays far from overflow).
constexpr float kFoldBelow = 0x1p-40f;
constexpr int kStaticLds = 4 * 8 * kRowPitch * 4;   // the four token-vector rows, bytes
constexpr int kLdsPerCu = 160 * 1024;               // gfx950 LDS per CU
// fp32 decode steps with at most this many 32-column waves use 16-column
// slices. Graph-replayed steps of 32 heads: 1 sequence 2.84 -> 2.56 us,
// 2 sequences even, 4 and 8 sequences slower (3.97 -> 4.33, 7.32 -> 9.66 us:
// every wave stages the whole token vectors, so narrower waves repeat more
// of that work once there are enough of them to fill the CUs).
constexpr int64_t kNarrowMaxWaves = 128;

// Sum of x over lanes l and l ^ 8 (DPP rotate by 8 inside each 16-lane row).
__device__ __forceinline__ float sum_xor8(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf,
                                                        false));
}
// Sum over lanes l and (l +- 4) mod 16 inside a row (DPP rotate by 4).
__device__ __forceinline__ float sum_ror4(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf,
                                                        false));
}
// Sum over lanes l and l ^ 1, l and l ^ 2 (DPP quad permutations).
__device__ __forceinline__ float sum_xor1(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf,
                                                        false));
}
__device__ __forceinline__ float sum_xor2(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf,
                                                        false));
}
// Sum over the whole wave, left in every lane.
__device__ __forceinline__ float wave_sum(float x) {
  return sum_xor32(sum_xor16(sum_xor1(sum_xor2(sum_ror4(sum_xor8(x))))));
}
// Reduce-scatter steps: permlane32_swap(a, b) gives {a_lo, b_lo} and
// {a_hi, b_hi} (lo = lanes 0-31, hi = 32-63), so their sum holds a summed
// over lanes l, l ^ 32 in the lanes with bit 5 clear and b's sum in those
// with bit 5 set. permlane16_swap does the same for bit 4.
__device__ __forceinline__ float sum_pair32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_pair16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// All-gather steps: x from the lane with bit 5 (bit 4) clear and set.
__device__ __forceinline__ void gather32(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ void gather16(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

// Two consecutive I/O elements kept raw until used.
template <class IO> struct Raw2;
template <> struct Raw2<float> {
  typedef float __attribute__((ext_vector_type(2))) T;
};
template <> struct Raw2<bf16> {
  typedef bf16 __attribute__((ext_vector_type(2))) T;
};

// State storage: four consecutive columns of one row. The state is touched
// once per call, so its accesses are nontemporal (streamed past the caches).
__device__ __forceinline__ float4 load_state4(const float* p) {
  const floatx4 v = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
  return float4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ float4 load_state4(const bf16* p) {
  const bf16x4 v = __builtin_nontemporal_load(reinterpret_cast<const bf16x4*>(p));
  return float4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ void store_state4(float* p, float4 x) {
  __builtin_nontemporal_store(floatx4{x.x, x.y, x.z, x.w}, reinterpret_cast<floatx4*>(p));
}
__device__ __forceinline__ void store_state4(bf16* p, float4 x) {
  bf16x4 v;
  v[0] = (bf16)x.x; v[1] = (bf16)x.y; v[2] = (bf16)x.z; v[3] = (bf16)x.w;
  __builtin_nontemporal_store(v, reinterpret_cast<bf16x4*>(p));
}

// Per-token inputs of one lane: channels 2 l, 2 l + 1 of q, k, log alpha;
// v of the one value column whose sums the lane finishes; beta.
template <class IO>
struct TokenIn {
  typename Raw2<IO>::T q, k;
  float2 la;
  IO v;
  float b;
};

template <class IO>
__device__ __forceinline__ void fetch_token(TokenIn<IO>& x, const IO* q, const IO* k,
                                            const IO* v, const float* log_alpha,
                                            const float* beta, int64_t row, int lane,
                                            int vcol) {
  const int64_t base = row * kD;
  x.q = *reinterpret_cast<const typename Raw2<IO>::T*>(q + base + 2 * lane);
  x.k = *reinterpret_cast<const typename Raw2<IO>::T*>(k + base + 2 * lane);
  x.la = *reinterpret_cast<const float2*>(log_alpha + base + 2 * lane);
  x.v = v[base + vcol];
  x.b = beta[row];
}

}  // namespace

// kSingle: exactly one token per sequence (the decode step), no token loop.
// kCols: value columns per wave. 32 by default (lane: column quad lane % 8,
// rows 16 (lane / 8) .. +15); 64 for the bf16-state decode step (lane: quad
// lane % 16, rows 32 (lane / 16) .. +31), so a lane's bf16 state row piece
// and the wave's row of the slice fill whole 128-byte lines; 16 for decode
// steps over a few (sequence, head) pairs (lane: quad lane % 4, rows
// 8 (lane / 4) .. +7), twice the waves with half the state each, since such
// a step is bound by one wave's load latency rather than by bandwidth.
template <class IO, class ST, bool kNorm, bool kSingle, int kCols>
__global__ __launch_bounds__(64) void recurrent_fwd_kernel(
    const IO* __restrict__ q, const IO* __restrict__ k, const IO* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta, const ST* h0,
    const int32_t* __restrict__ cu, int64_t seq_len, int64_t T, int32_t H, int64_t pairs,
    IO* __restrict__ o, ST* h_final) {
  static_assert(kCols == 16 || kCols == 32 || kCols == 64, "16-, 32- or 64-column slices");
  constexpr int kSl = kD / kCols;                  // waves per (sequence, head)
  constexpr int kQuads = kCols / 4;                // column quads per slice
  constexpr int kRows = kD / (64 / kQuads);        // key rows per lane
  // Block b runs on XCD b % 8 (round-robin dispatch); the slices of a
  // (sequence, head) pair get blocks on one XCD so the token vectors they
  // all read come from that XCD's L2.
  const int bid = blockIdx.x;
  const int rest = bid >> 3;
  const int w = rest & (kSl - 1);
  const int64_t p = (int64_t)(rest / kSl) * 8 + (bid & 7);
  if (p >= pairs) return;
  const int64_t n = p / H;
  const int h = (int)(p - n * H);

  int64_t bos, eos;
  if constexpr (kSingle) {
    bos = n;
    eos = n + 1;
  } else if (cu != nullptr) {
    bos = min<int64_t>(max<int64_t>(cu[n], 0), T);
    eos = min<int64_t>(max<int64_t>(cu[n + 1], bos), T);
  } else {
    bos = n * seq_len;
    eos = bos + seq_len;
  }

  const int lane = threadIdx.x;
  const int jq = lane % kQuads;   // column quad inside the slice
  const int rl = lane / kQuads;   // rows kRows rl .. kRows rl + kRows - 1
  const int col0 = kCols * w + 4 * jq;
  // after the column sums this lane holds column cq of its quad
  const int cq = 2 * ((lane >> 4) & 1) + (lane >> 5);

  // Wave-private token vectors, 16-row groups at a padded pitch.
  __shared__ __align__(16) float s_ka[8 * kRowPitch], s_qa[8 * kRowPitch];
  __shared__ __align__(16) float s_a[8 * kRowPitch], s_k[8 * kRowPitch];

  float4 s[kRows];
  const int64_t sbase = p * (int64_t)(kD * kD) + (int64_t)(kRows * rl) * kD + col0;
  if (h0 != nullptr) {
#pragma unroll
    for (int i = 0; i < kRows; ++i) s[i] = load_state4(h0 + sbase + i * kD);
  } else {
#pragma unroll
    for (int i = 0; i < kRows; ++i) s[i] = float4{0.f, 0.f, 0.f, 0.f};
  }
  // LDS float offset of the token-vector rows 4 m .. 4 m + 3 of this lane
  auto row4 = [&](int m) {
    const int r0 = kRows * rl + 4 * m;
    return (r0 >> 4) * kRowPitch + (r0 & 15);
  };

  const int widx = (lane >> 3) * kRowPitch + 2 * (lane & 7);  // channels 2 l, 2 l + 1
  // the token loop's running decay G of channels 2 l, 2 l + 1 (S = Diag(G) S^)
  constexpr bool kScaled = !kSingle;
  float G0 = 1.f, G1 = 1.f;
  // multiplies this lane's state rows by the per-channel factors staged in s_a
  auto scale_rows = [&]() {
#pragma unroll
    for (int m = 0; m < kRows / 4; ++m) {
      const float4 f = *reinterpret_cast<const float4*>(s_a + row4(m));
      const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float4& x = s[4 * m + r];
        x.x *= fv[r]; x.y *= fv[r]; x.z *= fv[r]; x.w *= fv[r];
      }
    }
  };
  TokenIn<IO> nxt;
  if (bos < eos) fetch_token(nxt, q, k, v, log_alpha, beta, bos * H + h, lane, col0 + cq);

  for (int64_t t = bos; t < eos; ++t) {
    const TokenIn<IO> cur = nxt;
    // Next token's inputs (the last token fetches itself again: the load is
    // unconditional so the counter waits stay exact).
    if constexpr (!kSingle) {
      const int64_t tn = t + 1 < eos ? t + 1 : t;
      fetch_token(nxt, q, k, v, log_alpha, beta, tn * H + h, lane, col0 + cq);
    }

    const float q0 = (float)cur.q[0], q1 = (float)cur.q[1];
    const float k0 = (float)cur.k[0], k1 = (float)cur.k[1];
    const float a0 = exp_f(cur.la.x), a1 = exp_f(cur.la.y);
    float qk = wave_sum(q0 * k0 + q1 * k1);
    // L2Norm: the raw q and k are staged and their scales applied to the
    // column sums and to the correction instead (e = rk S~^T k,
    // S~^T q^ = rq S~^T q, the update adds k (rk d)^T), so the two norm
    // reductions run beside the products instead of ahead of the staging
    float rk = 1.f, rq = 1.f;
    if constexpr (kNorm) {
      const float kk = wave_sum(k0 * k0 + k1 * k1);
      const float qq = wave_sum(q0 * q0 + q1 * q1);
      // hardware reciprocal square root (about 1 ulp): a correctly rounded
      // sqrt and division would cost ~50 instructions per token
      rk = __builtin_amdgcn_rsqf(kk + kL2NormEps);
      rq = __builtin_amdgcn_rsqf(qq + kL2NormEps);
      qk *= rk * rq;
    }
    __syncthreads();  // the previous token's reads of the rows are done
    bool fold = false;
    if constexpr (kScaled) {
      float g0 = G0 * a0, g1 = G1 * a1;
      fold = __builtin_amdgcn_ballot_w64(!(g0 >= kFoldBelow && g1 >= kFoldBelow)) != 0;
      if (fold) {
        // S~ = Diag(G alpha) S^ in place; G restarts at 1
        *reinterpret_cast<float2*>(s_a + widx) = float2{g0, g1};
        g0 = g1 = 1.f;
      }
      G0 = g0;
      G1 = g1;
      *reinterpret_cast<float2*>(s_ka + widx) = float2{g0 * k0, g1 * k1};
      *reinterpret_cast<float2*>(s_qa + widx) = float2{g0 * q0, g1 * q1};
      *reinterpret_cast<float2*>(s_k + widx) =
          float2{k0 * __builtin_amdgcn_rcpf(g0), k1 * __builtin_amdgcn_rcpf(g1)};
    } else {
      *reinterpret_cast<float2*>(s_ka + widx) = float2{a0 * k0, a1 * k1};
      *reinterpret_cast<float2*>(s_qa + widx) = float2{a0 * q0, a1 * q1};
      *reinterpret_cast<float2*>(s_a + widx) = float2{a0, a1};
      *reinterpret_cast<float2*>(s_k + widx) = float2{k0, k1};
    }
    __syncthreads();
    if (kScaled && fold) scale_rows();

    // Partial column sums over this lane's rows: e = S~^T k, pr = S~^T q.
    float4 pe = {0.f, 0.f, 0.f, 0.f}, pr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < kRows / 4; ++m) {
      const float4 ka = *reinterpret_cast<const float4*>(s_ka + row4(m));
      const float4 qa = *reinterpret_cast<const float4*>(s_qa + row4(m));
      const float kav[4] = {ka.x, ka.y, ka.z, ka.w};
      const float qav[4] = {qa.x, qa.y, qa.z, qa.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float4 x = s[4 * m + r];
        pe.x += kav[r] * x.x; pe.y += kav[r] * x.y; pe.z += kav[r] * x.z; pe.w += kav[r] * x.w;
        pr.x += qav[r] * x.x; pr.y += qav[r] * x.y; pr.z += qav[r] * x.z; pr.w += qav[r] * x.w;
      }
    }
    // Sums over the lanes of the quad (lane bits 3..5, or 4..5 for wide
    // slices) as a reduce-scatter: every exchange pairs two of the lane's
    // values, and the lane ends with e and pr of column cq = 2 bit4 + bit5
    // of its quad.
    const float e01 = sum_pair32(pe.x, pe.y), e23 = sum_pair32(pe.z, pe.w);
    const float p01 = sum_pair32(pr.x, pr.y), p23 = sum_pair32(pr.z, pr.w);
    float ec = sum_pair16(e01, e23), pc = sum_pair16(p01, p23);
    if constexpr (kCols <= 32) {   // lane bit 3
      ec = sum_xor8(ec);
      pc = sum_xor8(pc);
    }
    if constexpr (kCols == 16) {   // lane bit 2 (bit 3 already summed)
      ec = sum_ror4(ec);
      pc = sum_ror4(pc);
    }
    ec *= rk;
    pc *= rq;
    // d = beta (v - e), the correction written along k; every lane then
    // gathers the quad's four d values (times rk: the staged k is raw).
    const float dc = cur.b * ((float)cur.v - ec);
    float d4[4], dlo, dhi;
    gather32(rk * dc, dlo, dhi);     // d of columns 2 bit4 and 2 bit4 + 1
    gather16(dlo, d4[0], d4[2]);
    gather16(dhi, d4[1], d4[3]);
    const float4 d = {d4[0], d4[1], d4[2], d4[3]};

    if constexpr (kScaled) {
      // S^ += (k / G) d^T
#pragma unroll
      for (int m = 0; m < kRows / 4; ++m) {
        const float4 kv = *reinterpret_cast<const float4*>(s_k + row4(m));
        const float kvv[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float4& x = s[4 * m + r];
          x.x += kvv[r] * d.x;
          x.y += kvv[r] * d.y;
          x.z += kvv[r] * d.z;
          x.w += kvv[r] * d.w;
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < kRows / 4; ++m) {
        const float4 a = *reinterpret_cast<const float4*>(s_a + row4(m));
        const float4 kv = *reinterpret_cast<const float4*>(s_k + row4(m));
        const float av[4] = {a.x, a.y, a.z, a.w};
        const float kvv[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float4& x = s[4 * m + r];
          x.x = av[r] * x.x + kvv[r] * d.x;
          x.y = av[r] * x.y + kvv[r] * d.y;
          x.z = av[r] * x.z + kvv[r] * d.z;
          x.w = av[r] * x.w + kvv[r] * d.w;
        }
      }
    }

    // narrow slices: lanes l and l ^ 8 hold the same column
    // lanes that differ only in the summed bits below bit 4 hold the same column
    constexpr int kDup = kCols == 64 ? 0 : (kCols == 32 ? 8 : 12);
    if ((lane & kDup) == 0) o[(t * H + h) * kD + col0 + cq] = from_f<IO>(pc + qk * dc);
  }

  if (h_final != nullptr) {
    if constexpr (kScaled) {
      // S = Diag(G) S^
      __syncthreads();
      *reinterpret_cast<float2*>(s_a + widx) = float2{G0, G1};
      __syncthreads();
      scale_rows();
    }
#pragma unroll
    for (int i = 0; i < kRows; ++i) store_state4(h_final + sbase + i * kD, s[i]);
  }
}

hipError_t launch_recurrent_fwd(bool bf16_io, bool bf16_state, bool l2norm, const void* q,
                                const void* k, const void* v, const float* log_alpha,
                                const float* beta, const void* h0, const int32_t* cu,
                                int64_t seq_len, int64_t T, int32_t H, int64_t pairs,
                                void* o, void* h_final, hipStream_t stream) {
  if (pairs == 0) return hipSuccess;
  const bool single = cu == nullptr && seq_len == 1;
  // bf16 states in a decode step: 64-column slices, whole-line state rows;
  // fp32 decode steps over a few pairs (up to 32, one sequence of 32
  // heads): 16-column slices
  const bool wide = single && bf16_state;
  const bool narrow = single && !bf16_state && pairs * 4 <= kNarrowMaxWaves;
  const int64_t blocks = (pairs + 7) / 8 * 8 * (wide ? 2 : (narrow ? 8 : 4));
  dim3 grid((unsigned)blocks), block(64);
  // Resident workgroups per CU. With one or a few tokens per sequence the
  // kernel streams the states, and HBM serves that stream best with few
  // waves in flight per CU: on 256 x 32 states, capping residency by padding
  // each workgroup's LDS takes the fp32-state decode step from 200 to
  // 175 us (5 per CU), the bf16-state one from 131 to 109 us (8 per CU;
  // 96 us with the 64-column slices, 6 or 8 per CU),
  // L = 2 and 4 from 193 / 199 to 178 / 187 us (8 / 10 per CU). From about
  // 16 tokens on the token loop is VALU-bound and wants every wave it can
  // get, so no cap.
  const int64_t n_seqs = pairs / H;
  const int64_t avg_len = n_seqs > 0 ? T / n_seqs : 0;
  int cap = 0;
  if (single) cap = bf16_state ? 8 : 5;
  else if (avg_len <= 2) cap = 8;
  else if (avg_len <= 4) cap = 10;
  const size_t lds_pad = cap > 0 ? (size_t)(kLdsPerCu / cap - kStaticLds) : 0;
#define KDA_REC_LAUNCH(IO, ST, NORM, ONE, COLS)                                              \
  recurrent_fwd_kernel<IO, ST, NORM, ONE, COLS><<<grid, block, lds_pad, stream>>>(           \
      (const IO*)q, (const IO*)k, (const IO*)v, log_alpha, beta, (const ST*)h0, cu, seq_len, \
      T, H, pairs, (IO*)o, (ST*)h_final)
#define KDA_REC_NORM(IO, ST, COLS)                             \
  if (l2norm) {                                                \
    if (single) KDA_REC_LAUNCH(IO, ST, true, true, COLS);      \
    else KDA_REC_LAUNCH(IO, ST, true, false, 32);              \
  } else {                                                     \
    if (single) KDA_REC_LAUNCH(IO, ST, false, true, COLS);     \
    else KDA_REC_LAUNCH(IO, ST, false, false, 32);             \
  }
  if (bf16_io) {
    if (bf16_state) { KDA_REC_NORM(bf16, bf16, 64); }
    else if (narrow) { KDA_REC_NORM(bf16, float, 16); }
    else { KDA_REC_NORM(bf16, float, 32); }
  } else {
    if (bf16_state) { KDA_REC_NORM(float, bf16, 64); }
    else if (narrow) { KDA_REC_NORM(float, float, 16); }
    else { KDA_REC_NORM(float, float, 32); }
  }
#undef KDA_REC_NORM
#undef KDA_REC_LAUNCH
  return hipGetLastError();
}

}  // namespace kda
