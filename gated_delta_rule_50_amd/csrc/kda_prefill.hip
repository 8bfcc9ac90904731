// Chunked KDA prefill for gfx950: chunk map, intra-chunk UT transform and
// the inter-chunk state carry with the chunk output.
//
// Algorithm: "Kimi Linear: An Expressive, Efficient Attention Architecture"
// (paper-graph-ui review), section "Chunkwise Parallelization":
//   g_i      = sum_{t<=i} log alpha_t inside a chunk (Gamma rows exp(g_i)),
//   UT form  M = (I + StrictTril(Diag(beta)(Gamma*K)(K/Gamma)^T))^{-1} Diag(beta),
//            W = M (Gamma*K), U = M V,
//   Eq. 8    S' = Diag(gamma_C) S + (Gamma^{i->C}*K)^T (U - W S),
//   Eq. 9    O  = (Gamma*Q) S + Tril((Gamma*Q)(K/Gamma)^T)(U - W S).
//
// MI355X design (differs from the pages' Tensor-Core description):
//  * Everything that does not depend on the carried state runs in one fully
//    parallel kernel over (chunk, head) -- the gate cumsum, the decayed
//    A matrices, the triangular inverse, W, U -- and is regrouped so the
//    sequential kernel does the least work per chunk:
//        O = Qt S + Ut   with Qt = Gamma*Q - A_qk W and Ut = A_qk U,
//    i.e. Eq. 9 with the pseudo-value expanded. The sequential kernel then
//    needs two products per chunk: [-W; Qt] S (128 x 128 x 16 per column
//    tile: pseudo-value and output at once) and K'^T (U - W S).
//  * No 1/Gamma is formed anywhere. The decayed inner products
//    sum_c x_r[c] y_i[c] exp(g_r[c] - g_i[c]) use 16-row blocks: for a row
//    block starting at s, the row factor exp(g_r - g_s) <= 1 and, for
//    earlier column blocks, the column factor exp(g_s - g_i) <= 1 (the review's
//    "Numerical stability via secondary chunking", with per-block instead of
//    per-row references so the products stay on the matrix cores). Diagonal
//    blocks use the same factors; if a column factor there could exceed e^44
//    (extreme decays), that 16x16 block is recomputed exactly per element.
//  * The intermediates are written in the exact register-fragment order the
//    sequential kernel consumes, so its loads are contiguous 16-byte vectors
//    and no transposes happen on the sequential path.
#include "kda_device.h"

namespace kda {

// ------------------------------------------------------------- chunk map
// chunk_offset[n] = sum_{m<n} ceil(L_m / 64); status = 1 if cu_seqlens is
// malformed (cu[0] != 0, decreasing, outside [0, T], cu[N] != T) or the
// chunk count exceeds the slots the launch was sized for.
__global__ __launch_bounds__(256) void chunk_map_kernel(
    const int32_t* __restrict__ cu, int32_t n_seqs, int64_t T, int64_t n_slots,
    int32_t* __restrict__ chunk_offset, int32_t* __restrict__ status) {
  __shared__ int32_t s_scan[256];
  __shared__ int32_t s_carry, s_bad;
  const int t = threadIdx.x;
  if (t == 0) {
    s_carry = 0;
    s_bad = 0;
    chunk_offset[0] = 0;
  }
  __syncthreads();
  if (cu == nullptr) {
    if (t == 0) {
      chunk_offset[1] = (int32_t)((T + kC - 1) / kC);
      status[0] = 0;
    }
    return;
  }
  for (int base = 0; base < n_seqs; base += 256) {
    const int n = base + t;
    int cnt = 0;
    if (n < n_seqs) {
      const int64_t a = cu[n], b = cu[n + 1];
      if (b < a || a < 0 || b > T || (n == 0 && a != 0))
        s_bad = 1;
      else
        cnt = (int)((b - a + kC - 1) / kC);
    }
    s_scan[t] = cnt;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int x = t >= off ? s_scan[t - off] : 0;
      __syncthreads();
      s_scan[t] += x;
      __syncthreads();
    }
    if (n < n_seqs) chunk_offset[n + 1] = s_carry + s_scan[t];
    __syncthreads();
    if (t == 255) s_carry += s_scan[255];
    __syncthreads();
  }
  if (t == 0) {
    if ((int64_t)cu[n_seqs] != T || (int64_t)s_carry > n_slots) s_bad = 1;
    status[0] = s_bad;
  }
}

// ----------------------------------------------------------- intra-chunk
constexpr int kIntraThreads = 512;   // 8 waves
constexpr int kGS = kD + 4;          // LDS row stride of g (floats)
constexpr int kLS = kC + 4;          // LDS row stride of the 64 x 64 matrices
constexpr int kTS = 20;              // LDS row stride of 16 x 16 scratch blocks

// LDS row stride (elements) of the staged q / k / v rows.
template <class E>
struct Stage {
  static constexpr int kRS = kD + 16 / (int)sizeof(E);   // 16-byte pad per row
  static constexpr bool kStageV = sizeof(E) == 2;        // fp32 v is read from global
};

// acc += A (16x16) * B (16x16), fp32, operands in LDS (row strides lda, ldb).
__device__ __forceinline__ floatx4 blk16(floatx4 acc, const float* A, int lda,
                                         const float* B, int ldb, int r, int g) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = mma4(acc, A[r * lda + 4 * s + g], B[(4 * s + g) * ldb + r]);
  return acc;
}

// 16-byte vector of I/O elements (8 bf16 or 4 fp32).
template <class E>
using Vec16 = typename std::conditional<sizeof(E) == 2, bf16x8, float4>::type;

template <class E>
__global__ __launch_bounds__(kIntraThreads) void intra_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_offset,
    const int32_t* __restrict__ status, int32_t n_seqs, int64_t T, int32_t H,
    uint8_t* __restrict__ inter) {
  constexpr int RS = Stage<E>::kRS;
  constexpr bool kStageV = Stage<E>::kStageV;
  constexpr int kPer16 = 16 / (int)sizeof(E);          // elements per 16 bytes
  constexpr int kRow16 = kD / kPer16;                   // 16-byte pieces per row
  __shared__ __attribute__((aligned(16))) float sg[kC * kGS];     // g_i[c]
  __shared__ __attribute__((aligned(16))) E sK[kC * RS];
  __shared__ __attribute__((aligned(16))) E sQ[kC * RS];
  __shared__ __attribute__((aligned(16))) E sV[kStageV ? kC * RS : 8];
  __shared__ __attribute__((aligned(16))) float sL[kC * kLS];     // L, later P
  __shared__ __attribute__((aligned(16))) float sTi[kC * kLS];    // (I + L)^{-1}
  __shared__ __attribute__((aligned(16))) float sAqk[kC * kLS];   // A_qk
  __shared__ __attribute__((aligned(16))) float stmp[3 * 16 * kTS];
  __shared__ float sb[kC];
  __shared__ float spart[4 * kD];

  if (status[0] != 0) return;
  const int b = blockIdx.x, h = blockIdx.y;
  const int total = chunk_offset[n_seqs];
  if (b >= total) return;
  int lo = 0, hi = n_seqs;  // chunk_offset[lo] <= b < chunk_offset[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (chunk_offset[mid] <= b) lo = mid; else hi = mid;
  }
  const int n = lo;
  const int64_t seq_start = cu ? cu[n] : 0, seq_end = cu ? cu[n + 1] : T;
  const int64_t tok0 = seq_start + (int64_t)(b - chunk_offset[n]) * kC;
  const int len = (int)min((int64_t)kC, seq_end - tok0);

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int r = lane & 15, g = lane >> 4;
  auto row = [&](int i) -> int64_t { return ((tok0 + i) * H + h) * (int64_t)kD; };

  E* blk = reinterpret_cast<E*>(inter + ((int64_t)b * H + h) * Inter<E>::kBytes);
  E* XA = blk + Inter<E>::kXA;
  E* KT = blk + Inter<E>::kKT;
  E* UC = blk + Inter<E>::kUC;
  float* GC = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(blk) + Inter<E>::kGCByte);

  // ---- 0. stage the chunk: every global load is issued before the first
  //         LDS write, so the whole chunk arrives in one round trip. Rows
  //         past the sequence end are zero (identity tokens).
  {
    constexpr int kPieces = kC * kRow16;               // 16-byte pieces per tile
    constexpr int kPerThread = kPieces / kIntraThreads;
    Vec16<E> vk[kPerThread], vq[kPerThread], vv[kStageV ? kPerThread : 1];
    float4 vla[kC * (kD / 4) / kIntraThreads];
    const Vec16<E> zero16 = {};
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int pc = t + u * kIntraThreads, i = pc / kRow16, c = (pc % kRow16) * kPer16;
      vk[u] = i < len ? *reinterpret_cast<const Vec16<E>*>(k + row(i) + c) : zero16;
      vq[u] = i < len ? *reinterpret_cast<const Vec16<E>*>(q + row(i) + c) : zero16;
      if constexpr (kStageV)
        vv[u] = i < len ? *reinterpret_cast<const Vec16<E>*>(v + row(i) + c) : zero16;
    }
#pragma unroll
    for (int u = 0; u < kC * (kD / 4) / kIntraThreads; ++u) {
      const int pc = t + u * kIntraThreads, i = pc / (kD / 4), c = (pc % (kD / 4)) * 4;
      vla[u] = i < len ? *reinterpret_cast<const float4*>(log_alpha + row(i) + c)
                       : float4{0.f, 0.f, 0.f, 0.f};
    }
    const float bt = (t < kC && t < len) ? beta[(tok0 + t) * H + h] : 0.f;
    for (int x = t; x < kC * kLS; x += kIntraThreads) {
      sL[x] = 0.f;
      sTi[x] = 0.f;
      sAqk[x] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const int pc = t + u * kIntraThreads, i = pc / kRow16, c = (pc % kRow16) * kPer16;
      *reinterpret_cast<Vec16<E>*>(&sK[i * RS + c]) = vk[u];
      *reinterpret_cast<Vec16<E>*>(&sQ[i * RS + c]) = vq[u];
      if constexpr (kStageV) *reinterpret_cast<Vec16<E>*>(&sV[i * RS + c]) = vv[u];
    }
#pragma unroll
    for (int u = 0; u < kC * (kD / 4) / kIntraThreads; ++u) {
      const int pc = t + u * kIntraThreads, i = pc / (kD / 4), c = (pc % (kD / 4)) * 4;
      *reinterpret_cast<float4*>(&sg[i * kGS + c]) = vla[u];
    }
    if (t < kC) sb[t] = bt;
  }
  __syncthreads();

  // ---- 1. gate: g = inclusive cumsum of log alpha along the chunk; four
  //         16-row segments per channel, then segment offsets.
  {
    const int c = t & 127, seg = t >> 7;
    float acc = 0.f;
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) {
      acc += sg[(16 * seg + ii) * kGS + c];
      sg[(16 * seg + ii) * kGS + c] = acc;
    }
    spart[seg * kD + c] = acc;
    __syncthreads();
    float off = 0.f;
#pragma unroll
    for (int u = 0; u < 3; ++u) off += u < seg ? spart[u * kD + c] : 0.f;
    if (seg > 0) {
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) sg[(16 * seg + ii) * kGS + c] += off;
    }
  }
  __syncthreads();
  if (t < kD) GC[t] = exp_f(sg[(kC - 1) * kGS + t]);

  // ---- 2. decayed inner products A_kk (strict) and A_qk (inclusive) on
  //         16 x 16 blocks (I, J <= I): waves 0-3 take (3, w), waves 4-6
  //         take (2, w - 4), wave 7 takes (1, 0), (1, 1) and (0, 0). For row
  //         block I the reference is its first row s = 16 I: the row factor
  //         exp(g_r - g_s) <= 1 and, for J < I, the column factor
  //         exp(g_s - g_i) <= 1.
  {
    auto pair = [&](int u, int& I, int& J) {
      if (w < 4) { I = u == 0 ? 3 : -1; J = w; }
      else if (w < 7) { I = u == 0 ? 2 : -1; J = w - 4; }
      else { I = u < 2 ? 1 : 0; J = u == 1 ? 1 : 0; }
    };
    floatx4 akk[3], aqk[3];
    bool wide[3];
#pragma unroll
    for (int u = 0; u < 3; ++u) { akk[u] = zero4(); aqk[u] = zero4(); wide[u] = false; }
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      int I, J;
      pair(u, I, J);
      if (I < 0) continue;
      const int R = 16 * I + r, i = 16 * J + r;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int c0 = 32 * kb + 8 * g;
        float kr[8], qr[8], ki[8];
        load8(&sK[R * RS + c0], kr);
        load8(&sQ[R * RS + c0], qr);
        load8(&sK[i * RS + c0], ki);
        const float4 gs0 = *reinterpret_cast<const float4*>(&sg[(16 * I) * kGS + c0]);
        const float4 gs1 = *reinterpret_cast<const float4*>(&sg[(16 * I) * kGS + c0 + 4]);
        const float4 gr0 = *reinterpret_cast<const float4*>(&sg[R * kGS + c0]);
        const float4 gr1 = *reinterpret_cast<const float4*>(&sg[R * kGS + c0 + 4]);
        const float4 gi0 = *reinterpret_cast<const float4*>(&sg[i * kGS + c0]);
        const float4 gi1 = *reinterpret_cast<const float4*>(&sg[i * kGS + c0 + 4]);
        const float gs[8] = {gs0.x, gs0.y, gs0.z, gs0.w, gs1.x, gs1.y, gs1.z, gs1.w};
        const float gr[8] = {gr0.x, gr0.y, gr0.z, gr0.w, gr1.x, gr1.y, gr1.z, gr1.w};
        const float gi[8] = {gi0.x, gi0.y, gi0.z, gi0.w, gi1.x, gi1.y, gi1.z, gi1.w};
        Frag<E> fk, fq, fb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float f = exp_f(gr[e] - gs[e]);             // <= 1
          const float x = gs[e] - gi[e];                    // <= 0 unless J == I
          if (J == I && x > 44.f) wide[u] = true;
          fk.set(e, kr[e] * f);
          fq.set(e, qr[e] * f);
          fb.set(e, ki[e] * exp_f(fminf(x, 44.f)));
        }
        akk[u] = mma(akk[u], fk, fb);
        aqk[u] = mma(aqk[u], fq, fb);
      }
    }
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      int I, J;
      pair(u, I, J);
      if (I < 0) continue;
      if (J == I && __ballot(wide[u])) {
        // exact diagonal block: entries (Rr = 16 I + 4 g + e, i = 16 I + r)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int Rr = 16 * I + 4 * g + e, i = 16 * I + r;
          float skk = 0.f, sqk = 0.f;
          if (i <= Rr && Rr < len) {
            for (int c = 0; c < kD; ++c) {
              const float d = exp_f(sg[Rr * kGS + c] - sg[i * kGS + c]);
              const float kic = to_f(sK[i * RS + c]);
              skk += to_f(sK[Rr * RS + c]) * kic * d;
              sqk += to_f(sQ[Rr * RS + c]) * kic * d;
            }
          }
          akk[u][e] = skk;
          aqk[u][e] = sqk;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int Rr = 16 * I + 4 * g + e, i = 16 * J + r;
        sL[Rr * kLS + i] = i < Rr ? sb[Rr] * akk[u][e] : 0.f;
        sAqk[Rr * kLS + i] = i <= Rr ? aqk[u][e] : 0.f;
      }
    }
  }
  __syncthreads();

  // ---- 3. Ti = (I + L)^{-1}: diagonal 16 x 16 blocks by forward
  //         substitution (one column per lane, waves 0-3), then the
  //         off-diagonal blocks Ti_IJ = -Ti_II sum_{K=J}^{I-1} L_IK Ti_KJ,
  //         level by level.
  if (w < 4 && lane < 16) {
    const int base = 16 * w, jj = lane;
    float x[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      float s = rr == jj ? 1.f : 0.f;
#pragma unroll
      for (int ii = 0; ii < rr; ++ii) s -= sL[(base + rr) * kLS + base + ii] * x[ii];
      x[rr] = s;
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) sTi[(base + rr) * kLS + base + jj] = x[rr];
  }
  __syncthreads();
#pragma unroll
  for (int d = 1; d < 4; ++d) {
    if (w < 4 - d) {
      const int I = d + w, J = w;
      floatx4 acc = zero4();
      for (int K = J; K < I; ++K)
        acc = blk16(acc, &sL[(16 * I) * kLS + 16 * K], kLS, &sTi[(16 * K) * kLS + 16 * J], kLS, r, g);
#pragma unroll
      for (int e = 0; e < 4; ++e) stmp[w * 16 * kTS + (4 * g + e) * kTS + r] = acc[e];
    }
    __syncthreads();
    if (w < 4 - d) {
      const int I = d + w, J = w;
      floatx4 acc = blk16(zero4(), &sTi[(16 * I) * kLS + 16 * I], kLS, &stmp[w * 16 * kTS], kTS, r, g);
#pragma unroll
      for (int e = 0; e < 4; ++e) sTi[(16 * I + 4 * g + e) * kLS + 16 * J + r] = -acc[e];
    }
    __syncthreads();
  }

  // ---- 4. P = A_qk Ti (lower triangular) into sL's storage; 20 block
  //         products over 7 waves: (3,0) | (3,1) | (2,0) | (3,2)+(0,0) |
  //         (2,1)+(1,1) | (1,0)+(2,2) | (3,3).
  {
    auto plan = [&](int u, int& I, int& J) {
      const int tab[8][2][2] = {{{3, 0}, {-1, 0}}, {{3, 1}, {-1, 0}}, {{2, 0}, {-1, 0}},
                                {{3, 2}, {0, 0}},  {{2, 1}, {1, 1}},  {{1, 0}, {2, 2}},
                                {{3, 3}, {-1, 0}}, {{-1, 0}, {-1, 0}}};
      I = tab[w][u][0];
      J = tab[w][u][1];
    };
    floatx4 acc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      acc[u] = zero4();
      int I, J;
      plan(u, I, J);
      if (I < 0) continue;
      for (int K = J; K <= I; ++K)
        acc[u] = blk16(acc[u], &sAqk[(16 * I) * kLS + 16 * K], kLS, &sTi[(16 * K) * kLS + 16 * J], kLS, r, g);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int I, J;
      plan(u, I, J);
      if (I < 0) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) sL[(16 * I + 4 * g + e) * kLS + 16 * J + r] = acc[u][e];
    }
  }
  __syncthreads();
  const float* sP = sL;

  // ---- 5. [-W^T | Qt^T] = B1^T [-Ti^T | -P^T] + [0 | (Gamma*Q)^T] with
  //         B1 = Diag(beta)(Gamma*K); K'^T fragments on the side. Wave w owns
  //         key channels c in [16 w, 16 w + 16). The token-index contraction
  //         uses the split order, so each accumulator holds half of one of
  //         the sequential kernel's A-fragments.
  {
    const int m = w, cc = 16 * m + r, c4 = 16 * m + 4 * g;
    floatx4 acc[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      acc[nt] = zero4();
      if (nt < 4) continue;
      const int R = 16 * (nt - 4) + r;
      float qv[4];
      load4(&sQ[R * RS + c4], qv);
      const float4 gq = *reinterpret_cast<const float4*>(&sg[R * kGS + c4]);
      acc[nt][0] = exp_f(gq.x) * qv[0];
      acc[nt][1] = exp_f(gq.y) * qv[1];
      acc[nt][2] = exp_f(gq.z) * qv[2];
      acc[nt][3] = exp_f(gq.w) * qv[3];
    }
    const float gC = sg[(kC - 1) * kGS + cc];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      Frag<E> fa, fkt;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 32 * kb + split_k(g, e);
        const float kv = to_f(sK[i * RS + cc]);
        const float gi = sg[i * kGS + cc];
        fa.set(e, sb[i] * exp_f(gi) * kv);
        fkt.set(e, exp_f(gC - gi) * kv);
      }
      store_frag(KT + (m * 2 + kb) * kWave * 8, lane, fkt);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const float* src = nt < 4 ? sTi : sP;
        const int R = 16 * (nt & 3) + r;
        const float4 x0 = *reinterpret_cast<const float4*>(&src[R * kLS + 32 * kb + 4 * g]);
        const float4 x1 = *reinterpret_cast<const float4*>(&src[R * kLS + 32 * kb + 16 + 4 * g]);
        Frag<E> fb;
        fb.set(0, -x0.x); fb.set(1, -x0.y); fb.set(2, -x0.z); fb.set(3, -x0.w);
        fb.set(4, -x1.x); fb.set(5, -x1.y); fb.set(6, -x1.z); fb.set(7, -x1.w);
        acc[nt] = mma(acc[nt], fa, fb);
      }
    }
    // this wave's 16 channels are slots 0-3 (even m) or 4-7 (odd m) of the
    // A-fragment (row tile nt, k-block m / 2)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
      store_half_frag(XA + (nt * 4 + (m >> 1)) * kWave * 8, lane, m & 1, acc[nt]);
  }

  // ---- 6. U = Ti Diag(beta) V (C-fragments, rows = token) and
  //         Ut^T = (Diag(beta) V)^T P^T (C-fragments, rows = value column),
  //         the transposed form the sequential kernel's O^T product starts
  //         from. Wave w owns value columns [16 w, 16 w + 16); the same
  //         (beta V) fragment is the B operand of U and the A operand of Ut^T.
  {
    const int jt = w, j = 16 * jt + r;
    floatx4 acc[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[mt] = zero4();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      Frag<E> fv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 32 * kb + 8 * g + e;
        float vv;
        if constexpr (kStageV) vv = to_f(sV[i * RS + j]);
        else vv = i < len ? to_f(v[row(i) + j]) : 0.f;
        fv.set(e, sb[i] * vv);
      }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const float* src = mt < 4 ? sTi : sP;
        const int R = 16 * (mt & 3) + r;
        const float4 x0 = *reinterpret_cast<const float4*>(&src[R * kLS + 32 * kb + 8 * g]);
        const float4 x1 = *reinterpret_cast<const float4*>(&src[R * kLS + 32 * kb + 8 * g + 4]);
        Frag<E> fm;
        fm.set(0, x0.x); fm.set(1, x0.y); fm.set(2, x0.z); fm.set(3, x0.w);
        fm.set(4, x1.x); fm.set(5, x1.y); fm.set(6, x1.z); fm.set(7, x1.w);
        acc[mt] = mt < 4 ? mma(acc[mt], fm, fv) : mma(acc[mt], fv, fm);
      }
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) store_c4(UC + (jt * 8 + mt) * kWave * 4, lane, acc[mt]);
  }
}

// ------------------------------------------------------- sequential carry
// One wave per 16-column tile of the state. Per chunk:
//   X[0..3] = U + [-W] S            pseudo-value (rows = token)
//   X[4..7] = Ut^T + S^T Qt^T       O^T (rows = value column)
//   S = Diag(gamma_C) S + K'^T X[0..3]
// The state never leaves registers; its accumulator tiles feed the next
// products directly in the split K order (as B operand for -W S and as A
// operand for S^T Qt^T -- the two fragment layouts are the same).
//
// bf16 intermediates: each workgroup has one compute wave and one loader
// wave. The loader streams chunk b+2's block (fragments of [-W ; Qt], K'^T,
// this tile's [U ; Ut^T] and gamma_C) into a three-deep LDS ring with
// buffer->LDS DMA and waits only for its own loads; the compute wave never
// waits on memory except LDS, so its output stores stay in flight. fp32
// intermediates (twice the bytes; fp32 I/O only) are read from global memory
// by the compute wave directly.
constexpr int kRing = 3;

template <class E>
__device__ __forceinline__ void carry_chunk(floatx4 (&S)[8], const E* XA, const E* KT,
                                            const E* UC, const float* GC, E* __restrict__ o,
                                            int64_t tok0, int len, int H, int h, int lane,
                                            int j0) {
  const int g = lane >> 4;
  // Operand fragments are fetched one k-block ahead of the products that
  // use them, so LDS latency overlaps the matrix-core work.
  Frag<E> fa[2][8];
  floatx4 X[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) load_frag(XA + (mt * 4 + 0) * kWave * 8, lane, fa[0][mt]);
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) X[mt] = load_c4(UC + mt * kWave * 4, lane);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    if (kb + 1 < 4) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
        load_frag(XA + (mt * 4 + kb + 1) * kWave * 8, lane, fa[(kb + 1) & 1][mt]);
    } else {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) load_frag(KT + (mt * 2 + 0) * kWave * 8, lane, fa[0][mt]);
    }
    Frag<E> fs;
#pragma unroll
    for (int e = 0; e < 4; ++e) { fs.set(e, S[2 * kb][e]); fs.set(4 + e, S[2 * kb + 1][e]); }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) X[mt] = mma(X[mt], fa[kb & 1][mt], fs);
#pragma unroll
    for (int mt = 4; mt < 8; ++mt) X[mt] = mma(X[mt], fs, fa[kb & 1][mt]);
  }
  // O^T: lane (i = 16 nt + r, j = j0 + 4 g .. +3) holds four consecutive
  // outputs of one token, written as one 8-byte (bf16) store.
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int i = 16 * nt + (lane & 15);
    if (i < len) store4_io(o + ((tok0 + i) * H + h) * kD + j0 + 4 * g, X[4 + nt]);
  }
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    const float4 gm = *reinterpret_cast<const float4*>(GC + 16 * mt + 4 * g);
    S[mt][0] *= gm.x; S[mt][1] *= gm.y; S[mt][2] *= gm.z; S[mt][3] *= gm.w;
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    if (kb == 0) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) load_frag(KT + (mt * 2 + 1) * kWave * 8, lane, fa[1][mt]);
    }
    Frag<E> fv;
#pragma unroll
    for (int e = 0; e < 4; ++e) { fv.set(e, X[2 * kb][e]); fv.set(4 + e, X[2 * kb + 1][e]); }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) S[mt] = mma(S[mt], fa[kb][mt], fv);
  }
}

// Workgroup barrier without a memory fence: the compute wave reads only
// LDS that the loader wave has already waited for, and no wave writes LDS.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Staged bytes per chunk: [-W ; Qt] and K'^T (48 KiB), the tile's
// [U ; Ut^T] (4 KiB), gamma_C (512 B, in a 1 KiB slot).
constexpr int kStageShared = (kXAElems + kKTElems) * 2;
constexpr int kStageUC = 8 * kWave * 4 * 2;
constexpr int kStageBuf = kStageShared + kStageUC + 1024;
constexpr int kStageDMA = kStageBuf / 1024;   // 1 KiB DMA instructions per chunk

template <class E>
__global__ __launch_bounds__(128) void carry_kernel(
    const uint8_t* __restrict__ inter, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ chunk_offset, const int32_t* __restrict__ status,
    const float* __restrict__ h0, float* __restrict__ h_final, E* __restrict__ o,
    int32_t n_seqs, int64_t T, int32_t H) {
  constexpr bool kStaged = sizeof(E) == 2;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kStaged ? kRing * kStageBuf : 16];

  // XCD-aware order: consecutive ids go round-robin over the 8 XCDs; give the
  // 8 tiles of one (sequence, head) the same id % 8 so they share an L2.
  const int id = blockIdx.x;
  const int pair = (id & 7) + 8 * ((id >> 3) / 8);
  const int jt = (id >> 3) % 8;
  if (pair >= n_seqs * H) return;
  if (status[0] != 0) return;
  const int n = pair / H, h = pair % H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;  // w 0: compute, 1: loader
  const int g = lane >> 4;
  const int j = 16 * jt + (lane & 15);
  const int64_t seq_start = cu ? cu[n] : 0, seq_end = cu ? cu[n + 1] : T;
  const int b0 = chunk_offset[n], b1 = chunk_offset[n + 1];
  auto block_of = [&](int b) { return inter + ((int64_t)b * H + h) * Inter<E>::kBytes; };

  floatx4 S[8];
  if (w == 0) {
    const float* h0p = h0 ? h0 + (int64_t)pair * kD * kD : nullptr;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        S[mt][e] = h0p ? h0p[(16 * mt + 4 * g + e) * kD + j] : 0.f;
  }

  if constexpr (kStaged) {
    // loader: one 1 KiB DMA per instruction; SGPR offsets, no VGPR math
    auto issue = [&](int b) {
      const uint8_t* src = block_of(b);
      uint8_t* dst = lds + ((b - b0) % kRing) * kStageBuf;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)src, 0, (int)Inter<E>::kBytes, 0x00020000);
#pragma unroll
      for (int i = 0; i < kStageShared / 1024; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(dst + i * 1024), 16, lane * 16,
            i * 1024, 0, 0);
      const int uc = (int)(Inter<E>::kUC * sizeof(E)) + jt * kStageUC;
#pragma unroll
      for (int i = 0; i < kStageUC / 1024; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(dst + kStageShared + i * 1024), 16,
            lane * 16, uc + i * 1024, 0, 0);
      // gamma_C: 512 bytes; lanes >= 32 read past the block and get zeros
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(dst + kStageShared + kStageUC), 16,
          lane * 16, (int)Inter<E>::kGCByte, 0, 0);
    };
    if (w == 1) {
      if (b0 < b1) issue(b0);
      if (b0 + 1 < b1) {
        issue(b0 + 1);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kStageDMA) : "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
    }
    ring_barrier();
    for (int b = b0; b < b1; ++b) {
      if (w == 0) {
        const uint8_t* base = lds + ((b - b0) % kRing) * kStageBuf;
        const int64_t tok0 = seq_start + (int64_t)(b - b0) * kC;
        const int len = (int)min((int64_t)kC, seq_end - tok0);
        carry_chunk<E>(S, reinterpret_cast<const E*>(base),
                       reinterpret_cast<const E*>(base) + kXAElems,
                       reinterpret_cast<const E*>(base + kStageShared),
                       reinterpret_cast<const float*>(base + kStageShared + kStageUC), o, tok0,
                       len, H, h, lane, 16 * jt);
      } else {
        // chunk b+2 goes into the slot chunk b-1 used; then make sure chunk
        // b+1 (issued one iteration ago) has landed
        if (b + 2 < b1) {
          issue(b + 2);
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kStageDMA) : "memory");
        } else {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
      }
      ring_barrier();
    }
  } else {
    if (w == 0) {
      for (int b = b0; b < b1; ++b) {
        const E* blk = reinterpret_cast<const E*>(block_of(b));
        const int64_t tok0 = seq_start + (int64_t)(b - b0) * kC;
        const int len = (int)min((int64_t)kC, seq_end - tok0);
        carry_chunk<E>(S, blk + Inter<E>::kXA, blk + Inter<E>::kKT,
                       blk + Inter<E>::kUC + jt * 8 * kWave * 4,
                       reinterpret_cast<const float*>(
                           reinterpret_cast<const uint8_t*>(blk) + Inter<E>::kGCByte),
                       o, tok0, len, H, h, lane, 16 * jt);
      }
    }
  }
  if (w == 0 && h_final) {
    float* hf = h_final + (int64_t)pair * kD * kD;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) hf[(16 * mt + 4 * g + e) * kD + j] = S[mt][e];
  }
}

// ------------------------------------------------------------- launchers
size_t inter_block_bytes(bool bf16_io) {
  return bf16_io ? Inter<bf16>::kBytes : Inter<float>::kBytes;
}


// phases: bit 0 chunk map, bit 1 intra-chunk, bit 2 carry (all three, in
// order on one stream, make one prefill call).
hipError_t launch_chunk_fwd(int phases, bool bf16_io, const void* q, const void* k,
                            const void* v, const float* log_alpha, const float* beta,
                            const float* h0, const int32_t* cu, int32_t n_seqs, int64_t T,
                            int32_t H, int64_t n_slots, void* o, float* h_final,
                            int32_t* status, int32_t* chunk_offset, uint8_t* inter,
                            hipStream_t stream) {
  hipError_t err = hipSuccess;
  if (phases & 1) {
    chunk_map_kernel<<<1, 256, 0, stream>>>(cu, n_seqs, T, n_slots, chunk_offset, status);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if ((phases & 2) && T > 0 && n_slots > 0) {
    dim3 grid((unsigned)n_slots, (unsigned)H);
    if (bf16_io)
      intra_kernel<bf16><<<grid, kIntraThreads, 0, stream>>>(
          (const bf16*)q, (const bf16*)k, (const bf16*)v, log_alpha, beta, cu,
          chunk_offset, status, n_seqs, T, H, inter);
    else
      intra_kernel<float><<<grid, kIntraThreads, 0, stream>>>(
          (const float*)q, (const float*)k, (const float*)v, log_alpha, beta, cu,
          chunk_offset, status, n_seqs, T, H, inter);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (!(phases & 4)) return hipSuccess;
  const int64_t pairs = (int64_t)n_seqs * H;
  const int64_t nblocks = ((pairs + 7) / 8) * 8 * 8;   // 8 column tiles per pair
  if (bf16_io)
    carry_kernel<bf16><<<(unsigned)nblocks, 128, 0, stream>>>(
        inter, cu, chunk_offset, status, h0, h_final, (bf16*)o, n_seqs, T, H);
  else
    carry_kernel<float><<<(unsigned)nblocks, 128, 0, stream>>>(
        inter, cu, chunk_offset, status, h0, h_final, (float*)o, n_seqs, T, H);
  return hipGetLastError();
}

}  // namespace kda
