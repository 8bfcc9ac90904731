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
constexpr int kGS = kD + 4;   // LDS row stride of g (floats)
constexpr int kLS = kC + 4;   // LDS row stride of the 64 x 64 matrices
constexpr int kTS = 20;       // LDS row stride of 16 x 16 scratch blocks

// acc += A (16x16) * B (16x16), fp32, operands in LDS (row strides lda, ldb).
__device__ __forceinline__ floatx4 blk16(floatx4 acc, const float* A, int lda,
                                         const float* B, int ldb, int r, int g) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = mma4(acc, A[r * lda + 4 * s + g], B[(4 * s + g) * ldb + r]);
  return acc;
}

template <class E>
__global__ __launch_bounds__(256) void intra_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_offset,
    const int32_t* __restrict__ status, int32_t n_seqs, int64_t T, int32_t H,
    uint8_t* __restrict__ inter) {
  __shared__ __attribute__((aligned(16))) float sg[kC * kGS];     // g_i[c]
  __shared__ __attribute__((aligned(16))) float sL[kC * kLS];     // L, later P
  __shared__ __attribute__((aligned(16))) float sTi[kC * kLS];    // (I + L)^{-1}
  __shared__ __attribute__((aligned(16))) float sAqk[kC * kLS];   // A_qk
  __shared__ __attribute__((aligned(16))) float stmp[3 * 16 * kTS];
  __shared__ float sb[kC];
  __shared__ float shalf[kD];

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

  // ---- 1. gate: g = inclusive cumsum of log alpha over the chunk (padded
  //         rows contribute 0); zero the triangular work matrices.
  for (int x = t; x < kC * kLS; x += 256) {
    sL[x] = 0.f;
    sTi[x] = 0.f;
    sAqk[x] = 0.f;
  }
  {
    const int c = t & 127, half = t >> 7;
    float la[32];
#pragma unroll
    for (int ii = 0; ii < 32; ++ii) {
      const int i = half * 32 + ii;
      la[ii] = i < len ? log_alpha[row(i) + c] : 0.f;
    }
#pragma unroll
    for (int ii = 1; ii < 32; ++ii) la[ii] += la[ii - 1];
    if (half == 0) shalf[c] = la[31];
    __syncthreads();
    const float add = half ? shalf[c] : 0.f;
#pragma unroll
    for (int ii = 0; ii < 32; ++ii) sg[(half * 32 + ii) * kGS + c] = la[ii] + add;
    if (t < kC) sb[t] = t < len ? beta[(tok0 + t) * H + h] : 0.f;
  }
  __syncthreads();
  if (t < kD) GC[t] = exp_f(sg[(kC - 1) * kGS + t]);

  // ---- 2. decayed inner products A_kk (strict) and A_qk (inclusive) on
  //         16 x 16 blocks; wave w owns row block I = 3 - w, blocks J <= I.
  {
    const int I = 3 - w;
    floatx4 akk[4], aqk[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) { akk[J] = zero4(); aqk[J] = zero4(); }
    bool wide = false;
    const int R = 16 * I + r;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int c0 = 32 * kb + 8 * g;
      float kr[8], qr[8], gref[8];
      if (R < len) { load8(k + row(R) + c0, kr); load8(q + row(R) + c0, qr); }
      else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { kr[e] = 0.f; qr[e] = 0.f; }
      }
      Frag<E> fk, fq;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        gref[e] = sg[(16 * I) * kGS + c0 + e];
        const float f = exp_f(sg[R * kGS + c0 + e] - gref[e]);   // <= 1
        fk.set(e, kr[e] * f);
        fq.set(e, qr[e] * f);
      }
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        if (J > I) continue;
        const int i = 16 * J + r;
        float ki[8];
        if (i < len) load8(k + row(i) + c0, ki);
        else {
#pragma unroll
          for (int e = 0; e < 8; ++e) ki[e] = 0.f;
        }
        Frag<E> fb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = gref[e] - sg[i * kGS + c0 + e];  // <= 0 off the diagonal
          if (J == I && x > 44.f) wide = true;
          fb.set(e, ki[e] * exp_f(fminf(x, 44.f)));
        }
        akk[J] = mma(akk[J], fk, fb);
        aqk[J] = mma(aqk[J], fq, fb);
      }
    }
    if (__ballot(wide)) {
      // exact diagonal block: entries (R = 16 I + 4 g + e, i = 16 I + r)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int Rr = 16 * I + 4 * g + e, i = 16 * I + r;
        float skk = 0.f, sqk = 0.f;
        if (i <= Rr && Rr < len) {
          for (int c = 0; c < kD; ++c) {
            const float d = exp_f(sg[Rr * kGS + c] - sg[i * kGS + c]);
            const float ki = to_f(k[row(i) + c]);
            skk += to_f(k[row(Rr) + c]) * ki * d;
            sqk += to_f(q[row(Rr) + c]) * ki * d;
          }
        }
        akk[I][e] = skk;
        aqk[I][e] = sqk;
      }
    }
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      if (J > I) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int Rr = 16 * I + 4 * g + e, i = 16 * J + r;
        sL[Rr * kLS + i] = i < Rr ? sb[Rr] * akk[J][e] : 0.f;
        sAqk[Rr * kLS + i] = i <= Rr ? aqk[J][e] : 0.f;
      }
    }
  }
  __syncthreads();

  // ---- 3. Ti = (I + L)^{-1}: diagonal 16 x 16 blocks by forward
  //         substitution (one column per lane), then the off-diagonal blocks
  //         Ti_IJ = -Ti_II sum_{K=J}^{I-1} L_IK Ti_KJ level by level.
  if (lane < 16) {
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

  // ---- 4. P = A_qk Ti (lower triangular), into sL's storage.
  {
    // Five 16x16x16 block products per wave. Blocks (I, J) of P, K from J to
    // I: waves 0-2 take (3, w) and (w, 0); wave 3 takes (3,3) (2,1) (2,2)
    // (1,1). Slot u's block is chosen with wave-uniform selects.
    auto plan = [&](int u, int& I, int& J) {
      if (w < 3) {
        I = u == 0 ? 3 : (u == 1 ? w : -1);
        J = u == 0 ? w : 0;
      } else {
        I = u == 0 ? 3 : (u == 3 ? 1 : 2);
        J = u == 0 ? 3 : (u == 2 ? 2 : 1);
      }
    };
    floatx4 acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc[u] = zero4();
      int I, J;
      plan(u, I, J);
      if (I < 0) continue;
      for (int K = J; K <= I; ++K)
        acc[u] = blk16(acc[u], &sAqk[(16 * I) * kLS + 16 * K], kLS, &sTi[(16 * K) * kLS + 16 * J], kLS, r, g);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
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
  //         key channels c in [32 w, 32 w + 32). Contraction over the token
  //         index uses the split order so the accumulators are already the
  //         sequential kernel's A-fragments.
  {
    floatx4 acc[2][8];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      const int c4 = 16 * (2 * w + mi) + 4 * g;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        acc[mi][nt] = zero4();
        if (nt < 4) continue;
        const int R = 16 * (nt - 4) + r;
        if (R < len) {
          float qv[4];
          load4(q + row(R) + c4, qv);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[mi][nt][e] = exp_f(sg[R * kGS + c4 + e]) * qv[e];
        }
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      Frag<E> fa[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int m = 2 * w + mi, cc = 16 * m + r;
        const float gC = sg[(kC - 1) * kGS + cc];
        Frag<E> fkt;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 32 * kb + split_k(g, e);
          const float kv = i < len ? to_f(k[row(i) + cc]) : 0.f;
          const float gi = sg[i * kGS + cc];
          fa[mi].set(e, sb[i] * exp_f(gi) * kv);
          fkt.set(e, exp_f(gC - gi) * kv);
        }
        store_frag(KT + (m * 2 + kb) * kWave * 8, lane, fkt);
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const float* src = nt < 4 ? sTi : sP;
        const int R = 16 * (nt & 3) + r;
        const float4 x0 = *reinterpret_cast<const float4*>(&src[R * kLS + 32 * kb + 4 * g]);
        const float4 x1 = *reinterpret_cast<const float4*>(&src[R * kLS + 32 * kb + 16 + 4 * g]);
        Frag<E> fb;
        fb.set(0, -x0.x); fb.set(1, -x0.y); fb.set(2, -x0.z); fb.set(3, -x0.w);
        fb.set(4, -x1.x); fb.set(5, -x1.y); fb.set(6, -x1.z); fb.set(7, -x1.w);
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) acc[mi][nt] = mma(acc[mi][nt], fa[mi], fb);
      }
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      Frag<E> f;
#pragma unroll
      for (int e = 0; e < 4; ++e) { f.set(e, acc[0][nt][e]); f.set(4 + e, acc[1][nt][e]); }
      store_frag(XA + (nt * 4 + w) * kWave * 8, lane, f);
    }
  }

  // ---- 6. [U ; Ut] = [Ti ; P] Diag(beta) V; wave w owns value columns
  //         [32 w, 32 w + 32). Accumulators are the C-fragments the
  //         sequential kernel starts from.
  {
    floatx4 acc[8][2];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) { acc[mt][0] = zero4(); acc[mt][1] = zero4(); }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      Frag<E> fv[2];
#pragma unroll
      for (int ji = 0; ji < 2; ++ji) {
        const int j = 16 * (2 * w + ji) + r;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 32 * kb + 8 * g + e;
          fv[ji].set(e, i < len ? sb[i] * to_f(v[row(i) + j]) : 0.f);
        }
      }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const float* src = mt < 4 ? sTi : sP;
        const int R = 16 * (mt & 3) + r;
        const float4 x0 = *reinterpret_cast<const float4*>(&src[R * kLS + 32 * kb + 8 * g]);
        const float4 x1 = *reinterpret_cast<const float4*>(&src[R * kLS + 32 * kb + 8 * g + 4]);
        Frag<E> fa;
        fa.set(0, x0.x); fa.set(1, x0.y); fa.set(2, x0.z); fa.set(3, x0.w);
        fa.set(4, x1.x); fa.set(5, x1.y); fa.set(6, x1.z); fa.set(7, x1.w);
#pragma unroll
        for (int ji = 0; ji < 2; ++ji) acc[mt][ji] = mma(acc[mt][ji], fa, fv[ji]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int ji = 0; ji < 2; ++ji)
        store_c4(UC + ((2 * w + ji) * 8 + mt) * kWave * 4, lane, acc[mt][ji]);
  }
}

// ------------------------------------------------------- sequential carry
// One wave per 16-column tile of the state; NW waves per workgroup cover NW
// tiles of the same (sequence, head). Per chunk:
//   X = [U ; Ut] + [-W ; Qt] S      (X rows 0..63: pseudo-value, 64..127: O)
//   S = Diag(gamma_C) S + K'^T X[0..63]
// The state never leaves registers; the accumulator tiles feed the next
// product directly in the split K order.
template <class E, int NW>
__global__ __launch_bounds__(64 * NW) void carry_kernel(
    const uint8_t* __restrict__ inter, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ chunk_offset, const int32_t* __restrict__ status,
    const float* __restrict__ h0, float* __restrict__ h_final, E* __restrict__ o,
    int32_t n_seqs, int64_t T, int32_t H) {
  constexpr int G = 8 / NW;  // workgroups per (sequence, head)
  // XCD-aware order: consecutive ids go round-robin over the 8 XCDs; give all
  // G workgroups of one (sequence, head) the same id % 8 so they share an L2.
  const int id = blockIdx.x;
  const int xcd = id & 7, slot = id >> 3;
  const int pair = xcd + 8 * (slot / G);
  const int tg = slot % G;
  if (pair >= n_seqs * H) return;
  if (status[0] != 0) return;
  const int n = pair / H, h = pair % H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int jt = tg * NW + w;
  const int j = 16 * jt + r;

  floatx4 S[8];
  const float* h0p = h0 ? h0 + (int64_t)pair * kD * kD : nullptr;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      S[mt][e] = h0p ? h0p[(16 * mt + 4 * g + e) * kD + j] : 0.f;

  const int64_t seq_start = cu ? cu[n] : 0, seq_end = cu ? cu[n + 1] : T;
  const int b0 = chunk_offset[n], b1 = chunk_offset[n + 1];
  for (int b = b0; b < b1; ++b) {
    const E* blk = reinterpret_cast<const E*>(inter + ((int64_t)b * H + h) * Inter<E>::kBytes);
    const E* XA = blk + Inter<E>::kXA;
    const E* KT = blk + Inter<E>::kKT;
    const E* UC = blk + Inter<E>::kUC;
    const float* GC = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(blk) + Inter<E>::kGCByte);
    const int64_t tok0 = seq_start + (int64_t)(b - b0) * kC;
    const int len = (int)min((int64_t)kC, seq_end - tok0);

    floatx4 X[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) X[mt] = load_c4(UC + (jt * 8 + mt) * kWave * 4, lane);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      Frag<E> fb;
#pragma unroll
      for (int e = 0; e < 4; ++e) { fb.set(e, S[2 * kb][e]); fb.set(4 + e, S[2 * kb + 1][e]); }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        Frag<E> fa;
        load_frag(XA + (mt * 4 + kb) * kWave * 8, lane, fa);
        X[mt] = mma(X[mt], fa, fb);
      }
    }
#pragma unroll
    for (int mt = 4; mt < 8; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * (mt - 4) + 4 * g + e;
        if (i < len) o[((tok0 + i) * H + h) * kD + j] = from_f<E>(X[mt][e]);
      }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const float4 gm = *reinterpret_cast<const float4*>(GC + 16 * mt + 4 * g);
      S[mt][0] *= gm.x; S[mt][1] *= gm.y; S[mt][2] *= gm.z; S[mt][3] *= gm.w;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      Frag<E> fb;
#pragma unroll
      for (int e = 0; e < 4; ++e) { fb.set(e, X[2 * kb][e]); fb.set(4 + e, X[2 * kb + 1][e]); }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        Frag<E> fa;
        load_frag(KT + (mt * 2 + kb) * kWave * 8, lane, fa);
        S[mt] = mma(S[mt], fa, fb);
      }
    }
  }
  if (h_final) {
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

constexpr int kCarryWaves = 1;

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
      intra_kernel<bf16><<<grid, 256, 0, stream>>>(
          (const bf16*)q, (const bf16*)k, (const bf16*)v, log_alpha, beta, cu,
          chunk_offset, status, n_seqs, T, H, inter);
    else
      intra_kernel<float><<<grid, 256, 0, stream>>>(
          (const float*)q, (const float*)k, (const float*)v, log_alpha, beta, cu,
          chunk_offset, status, n_seqs, T, H, inter);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (!(phases & 4)) return hipSuccess;
  const int64_t pairs = (int64_t)n_seqs * H;
  const int64_t groups = 8 / kCarryWaves;
  const int64_t nblocks = ((pairs + 7) / 8) * 8 * groups;
  if (bf16_io)
    carry_kernel<bf16, kCarryWaves><<<(unsigned)nblocks, 64 * kCarryWaves, 0, stream>>>(
        inter, cu, chunk_offset, status, h0, h_final, (bf16*)o, n_seqs, T, H);
  else
    carry_kernel<float, kCarryWaves><<<(unsigned)nblocks, 64 * kCarryWaves, 0, stream>>>(
        inter, cu, chunk_offset, status, h0, h_final, (float*)o, n_seqs, T, H);
  return hipGetLastError();
}

}  // namespace kda
