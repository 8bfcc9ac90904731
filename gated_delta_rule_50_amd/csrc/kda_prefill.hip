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
#include <algorithm>

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
// One workgroup of four waves per (chunk, head). Wave I owns the 16-token
// block I of the chunk and keeps its rows in registers in the "piece"
// layout: lane (r, g) holds token 16 I + r and, for each 16-channel tile ct,
// the channels 16 ct + 4 g .. 16 ct + 4 g + 3. Pieces 2 kb and 2 kb + 1 form
// a split-order fragment of the 32-channel slice kb, and one piece is the
// accumulator layout of a transposed 16 x 16 tile, so
//   * the A tiles (contractions over channels) take row pieces directly,
//   * a product with the identity turns row pieces into a token-major
//     accumulator tile (a transpose on the matrix cores), and
//   * every contraction over tokens uses accumulator tiles as operands:
//     X in the accumulator layout is the B operand of (. X) and the A
//     operand of (X^T .), so both orientations of a product come from the
//     same registers with A and B swapped.
// The triangular solve runs block by block: wave I inverts its diagonal
// block in registers ((I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8) for
// the nilpotent 16 x 16 N), then, after the blocks before it,
//   [W_I | U_I] = Ti_II ([B_I | V'_I] - sum_{J<I} L_IJ [W_J | U_J]),
// and finally Qt_I = Gamma Q_I - sum_{J<=I} A_qk,IJ W_J, Ut_I = sum A_qk,IJ U_J.
// Only the column factors Kf (for the A tiles) and W_J | U_J (for the later
// blocks) pass through LDS; four workgroup barriers per chunk.
constexpr int kIntraThreads = 256;   // 4 waves

// Workgroup barrier that waits for this wave's LDS traffic only (outstanding
// global stores stay in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Inclusive prefix sum over the 16 lanes r of each DPP row (lane l = r + 16 g).
template <int kCtrl>
__device__ __forceinline__ float dpp_in_row(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_scan16(float x) {
  x += dpp_in_row<0x111>(x);   // row_shr:1
  x += dpp_in_row<0x112>(x);   // row_shr:2
  x += dpp_in_row<0x114>(x);   // row_shr:4
  x += dpp_in_row<0x118>(x);   // row_shr:8
  return x;
}

// Eight consecutive elements as an MFMA fragment.
__device__ __forceinline__ void lds_frag(const bf16* p, Frag<bf16>& f) {
  f.v = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void lds_frag(const float* p, Frag<float>& f) { load8(p, f.v); }

template <class E>
__global__ __launch_bounds__(kIntraThreads) void intra_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_offset,
    const int32_t* __restrict__ status, int32_t n_seqs, int64_t T, int32_t H,
    uint8_t* __restrict__ inter) {
  // LDS:
  //   sKf   Kf fragments of the four blocks [J][kb][lane][8]; once every wave
  //         is past its A tiles, its two halves hold W | U of blocks 1 and 2
  //   sWU0  W | U of block 0 as accumulator tiles [tile][lane][4]
  //   sTot  per-block sums of log alpha; sE = exp(sum), sEi = exp(-sum)
  //   sB    beta
  //   sF    per-block channel factors (five rows per block)
  constexpr int kWU = 16 * kWave * 4;
  __shared__ __attribute__((aligned(16))) E sKf[4 * 4 * kWave * 8];
  __shared__ __attribute__((aligned(16))) E sWU0[kWU];
  __shared__ __attribute__((aligned(16))) float sTot[4 * kD];
  __shared__ __attribute__((aligned(16))) float sE[4 * kD];
  __shared__ __attribute__((aligned(16))) float sEi[4 * kD];
  __shared__ __attribute__((aligned(16))) float sB[kC];
  __shared__ __attribute__((aligned(16))) float sF[4 * 5 * kD];
  auto wu_slot = [&](int J) -> E* { return J == 0 ? sWU0 : sKf + (J - 1) * kWU; };

  if (status[0] != 0) return;
  const int b = blockIdx.x, h = blockIdx.y;
  const int total = chunk_offset[n_seqs];
  if (b >= total) return;
  int lo = 0, hi = n_seqs;  // chunk_offset[lo] <= b < chunk_offset[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (chunk_offset[mid] <= b) lo = mid; else hi = mid;
  }
  const int64_t seq_start = cu ? cu[lo] : 0, seq_end = cu ? cu[lo + 1] : T;
  const int64_t tok0 = seq_start + (int64_t)(b - chunk_offset[lo]) * kC;
  const int len = (int)min((int64_t)kC, seq_end - tok0);

  const int lane = threadIdx.x & 63;
  const int I = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // token block
  const int r = lane & 15, g = lane >> 4;
  const int i = 16 * I + r;
  const bool valid = i < len;
  auto row = [&](int x) -> int64_t { return ((tok0 + x) * H + h) * (int64_t)kD; };

  E* blk = reinterpret_cast<E*>(inter + ((int64_t)b * H + h) * Inter<E>::kBytes);
  E* XA = blk + Inter<E>::kXA;
  E* KT = blk + Inter<E>::kKT;
  E* UC = blk + Inter<E>::kUC;
  float* GC = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(blk) + Inter<E>::kGCByte);

  // ---- 0. loads of k, q, log alpha and beta. Tokens past the end of the
  //         sequence read the last valid row and become zeros (identity
  //         tokens). v is loaded after the A tiles.
  const int64_t ro = row(min(i, len - 1));
  Frag16<E> zero;
#pragma unroll
  for (int e = 0; e < 4; ++e) zero.set(e, 0.f);
  Frag16<E> kx[8], qx[8];
  float la[8][4];
  float bt;
  {
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const int64_t o = ro + 16 * ct + 4 * g;
      const Frag16<E> a = ld16(k + o), c = ld16(q + o);
      const float4 l = *reinterpret_cast<const float4*>(log_alpha + o);
      kx[ct] = valid ? a : zero;
      qx[ct] = valid ? c : zero;
      la[ct][0] = valid ? l.x : 0.f; la[ct][1] = valid ? l.y : 0.f;
      la[ct][2] = valid ? l.z : 0.f; la[ct][3] = valid ? l.w : 0.f;
    }
    const float x = beta[(tok0 + min(i, len - 1)) * H + h];
    bt = valid ? x : 0.f;
  }

  // ---- 1. gate: l_i = sum of log alpha over rows 16 I .. i (a scan across
  //         the 16 lanes of a DPP row). The block sums and their
  //         exponentials go to LDS for the other blocks. Row factors
  //         Kr = k e^l, Qr = q e^l and column factors Kf = k e^{l_e - l}
  //         (e = last row of the block) are all <= 1 times the input.
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) la[ct][e] = row_scan16(la[ct][e]);
  if (r == 15) {
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
      *reinterpret_cast<float4*>(&sTot[I * kD + 16 * ct + 4 * g]) =
          float4{la[ct][0], la[ct][1], la[ct][2], la[ct][3]};
  }
  if (g == 0) sB[i] = bt;
  asm volatile("" ::: "memory");
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = lane + 64 * u;
    const float s = sTot[I * kD + c];
    sE[I * kD + c] = exp_f(s);
    sEi[I * kD + c] = exp_f(fminf(-s, 88.f));
  }
  Frag16<E> Kr[8], Qr[8];
  Frag<E> kfI[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int ct = 2 * kb + hh;
      const floatx4 s = *reinterpret_cast<const floatx4*>(&sTot[I * kD + 16 * ct + 4 * g]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float kv = kx[ct].get(e), fr = exp_f(la[ct][e]);
        kfI[kb].set(4 * hh + e, kv * exp_f(s[e] - la[ct][e]));
        Kr[ct].set(e, kv * fr);
        Qr[ct].set(e, qx[ct].get(e) * fr);
      }
    }
    store8(&sKf[((I * 4 + kb) * kWave + lane) * 8], kfI[kb]);
  }
  lds_barrier();

  // ---- 2. per-channel factors of this block, with p_J = g before block J
  //         and E_J = exp(block sum J):
  //           exp(p_I) = prod_{K<I} E_K,  exp(g_C - p_{I+1}) = prod_{K>I} E_K,
  //           D_IJ = exp(p_I - p_{J+1}) = prod_{J<K<I} E_K (<= 1, J < I),
  //         two channels per lane into this wave's rows of sF.
  float* const sFw = sF + I * 5 * kD;   // rows: exp(p_I), exp(g_C - p_{I+1}), D_I0..D_I2
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = lane + 64 * u;
    float ev[4];
#pragma unroll
    for (int K = 0; K < 4; ++K) ev[K] = sE[K * kD + c];
    float a = 1.f, bb = 1.f, d[3] = {1.f, 1.f, 1.f};
#pragma unroll
    for (int K = 0; K < 4; ++K) {
      a *= K < I ? ev[K] : 1.f;
      bb *= K > I ? ev[K] : 1.f;
#pragma unroll
      for (int J = 0; J < 3; ++J) d[J] *= (J < K && K < I) ? ev[K] : 1.f;
    }
    sFw[c] = a;
    sFw[kD + c] = bb;
#pragma unroll
    for (int J = 0; J < 3; ++J) sFw[(2 + J) * kD + c] = d[J];
    if (I == 0) GC[c] = ev[0] * ev[1] * ev[2] * ev[3];   // gamma_C = exp(g_C)
  }
  asm volatile("" ::: "memory");

  // beta Gamma K and Gamma Q row pieces; K' = Kf exp(g_C - p_{I+1}) =
  // k exp(g_C - g) becomes K'^T fragments for the sequential kernel: a K'
  // row piece times the identity is the token-major tile (lane (r, g):
  // K'[16I + 4g + e][16ct + r]), the half of the split-order fragment this
  // block's tokens fill.
  Frag16<E> idf;
#pragma unroll
  for (int e = 0; e < 4; ++e) idf.set(e, 4 * g + e == r ? 1.f : 0.f);
  Frag16<E> Bx[8], GQ[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    const floatx4 gs = *reinterpret_cast<const floatx4*>(&sFw[16 * ct + 4 * g]);
    const floatx4 ek = *reinterpret_cast<const floatx4*>(&sFw[kD + 16 * ct + 4 * g]);
    Frag16<E> kp;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      Bx[ct].set(e, bt * gs[e] * Kr[ct].get(e));
      GQ[ct].set(e, gs[e] * Qr[ct].get(e));
      kp.set(e, kfI[ct >> 1].get(4 * (ct & 1) + e) * ek[e]);
    }
    store_half_frag(KT + (ct * 2 + (I >> 1)) * kWave * 8, lane, I & 1, mma16(zero4(), kp, idf));
  }

  // v rows, needed from step 4 on
  Frag16<E> vx[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    const Frag16<E> d = ld16(v + ro + 16 * ct + 4 * g);
    vx[ct] = valid ? d : zero;
  }

  // A tiles. For J < I, A_kk[i][j] = sum_c (Kr_i D_IJ) Kf_j (same for A_qk
  // with Qr); the diagonal block uses D_II = exp(-block sum) >= 1, and where
  // that could exceed e^44 the block is recomputed exactly below. Lane (r, g)
  // accumulates akT[J][e] = A_kk[16I + r][16J + 4g + e],
  // aqT[J][e] = A_qk[16I + r][16J + 4g + e] and akD[e] = A_kk[16I + 4g + e][16I + r].
  floatx4 akT[4], aqT[4], akD = zero4();
  bool wide = false;
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    akT[J] = zero4();
    aqT[J] = zero4();
    if (J > I) continue;
    const float* Drow = J < I ? sFw + (2 + (J < 3 ? J : 0)) * kD : sEi + I * kD;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const floatx4 d0 = *reinterpret_cast<const floatx4*>(&Drow[32 * kb + 4 * g]);
      const floatx4 d1 = *reinterpret_cast<const floatx4*>(&Drow[32 * kb + 16 + 4 * g]);
      Frag<E> fk, fq;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        fk.set(e, Kr[2 * kb].get(e) * d0[e]);
        fk.set(4 + e, Kr[2 * kb + 1].get(e) * d1[e]);
        fq.set(e, Qr[2 * kb].get(e) * d0[e]);
        fq.set(4 + e, Qr[2 * kb + 1].get(e) * d1[e]);
      }
      if (J < I) {
        Frag<E> fa;
        lds_frag(&sKf[((J * 4 + kb) * kWave + lane) * 8], fa);
        akT[J] = mma(akT[J], fa, fk);
        aqT[J] = mma(aqT[J], fa, fq);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) wide |= d0[e] > 1.2851e19f || d1[e] > 1.2851e19f;  // e^44
        akT[J] = mma(akT[J], kfI[kb], fk);
        aqT[J] = mma(aqT[J], kfI[kb], fq);
        akD = mma(akD, fk, kfI[kb]);
      }
    }
  }

  // exact diagonal block when its factors could overflow: g differences
  // summed from the raw log alphas
  if (__builtin_amdgcn_ballot_w64(wide)) {
    auto exact = [&](int a, int c0, float& skk, float& sqk) {   // rows a >= c0
      skk = sqk = 0.f;
      if (a >= len || c0 > a) return;
      for (int c = 0; c < kD; ++c) {
        float dg = 0.f;
        for (int x = c0 + 1; x <= a; ++x) dg += log_alpha[row(x) + c];
        const float d = exp_f(dg);
        const float kc = to_f(k[row(c0) + c]);
        skk += to_f(k[row(a) + c]) * kc * d;
        sqk += to_f(q[row(a) + c]) * kc * d;
      }
    };
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      if (J != I) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float skk, sqk, tkk, tqk;
        exact(16 * I + r, 16 * I + 4 * g + e, skk, sqk);
        exact(16 * I + 4 * g + e, 16 * I + r, tkk, tqk);
        akT[J][e] = skk;
        aqT[J][e] = sqk;
        akD[e] = tkk;
      }
    }
  }

  // ---- 3. Ti_II = (I + N)^{-1}, N = strictly lower beta_i A_kk of the
  //         diagonal block, held as TiT = Ti_II^T in the accumulator layout.
  //         X = N^T; Ti_II^T = (I + X)^{-1} = (I - X)(I + X^2)(I + X^4)(I + X^8).
  floatx4 Xc, Nc, Ic;
  {
    const float4 b4 = *reinterpret_cast<const float4*>(&sB[16 * I + 4 * g]);
    const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      if (J != I) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Xc[e] = 4 * g + e < r ? bt * akT[J][e] : 0.f;       // N[r][4g+e]
        Nc[e] = r < 4 * g + e ? bb[e] * akD[e] : 0.f;       // N[4g+e][r]
        Ic[e] = 4 * g + e == r ? 1.f : 0.f;
      }
    }
  }
  Frag16<E> tiT;
  {
    const floatx4 X2 = mm16(Nc, Xc), X2T = mm16(Xc, Nc);
    const floatx4 X4 = mm16(X2T, X2), X4T = mm16(X2, X2T);
    const floatx4 X8 = mm16(X4T, X4);
    const floatx4 P1 = Ic - Xc + X2 - mm16(Nc, X2);
    const floatx4 P1T = Ic - Nc + X2T - mm16(X2, Nc);
    const floatx4 P2 = P1 + mm16(P1T, X4), P2T = P1T + mm16(X4, P1T);
    tiT = frag16<E>(P2 + mm16(P2T, X8));
  }
  // -L_IJ (J < I) as A operands, A_qk (J <= I, masked on the diagonal) and
  // its negation as B operands, beta V row pieces
  Frag16<E> nL[3], aq[4], naq[4], Vb[8];
#pragma unroll
  for (int J = 0; J < 4; ++J) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = (J < I || 4 * g + e <= r) ? aqT[J][e] : 0.f;
      aq[J].set(e, x);
      naq[J].set(e, -x);
      if (J < 3) nL[J].set(e, -bt * akT[J][e]);
    }
  }
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) Vb[ct].set(e, bt * vx[ct].get(e));

  // ---- 4. blocked forward substitution, one block per barrier interval.
  Frag16<E> wu[16];   // W_I (tiles 0-7, key channels) | U_I (8-15, value columns)
  for (int s = 0; s < I; ++s) lds_barrier();
  {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      floatx4 M[8];
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) M[ct] = mma16(zero4(), hf ? Vb[ct] : Bx[ct], idf);
#pragma unroll
      for (int J = 0; J < 3; ++J) {
        if (J >= I) continue;
        const E* src = wu_slot(J) + (hf * 8 * kWave + lane) * 4;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          const Frag16<E> w = ld16(src + ct * kWave * 4);
          M[ct] = mma16(M[ct], nL[J], w);
        }
      }
      floatx4 wt[8];
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const Frag16<E> mb = frag16<E>(M[ct]);
        const floatx4 o = mma16(zero4(), tiT, mb);    // W_I / U_I tile, token-major
        wu[hf * 8 + ct] = frag16<E>(o);
        if (hf) store_c4(UC + (ct * 8 + I) * kWave * 4, lane, o);
        else wt[ct] = mma16(zero4(), mb, tiT);        // W_I^T tile
      }
      if (!hf) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          Frag<E> f;
#pragma unroll
          for (int e = 0; e < 4; ++e) { f.set(e, -wt[2 * kb][e]); f.set(4 + e, -wt[2 * kb + 1][e]); }
          store_frag(XA + (I * 4 + kb) * kWave * 8, lane, f);
        }
      }
      if (I < 3) {
        E* dst = wu_slot(I) + (hf * 8 * kWave + lane) * 4;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) st16(dst + ct * kWave * 4, wu[hf * 8 + ct]);
      }
    }
  }
  for (int s = I; s < 3; ++s) lds_barrier();

  // ---- 5. Qt_I^T = (Gamma Q_I)^T - sum_{J<=I} W_J^T A_qk,IJ^T and
  //         Ut_I^T = sum_{J<=I} U_J^T A_qk,IJ^T (rows = channel / value column).
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    floatx4 acc[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[ct][e] = hf ? 0.f : GQ[ct].get(e);
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      if (J > I) continue;
      const Frag16<E>& bop = hf ? aq[J] : naq[J];
      if (J < I) {
        const E* src = wu_slot(J) + (hf * 8 * kWave + lane) * 4;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          const Frag16<E> w = ld16(src + ct * kWave * 4);
          acc[ct] = mma16(acc[ct], w, bop);
        }
      } else {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) acc[ct] = mma16(acc[ct], wu[hf * 8 + ct], bop);
      }
    }
    if (!hf) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        Frag<E> f;
#pragma unroll
        for (int e = 0; e < 4; ++e) { f.set(e, acc[2 * kb][e]); f.set(4 + e, acc[2 * kb + 1][e]); }
        store_frag(XA + ((4 + I) * 4 + kb) * kWave * 8, lane, f);
      }
    } else {
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) store_c4(UC + (ct * 8 + 4 + I) * kWave * 4, lane, acc[ct]);
    }
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
