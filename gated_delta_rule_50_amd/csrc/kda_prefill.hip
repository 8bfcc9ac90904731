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
// One workgroup per (chunk, head); two fit on a CU (LDS <= 80 KiB, <= 128
// VGPRs), so one workgroup's loads overlap the other's compute.
constexpr int kIntraThreads = 512;   // 8 waves
constexpr int kLS = kC + 4;          // row stride (floats) of the 64 x 64 fp32 buffers
constexpr int kTS = 20;              // row stride of 16 x 16 fp32 scratch blocks

// Staged rows: 128 elements per row, no padding; 16-byte pieces are XOR
// swizzled by the row (piece p of row i sits at p ^ (i & 15) for bf16, at
// p ^ (i & 31) for fp32) so row reads, column gathers and row writes by
// lanes of different rows hit different banks.
template <class E>
struct Rows {
  static constexpr int kPer16 = 16 / (int)sizeof(E);   // elements per piece
  static constexpr int kPieces = kD / kPer16;           // pieces per row
  __device__ static int at(int i, int c) {               // element offset of (i, c)
    const int p = (c / kPer16) ^ (i & (kPieces - 1));
    return i * kD + p * kPer16 + c % kPer16;
  }
};

// 64 x 64 bf16 matrix, 8 pieces per row, swizzled the same way.
__device__ __forceinline__ int mat_at(int i, int c) {
  return i * kC + (((c >> 3) ^ (i & 7)) << 3) + (c & 7);
}

template <class E>
using Vec16 = typename std::conditional<sizeof(E) == 2, bf16x8, float4>::type;

// Workgroup barrier that waits for this wave's LDS traffic only (outstanding
// global stores stay in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Eight consecutive elements as an MFMA fragment.
__device__ __forceinline__ void lds_frag(const bf16* p, Frag<bf16>& f) {
  f.v = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void lds_frag(const float* p, Frag<float>& f) { load8(p, f.v); }

// Element (r, k) of a 16 x 16 block of Ti, stored strictly lower in `M`
// (row stride kLS) with an implied unit diagonal and zero upper part.
__device__ __forceinline__ float ti_at(const float* M, int R, int K) {
  return K < R ? M[R * kLS + K] : (K == R ? 1.f : 0.f);
}

template <class E>
__global__ __launch_bounds__(kIntraThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void intra_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_offset,
    const int32_t* __restrict__ status, int32_t n_seqs, int64_t T, int32_t H,
    uint8_t* __restrict__ inter) {
  using R = Rows<E>;
  // LDS, by lifetime:
  //   sK   k, then Kr = k exp(g - g_s)          (s = first row of the 16-row block)
  //   sQ   q, then Qr = q exp(g - g_s)
  //   rM   Kf = k exp(g_e - g) (e = last row of the block), until the A tiles
  //        are done; then M1 = [L strictly lower | A_qk^T upper + diagonal]
  //        and M2 = [Ti strictly lower | P^T upper + diagonal]; after P, M1's
  //        storage takes the bf16 copies of Ti and P (bf16 I/O)
  //   sF   per block / block-pair / channel factors
  //   sX   per (block, channel) sums of log alpha, later 16 x 16 scratch
  __shared__ __attribute__((aligned(16))) E sK[kC * kD];
  __shared__ __attribute__((aligned(16))) E sQ[kC * kD];
  __shared__ __attribute__((aligned(16))) float rM[2 * kC * kLS];
  __shared__ __attribute__((aligned(16))) float sF[(4 + 4 + 10) * kD];
  __shared__ __attribute__((aligned(16))) float sX[3 * 16 * kTS];
  __shared__ float sb[kC];
  E* const sKf = reinterpret_cast<E*>(rM);
  float* const M1 = rM;
  float* const M2 = rM + kC * kLS;
  bf16* const sTib = reinterpret_cast<bf16*>(rM);
  bf16* const sPb = reinterpret_cast<bf16*>(rM) + kC * kC;
  float* const sEs = sF;              // exp(g_s[c]) per block
  float* const sEc = sF + 4 * kD;     // exp(g_C[c] - g_e[c]) per block
  float* const sDf = sF + 8 * kD;     // exp(g_{s_I}[c] - g_{e_J}[c]), J <= I
  float* const xTot = sX;             // per-block sums of log alpha (4 x 128)
  float* const stmp = sX;             // 3 scratch blocks (after the exchange)

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

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int r = lane & 15, g = lane >> 4;
  auto row = [&](int i) -> int64_t { return ((tok0 + i) * H + h) * (int64_t)kD; };
  auto pidx = [](int I, int J) { return I * (I + 1) / 2 + J; };

  E* blk = reinterpret_cast<E*>(inter + ((int64_t)b * H + h) * Inter<E>::kBytes);
  E* XA = blk + Inter<E>::kXA;
  E* KT = blk + Inter<E>::kKT;
  E* UC = blk + Inter<E>::kUC;
  float* GC = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(blk) + Inter<E>::kGCByte);

  // ---- 0. loads, all issued up front. k and q rows go to LDS; each thread
  //         keeps one channel c of one 16-row block of log alpha.
  const int cch = t & 127, seg = t >> 7;       // channel, 16-row block
  float la[16];
  {
    constexpr int kPer = kC * R::kPieces / kIntraThreads;
    Vec16<E> vk[kPer], vq[kPer];
    const Vec16<E> zero16 = {};
    // Rows past the sequence end (identity tokens) are loaded from the last
    // valid row and replaced by zeros with a select: no branches, no
    // out-of-range addresses (a chunk always has len >= 1).
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int pc = t + u * kIntraThreads, i = pc / R::kPieces, c = (pc % R::kPieces) * R::kPer16;
      const int ic = min(i, len - 1);
      const Vec16<E> a = *reinterpret_cast<const Vec16<E>*>(k + row(ic) + c);
      const Vec16<E> b2 = *reinterpret_cast<const Vec16<E>*>(q + row(ic) + c);
      vk[u] = i < len ? a : zero16;
      vq[u] = i < len ? b2 : zero16;
    }
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) {
      const int i = 16 * seg + ii;
      const float x = log_alpha[row(min(i, len - 1)) + cch];
      la[ii] = i < len ? x : 0.f;
    }
    if (t < kC) {
      const float x = beta[(tok0 + min(t, len - 1)) * H + h];
      sb[t] = t < len ? x : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int pc = t + u * kIntraThreads, i = pc / R::kPieces, c = (pc % R::kPieces) * R::kPer16;
      *reinterpret_cast<Vec16<E>*>(&sK[R::at(i, c)]) = vk[u];
      *reinterpret_cast<Vec16<E>*>(&sQ[R::at(i, c)]) = vq[u];
    }
  }

  // ---- 1. gate: in-register cumsum of this thread's 16 log alphas, block
  //         offsets through LDS, then g_i for the thread's rows.
#pragma unroll
  for (int ii = 1; ii < 16; ++ii) la[ii] += la[ii - 1];
  xTot[seg * kD + cch] = la[15];
  lds_barrier();
  {
    float off = 0.f;
#pragma unroll
    for (int u = 0; u < 3; ++u) off += u < seg ? xTot[u * kD + cch] : 0.f;
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) la[ii] += off;          // la[] now holds g
  }
  // ---- 1b. decay factors for this thread's rows (each element once):
  //          Kr = k exp(g - g_s), Qr = q exp(g - g_s), Kf = k exp(g_e - g),
  //          all <= 1 in magnitude times the input. Per block and block pair:
  //          exp(g_s), exp(g_C - g_e), D_IJ = exp(g_{s_I} - g_{e_J}) (<= 1 for
  //          J < I), with g at a block's last row = sum of the block sums
  //          up to it.
#pragma unroll
  for (int ii = 0; ii < 16; ++ii) {
    const int i = 16 * seg + ii, o = R::at(i, cch);
    const float fr = exp_f(la[ii] - la[0]);
    const float fc = exp_f(la[15] - la[ii]);
    const float kv = to_f(sK[o]);
    sK[o] = from_f<E>(kv * fr);
    sQ[o] = from_f<E>(to_f(sQ[o]) * fr);
    sKf[o] = from_f<E>(kv * fc);
  }
  {
    float ge[4];
    ge[0] = xTot[cch];
#pragma unroll
    for (int J = 1; J < 4; ++J) ge[J] = ge[J - 1] + xTot[J * kD + cch];
    sEs[seg * kD + cch] = exp_f(la[0]);
    sEc[seg * kD + cch] = exp_f(ge[3] - la[15]);
    if (seg == 3) GC[cch] = exp_f(ge[3]);
#pragma unroll
    for (int J = 0; J < 4; ++J)
      if (J <= seg) sDf[pidx(seg, J) * kD + cch] = exp_f(fminf(la[0] - ge[J], 88.f));
  }
  lds_barrier();

  // ---- 2. A_kk (strict) and A_qk (inclusive) on 16 x 16 blocks (I, J):
  //         waves 0-3 (3, w); 4-5 (2, w-4); 6 (2,2)+(0,0); 7 (1,0)+(1,1).
  //         Column factor of pair (I, J): Kf * D_IJ. A diagonal block whose
  //         D could exceed e^44 is recomputed exactly from the raw inputs.
  auto pair = [&](int u, int& I, int& J) {
    if (w < 4) { I = u == 0 ? 3 : -1; J = w; }
    else if (w < 6) { I = u == 0 ? 2 : -1; J = w - 4; }
    else if (w == 6) { I = u == 0 ? 2 : 0; J = I; }
    else { I = 1; J = u; }
  };
  floatx4 akk[2], aqk[2];
  {
    bool wide[2] = {false, false};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      akk[u] = zero4();
      aqk[u] = zero4();
      int I, J;
      pair(u, I, J);
      if (I < 0) continue;
      const int Rw = 16 * I + r, i = 16 * J + r;
      const float* D = sDf + pidx(I, J) * kD;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int c0 = 32 * kb + 8 * g;
        Frag<E> fk, fq, fb;
        if constexpr (sizeof(E) == 2) {
          lds_frag(&sK[R::at(Rw, c0)], fk);
          lds_frag(&sQ[R::at(Rw, c0)], fq);
        } else {
          float a8[8], b8[8];
          load4(&sK[R::at(Rw, c0)], a8); load4(&sK[R::at(Rw, c0 + 4)], a8 + 4);
          load4(&sQ[R::at(Rw, c0)], b8); load4(&sQ[R::at(Rw, c0 + 4)], b8 + 4);
#pragma unroll
          for (int e = 0; e < 8; ++e) { fk.set(e, a8[e]); fq.set(e, b8[e]); }
        }
        float kf[8];
        if constexpr (sizeof(E) == 2) {
          load8(&sKf[R::at(i, c0)], kf);
        } else {
          load4(&sKf[R::at(i, c0)], kf); load4(&sKf[R::at(i, c0 + 4)], kf + 4);
        }
        const float4 d0 = *reinterpret_cast<const float4*>(D + c0);
        const float4 d1 = *reinterpret_cast<const float4*>(D + c0 + 4);
        const float dd[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (J == I && dd[e] > 1.2851e19f) wide[u] = true;   // e^44
          fb.set(e, kf[e] * dd[e]);
        }
        akk[u] = mma(akk[u], fk, fb);
        aqk[u] = mma(aqk[u], fq, fb);
      }
    }
    // K'^T fragments (K'_i = k_i exp(g_C - g_i) = Kf_i exp(g_C - g_e)) for
    // the sequential kernel: wave w owns channels [16 w, 16 w + 16), token
    // index in the split order.
    {
      const int cc = 16 * w + r;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const float ec0 = sEc[(2 * kb) * kD + cc], ec1 = sEc[(2 * kb + 1) * kD + cc];
        Frag<E> fkt;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 32 * kb + split_k(g, e);
          fkt.set(e, (e < 4 ? ec0 : ec1) * to_f(sKf[R::at(i, cc)]));
        }
        store_frag(KT + (w * 2 + kb) * kWave * 8, lane, fkt);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int I, J;
      pair(u, I, J);
      if (I < 0 || J != I || !__ballot(wide[u])) continue;
      // exact diagonal block: entries (Rr = 16 I + 4 g + e, i = 16 I + r),
      // g differences summed from the raw log alphas
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int Rr = 16 * I + 4 * g + e, i = 16 * I + r;
        float skk = 0.f, sqk = 0.f;
        if (i <= Rr && Rr < len) {
          for (int c = 0; c < kD; ++c) {
            float dg = 0.f;
            for (int x = i + 1; x <= Rr; ++x) dg += log_alpha[row(x) + c];
            const float d = exp_f(dg);
            const float kic = to_f(k[row(i) + c]);
            skk += to_f(k[row(Rr) + c]) * kic * d;
            sqk += to_f(q[row(Rr) + c]) * kic * d;
          }
        }
        akk[u][e] = skk;
        aqk[u][e] = sqk;
      }
    }
  }
  lds_barrier();   // Kf is dead: its storage becomes M1 / M2
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    int I, J;
    pair(u, I, J);
    if (I < 0) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int Rr = 16 * I + 4 * g + e, i = 16 * J + r;
      if (i < Rr) M1[Rr * kLS + i] = sb[Rr] * akk[u][e];       // L
      if (i <= Rr) M1[i * kLS + Rr] = aqk[u][e];                // A_qk^T
    }
  }
  lds_barrier();

  // ---- 3. Ti = (I + L)^{-1}: diagonal 16 x 16 blocks by forward
  //         substitution (one column per lane, waves 0-3), then off-diagonal
  //         blocks Ti_IJ = -Ti_II sum_{K=J}^{I-1} L_IK Ti_KJ level by level.
  if (w < 4 && lane < 16) {
    const int base = 16 * w, jj = lane;
    float x[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      asm volatile("" ::: "memory");   // row rr of L read just before use
      float sacc = rr == jj ? 1.f : 0.f;
#pragma unroll
      for (int ii = 0; ii < rr; ++ii) sacc -= M1[(base + rr) * kLS + base + ii] * x[ii];
      x[rr] = sacc;
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
      if (rr > jj) M2[(base + rr) * kLS + base + jj] = x[rr];
  }
  lds_barrier();
#pragma unroll
  for (int d = 1; d < 4; ++d) {
    if (w < 4 - d) {
      const int I = d + w, J = w;
      floatx4 acc = zero4();
      for (int K = J; K < I; ++K) {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int kk = 4 * s4 + g;
          acc = mma4(acc, M1[(16 * I + r) * kLS + 16 * K + kk],
                     K == J ? ti_at(M2, 16 * K + kk, 16 * J + r) - (kk == r ? 0.f : 0.f)
                            : M2[(16 * K + kk) * kLS + 16 * J + r]);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) stmp[w * 16 * kTS + (4 * g + e) * kTS + r] = acc[e];
    }
    lds_barrier();
    if (w < 4 - d) {
      const int I = d + w, J = w;
      floatx4 acc = zero4();
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int kk = 4 * s4 + g;
        acc = mma4(acc, ti_at(M2, 16 * I + r, 16 * I + kk), stmp[w * 16 * kTS + kk * kTS + r]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) M2[(16 * I + 4 * g + e) * kLS + 16 * J + r] = -acc[e];
    }
    lds_barrier();
  }

  // ---- 4. P = A_qk Ti (lower triangular), stored transposed in M2's upper
  //         part: 20 block products over 7 waves.
  {
    auto plan = [&](int u, int& I, int& J) {
      switch (w) {
        case 0: I = u == 0 ? 3 : -1; J = 0; break;
        case 1: I = u == 0 ? 3 : -1; J = 1; break;
        case 2: I = u == 0 ? 2 : -1; J = 0; break;
        case 3: I = u == 0 ? 3 : 0; J = u == 0 ? 2 : 0; break;
        case 4: I = u == 0 ? 2 : 1; J = 1; break;
        case 5: I = u == 0 ? 1 : 2; J = u == 0 ? 0 : 2; break;
        case 6: I = u == 0 ? 3 : -1; J = 3; break;
        default: I = -1; J = 0; break;
      }
    };
    floatx4 acc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      acc[u] = zero4();
      int I, J;
      plan(u, I, J);
      if (I < 0) continue;
      for (int K = J; K <= I; ++K) {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int kk = 4 * s4 + g;
          // A_qk[16 I + r][16 K + kk] from its transposed storage (zero above
          // the diagonal of a diagonal block)
          const float a = (K < I || kk <= r) ? M1[(16 * K + kk) * kLS + 16 * I + r] : 0.f;
          const float bm = K == J ? ti_at(M2, 16 * K + kk, 16 * J + r)
                                  : M2[(16 * K + kk) * kLS + 16 * J + r];
          acc[u] = mma4(acc[u], a, bm);
        }
      }
    }
    lds_barrier();   // every read of Ti's diagonal blocks precedes P's writes
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int I, J;
      plan(u, I, J);
      if (I < 0) continue;
      // lane holds P[16 I + 4 g + e][16 J + r] -> M2[16 J + r][16 I + 4 g + e]
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (I > J || 4 * g + e >= r) M2[(16 * J + r) * kLS + 16 * I + 4 * g + e] = acc[u][e];
    }
  }
  lds_barrier();
  // Rows of Ti and P as operand fragments: bf16 copies (row-major,
  // swizzled) for bf16 I/O, masked reads of M2 for fp32.
  if constexpr (sizeof(E) == 2) {
    const int i = t & 63, c0 = (t >> 6) * 8;
    Frag<bf16> ft, fp;
#pragma unroll
    for (int z = 0; z < 8; ++z) {
      const int c = c0 + z;
      ft.set(z, ti_at(M2, i, c));
      fp.set(z, c <= i ? M2[c * kLS + i] : 0.f);
    }
    lds_barrier();   // M1's storage (A_qk^T) is free once P is done
    store8(&sTib[mat_at(i, c0)], ft);
    store8(&sPb[mat_at(i, c0)], fp);
    lds_barrier();
  }
  auto mat_frag = [&](bool isP, int Rr, int k0, Frag<E>& f) {
    if constexpr (sizeof(E) == 2) {
      lds_frag((isP ? sPb : sTib) + mat_at(Rr, k0), f);
    } else {
#pragma unroll
      for (int z = 0; z < 8; ++z) {
        const int c = k0 + z;
        f.set(z, isP ? (c <= Rr ? M2[c * kLS + Rr] : 0.f) : ti_at(M2, Rr, c));
      }
    }
  };

  // v rows for step 6, fetched now so step 5 hides the latency (rows past
  // the end repeat the last row; step 6 multiplies them by beta = 0)
  constexpr int kPerV = kC * R::kPieces / kIntraThreads;
  Vec16<E> vvec[kPerV];
#pragma unroll
  for (int u = 0; u < kPerV; ++u) {
    const int pc = t + u * kIntraThreads, i = pc / R::kPieces, c = (pc % R::kPieces) * R::kPer16;
    vvec[u] = *reinterpret_cast<const Vec16<E>*>(v + row(min(i, len - 1)) + c);
  }

  // ---- 5. [-W^T | Qt^T] = (-B1)^T [Ti^T | P^T] + [0 | (Gamma*Q)^T] with
  //         B1 = Diag(beta) exp(g_s) Kr and Gamma*Q = exp(g_s) Qr. Wave w
  //         owns key channels [16 w, 16 w + 16).
  {
    const int cc = 16 * w + r, c4 = 16 * w + 4 * g;
    floatx4 acc[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      acc[nt] = zero4();
      if (nt < 4) continue;
      const int Rr = 16 * (nt - 4) + r;
      float qv[4];
      load4(&sQ[R::at(Rr, c4)], qv);
      const float4 es = *reinterpret_cast<const float4*>(&sEs[(Rr >> 4) * kD + c4]);
      acc[nt][0] = es.x * qv[0];
      acc[nt][1] = es.y * qv[1];
      acc[nt][2] = es.z * qv[2];
      acc[nt][3] = es.w * qv[3];
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      Frag<E> fa;
      const int i0 = 32 * kb + 8 * g;                 // standard order: one block
      const float es = -sEs[(i0 >> 4) * kD + cc];
#pragma unroll
      for (int e = 0; e < 8; ++e) fa.set(e, sb[i0 + e] * es * to_f(sK[R::at(i0 + e, cc)]));
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        Frag<E> fb;
        mat_frag(nt >= 4, 16 * (nt & 3) + r, i0, fb);
        acc[nt] = mma(acc[nt], fa, fb);
      }
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
      store_half_frag(XA + (nt * 4 + (w >> 1)) * kWave * 8, lane, w & 1, acc[nt]);
  }

  // v takes Kr's storage once every wave is past step 5
  lds_barrier();
  E* const sV = sK;
#pragma unroll
  for (int u = 0; u < kPerV; ++u) {
    const int pc = t + u * kIntraThreads, i = pc / R::kPieces, c = (pc % R::kPieces) * R::kPer16;
    *reinterpret_cast<Vec16<E>*>(&sV[R::at(i, c)]) = vvec[u];
  }
  lds_barrier();

  // ---- 6. U = Ti (beta V) (rows = token) and Ut^T = (beta V)^T P^T (rows =
  //         value column); the same (beta V) fragment serves as B and as A.
  //         Wave w owns value columns [16 w, 16 w + 16).
  {
    floatx4 acc[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[mt] = zero4();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int i0 = 32 * kb + 8 * g;
      Frag<E> fv;
#pragma unroll
      for (int e = 0; e < 8; ++e) fv.set(e, sb[i0 + e] * to_f(sV[R::at(i0 + e, 16 * w + r)]));
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        Frag<E> fm;
        mat_frag(mt >= 4, 16 * (mt & 3) + r, i0, fm);
        acc[mt] = mt < 4 ? mma(acc[mt], fm, fv) : mma(acc[mt], fv, fm);
      }
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) store_c4(UC + (w * 8 + mt) * kWave * 4, lane, acc[mt]);
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
