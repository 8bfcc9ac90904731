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
constexpr int kIntraThreads = 512;   // 8 waves
constexpr int kGS = kD + 4;          // LDS row stride of g (floats)
constexpr int kLS = kC + 4;          // LDS row stride of the 64 x 64 fp32 matrices
constexpr int kTS = 20;              // LDS row stride of 16 x 16 scratch blocks
constexpr int kBS = kC + 8;          // LDS row stride of the bf16 copies of Ti and P

// Staging layout of one chunk's q / k / v rows in LDS.
template <class E>
struct Stage {
  static constexpr int kRS = kD + 16 / (int)sizeof(E);   // 16-byte pad per row
  static constexpr bool kStageV = sizeof(E) == 2;        // fp32 v is read from global
  static constexpr int kPer16 = 16 / (int)sizeof(E);      // elements per 16 bytes
  static constexpr int kRow16 = kD / kPer16;              // 16-byte pieces per row
  static constexpr int kPieces = kC * kRow16 / kIntraThreads;  // per thread, per tensor
  static constexpr int kLA = kC * (kD / 4) / kIntraThreads;    // float4 of log alpha
};

// 16-byte vector of I/O elements (8 bf16 or 4 fp32).
template <class E>
using Vec16 = typename std::conditional<sizeof(E) == 2, bf16x8, float4>::type;

// acc += A (16x16) * B (16x16), fp32, operands in LDS (row strides lda, ldb).
__device__ __forceinline__ floatx4 blk16(floatx4 acc, const float* A, int lda,
                                         const float* B, int ldb, int r, int g) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = mma4(acc, A[r * lda + 4 * s + g], B[(4 * s + g) * ldb + r]);
  return acc;
}

// Workgroup barrier that waits for this wave's LDS traffic only: outstanding
// global loads (the next chunk's prefetch) and stores stay in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt unchanged
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Eight consecutive elements of an LDS row as an MFMA operand fragment.
__device__ __forceinline__ void lds_frag(const bf16* p, Frag<bf16>& f) {
  f.v = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void lds_frag(const float* p, Frag<float>& f) {
  load8(p, f.v);
}

// One chunk-head's inputs, prefetched into registers.
template <class E>
struct ChunkIn {
  Vec16<E> k[Stage<E>::kPieces], q[Stage<E>::kPieces];
  Vec16<E> v[Stage<E>::kStageV ? Stage<E>::kPieces : 1];
  float4 la[Stage<E>::kLA];
  float beta;
};

struct ChunkPos {
  int b, h, len;
  int64_t tok0;
};

__device__ __forceinline__ ChunkPos chunk_pos(int64_t item, int H, const int32_t* cu,
                                              const int32_t* chunk_offset, int n_seqs,
                                              int64_t T) {
  ChunkPos c;
  c.b = (int)(item / H);
  c.h = (int)(item % H);
  int lo = 0, hi = n_seqs;  // chunk_offset[lo] <= b < chunk_offset[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (chunk_offset[mid] <= c.b) lo = mid; else hi = mid;
  }
  const int64_t seq_start = cu ? cu[lo] : 0, seq_end = cu ? cu[lo + 1] : T;
  c.tok0 = seq_start + (int64_t)(c.b - chunk_offset[lo]) * kC;
  c.len = (int)min((int64_t)kC, seq_end - c.tok0);
  return c;
}

template <class E>
__device__ __forceinline__ void load_chunk(ChunkIn<E>& in, const ChunkPos& c, int t,
                                           const E* q, const E* k, const E* v,
                                           const float* log_alpha, const float* beta, int H) {
  using St = Stage<E>;
  const Vec16<E> zero16 = {};
  auto row = [&](int i) -> int64_t { return ((c.tok0 + i) * H + c.h) * (int64_t)kD; };
#pragma unroll
  for (int u = 0; u < St::kPieces; ++u) {
    const int pc = t + u * kIntraThreads, i = pc / St::kRow16, col = (pc % St::kRow16) * St::kPer16;
    in.k[u] = i < c.len ? *reinterpret_cast<const Vec16<E>*>(k + row(i) + col) : zero16;
    in.q[u] = i < c.len ? *reinterpret_cast<const Vec16<E>*>(q + row(i) + col) : zero16;
    if constexpr (St::kStageV)
      in.v[u] = i < c.len ? *reinterpret_cast<const Vec16<E>*>(v + row(i) + col) : zero16;
  }
#pragma unroll
  for (int u = 0; u < St::kLA; ++u) {
    const int pc = t + u * kIntraThreads, i = pc / (kD / 4), col = (pc % (kD / 4)) * 4;
    in.la[u] = i < c.len ? *reinterpret_cast<const float4*>(log_alpha + row(i) + col)
                         : float4{0.f, 0.f, 0.f, 0.f};
  }
  in.beta = (t < kC && t < c.len) ? beta[(c.tok0 + t) * H + c.h] : 0.f;
}

// Persistent over (chunk, head) items: while one item is computed, the next
// one's inputs are already on their way into registers.
template <class E>
__global__ __launch_bounds__(kIntraThreads) void intra_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_offset,
    const int32_t* __restrict__ status, int32_t n_seqs, int64_t T, int32_t H,
    uint8_t* __restrict__ inter) {
  using St = Stage<E>;
  constexpr int RS = St::kRS;
  constexpr bool kStageV = St::kStageV;
  // LDS, by lifetime:
  //   rA   g (steps 0-2), then the bf16 Ti / P copies and 16x16 scratch
  //   sK   k, then Kr = k exp(g - g_s)        (row factor, s = block start)
  //   sQ   q, then Qr = q exp(g - g_s)
  //   sV   v, then beta v                      (bf16 only)
  //   rE   Kf = k exp(g_e - g) (steps 1-2, e = block end), then Ti | A_qk
  //   sL   L, then P = A_qk Ti
  //   sF   per block / block pair / channel factors
  __shared__ __attribute__((aligned(16))) float rA[kC * kGS];
  __shared__ __attribute__((aligned(16))) E sK[kC * RS];
  __shared__ __attribute__((aligned(16))) E sQ[kC * RS];
  __shared__ __attribute__((aligned(16))) E sV[kStageV ? kC * RS : 8];
  __shared__ __attribute__((aligned(16))) float rE[2 * kC * kLS];
  __shared__ __attribute__((aligned(16))) float sL[kC * kLS];
  __shared__ __attribute__((aligned(16))) float sF[(4 + 4 + 10) * kD];
  __shared__ float sb[kC];
  float* const sg = rA;
  E* const sKf = reinterpret_cast<E*>(rE);
  float* const sTi = rE;
  float* const sAqk = rE + kC * kLS;
  float* const sEs = sF;              // exp(g_s[c]) per block start s
  float* const sEc = sF + 4 * kD;     // exp(g_C[c] - g_e[c]) per block end e
  float* const sDf = sF + 8 * kD;     // exp(g_{s_I}[c] - g_{e_J}[c]), pair index below
  bf16* const sTib = reinterpret_cast<bf16*>(rA);            // bf16 Ti, rows of kBS
  bf16* const sPb = reinterpret_cast<bf16*>(rA) + kC * kBS;  // bf16 P
  float* const stmp = rA + kC * kBS;                         // after both bf16 copies

  if (status[0] != 0) return;
  const int64_t n_items = (int64_t)chunk_offset[n_seqs] * H;
  int64_t item = blockIdx.x;
  if (item >= n_items) return;

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int r = lane & 15, g = lane >> 4;
  // block pair (I, J <= I) -> index into sDf
  auto pidx = [](int I, int J) { return I * (I + 1) / 2 + J; };

  ChunkIn<E> in;
  ChunkPos cp = chunk_pos(item, H, cu, chunk_offset, n_seqs, T);
  load_chunk<E>(in, cp, t, q, k, v, log_alpha, beta, H);

  for (; item < n_items; item += gridDim.x) {
    const int len = cp.len, h = cp.h;
    const int64_t tok0 = cp.tok0;
    E* blk = reinterpret_cast<E*>(inter + ((int64_t)cp.b * H + h) * Inter<E>::kBytes);
    E* XA = blk + Inter<E>::kXA;
    E* KT = blk + Inter<E>::kKT;
    E* UC = blk + Inter<E>::kUC;
    float* GC = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(blk) + Inter<E>::kGCByte);

    // ---- 0. stage this chunk (rows past the sequence end are zeros, i.e.
    //         identity tokens), then start fetching the next one.
#pragma unroll
    for (int u = 0; u < St::kPieces; ++u) {
      const int pc = t + u * kIntraThreads, i = pc / St::kRow16, c = (pc % St::kRow16) * St::kPer16;
      *reinterpret_cast<Vec16<E>*>(&sK[i * RS + c]) = in.k[u];
      *reinterpret_cast<Vec16<E>*>(&sQ[i * RS + c]) = in.q[u];
      if constexpr (kStageV) *reinterpret_cast<Vec16<E>*>(&sV[i * RS + c]) = in.v[u];
    }
#pragma unroll
    for (int u = 0; u < St::kLA; ++u) {
      const int pc = t + u * kIntraThreads, i = pc / (kD / 4), c = (pc % (kD / 4)) * 4;
      *reinterpret_cast<float4*>(&sg[i * kGS + c]) = in.la[u];
    }
    if (t < kC) sb[t] = in.beta;
    lds_barrier();

    // ---- 1. gate: g = inclusive cumsum of log alpha along the chunk, in
    //         four 16-row segments per channel plus segment offsets.
    {
      const int c = t & 127, seg = t >> 7;
      float acc = 0.f;
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) {
        acc += sg[(16 * seg + ii) * kGS + c];
        sg[(16 * seg + ii) * kGS + c] = acc;
      }
      lds_barrier();
      float off = 0.f;
#pragma unroll
      for (int u = 0; u < 3; ++u) off += u < seg ? sg[(16 * u + 15) * kGS + c] : 0.f;
      lds_barrier();
      if (seg > 0) {
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) sg[(16 * seg + ii) * kGS + c] += off;
      }
    }
    lds_barrier();

    // ---- 1b. decay factors, each computed once. For row r in 16-row block
    //          with start s and end e: row factor exp(g_r - g_s) <= 1 and
    //          column factor exp(g_e - g_r) <= 1. The column factor of block
    //          pair (I, J) is exp(g_{s_I} - g_r) = Kf_r * D_IJ with
    //          D_IJ = exp(g_{s_I} - g_{e_J}): <= 1 for J < I; for J = I it
    //          can be large, and past e^44 the block is recomputed exactly.
    {
      // eight consecutive channels of one row per step
#pragma unroll 1
      for (int u = 0; u < kC * kD / 8 / kIntraThreads; ++u) {
        const int x = t + u * kIntraThreads, i = x >> 4, c0 = (x & 15) * 8;
        const int s = i & ~15, e = s + 15;
        float gi[8], gs[8], ge[8], kv[8], qv[8], fr[8], fc[8];
        load8(&sg[i * kGS + c0], gi);
        load8(&sg[s * kGS + c0], gs);
        load8(&sg[e * kGS + c0], ge);
        load8(&sK[i * RS + c0], kv);
        load8(&sQ[i * RS + c0], qv);
#pragma unroll
        for (int z = 0; z < 8; ++z) {
          fr[z] = exp_f(gi[z] - gs[z]);
          fc[z] = exp_f(ge[z] - gi[z]);
        }
        Frag<E> a, b2, c2;
#pragma unroll
        for (int z = 0; z < 8; ++z) {
          a.set(z, kv[z] * fr[z]);
          b2.set(z, qv[z] * fr[z]);
          c2.set(z, kv[z] * fc[z]);
        }
        store8(&sK[i * RS + c0], a);
        store8(&sQ[i * RS + c0], b2);
        store8(&sKf[i * RS + c0], c2);
        if constexpr (kStageV) {
          float vv[8];
          load8(&sV[i * RS + c0], vv);
          const float bi = sb[i];
          Frag<E> d2;
#pragma unroll
          for (int z = 0; z < 8; ++z) d2.set(z, vv[z] * bi);
          store8(&sV[i * RS + c0], d2);
        }
      }
      if (t < kD) {
        const int c = t;
        const float gC = sg[(kC - 1) * kGS + c];
        GC[c] = exp_f(gC);
#pragma unroll
        for (int bI = 0; bI < 4; ++bI) {
          sEs[bI * kD + c] = exp_f(sg[(16 * bI) * kGS + c]);
          sEc[bI * kD + c] = exp_f(gC - sg[(16 * bI + 15) * kGS + c]);
        }
      } else if (t < 2 * kD) {
        const int c = t - kD;
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
          for (int J = 0; J <= I; ++J)
            sDf[pidx(I, J) * kD + c] = exp_f(fminf(sg[(16 * I) * kGS + c] - sg[(16 * J + 15) * kGS + c], 88.f));
      }
    }
    lds_barrier();

    // ---- 2. A_kk (strict) and A_qk (inclusive) on 16 x 16 blocks (I, J):
    //         waves 0-3 (3, w); 4-5 (2, w-4); 6 (2,2)+(0,0); 7 (1,0)+(1,1).
    //         Accumulators stay in registers across the barrier that ends
    //         the reads of Kf (whose storage becomes Ti / A_qk).
    floatx4 akk[2], aqk[2];
    {
      auto pair = [&](int u, int& I, int& J) {
        if (w < 4) { I = u == 0 ? 3 : -1; J = w; }
        else if (w < 6) { I = u == 0 ? 2 : -1; J = w - 4; }
        else if (w == 6) { I = u == 0 ? 2 : 0; J = I; }
        else { I = 1; J = u; }
      };
      bool wide[2] = {false, false};
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        akk[u] = zero4();
        aqk[u] = zero4();
        int I, J;
        pair(u, I, J);
        if (I < 0) continue;
        const int R = 16 * I + r, i = 16 * J + r;
        const float* D = sDf + pidx(I, J) * kD;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const int c0 = 32 * kb + 8 * g;
          Frag<E> fk, fq, fb;
          lds_frag(&sK[R * RS + c0], fk);
          lds_frag(&sQ[R * RS + c0], fq);
          float kf[8];
          load8(&sKf[i * RS + c0], kf);
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
      // K'^T fragments for the sequential kernel, K'_i = k_i exp(g_C - g_i) =
      // Kf_i exp(g_C - g_e): wave w owns key channels [16 w, 16 w + 16); token
      // index in the split order the sequential kernel consumes.
      {
        const int m = w, cc = 16 * m + r;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const float ec0 = sEc[(2 * kb) * kD + cc], ec1 = sEc[(2 * kb + 1) * kD + cc];
          Frag<E> fkt;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int i = 32 * kb + split_k(g, e);
            fkt.set(e, (e < 4 ? ec0 : ec1) * to_f(sKf[i * RS + cc]));
          }
          store_frag(KT + (m * 2 + kb) * kWave * 8, lane, fkt);
        }
      }
      lds_barrier();
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        int I, J;
        pair(u, I, J);
        if (I < 0) continue;
        if (J == I && __ballot(wide[u])) {
          // exact diagonal block from the raw inputs: entries
          // (Rr = 16 I + 4 g + e, i = 16 I + r)
          auto row = [&](int x) -> int64_t { return ((tok0 + x) * H + h) * (int64_t)kD; };
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int Rr = 16 * I + 4 * g + e, i = 16 * I + r;
            float skk = 0.f, sqk = 0.f;
            if (i <= Rr && Rr < len) {
              for (int c = 0; c < kD; ++c) {
                const float d = exp_f(sg[Rr * kGS + c] - sg[i * kGS + c]);
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
    }
    // upper 16 x 16 blocks of Ti and L (later P) must read as zero; A_qk's
    // upper blocks are never read
    for (int x = t; x < 6 * 256; x += kIntraThreads) {
      const int blkid = x >> 8, e = x & 255;
      const int I = blkid < 3 ? 0 : (blkid < 5 ? 1 : 2);
      const int J = blkid < 3 ? blkid + 1 : (blkid < 5 ? blkid - 1 : 3);
      const int o = (16 * I + (e >> 4)) * kLS + 16 * J + (e & 15);
      sTi[o] = 0.f;
      sL[o] = 0.f;
    }
    lds_barrier();
    {
      auto pair = [&](int u, int& I, int& J) {
        if (w < 4) { I = u == 0 ? 3 : -1; J = w; }
        else if (w < 6) { I = u == 0 ? 2 : -1; J = w - 4; }
        else if (w == 6) { I = u == 0 ? 2 : 0; J = I; }
        else { I = 1; J = u; }
      };
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        int I, J;
        pair(u, I, J);
        if (I < 0) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int Rr = 16 * I + 4 * g + e, i = 16 * J + r;
          sL[Rr * kLS + i] = i < Rr ? sb[Rr] * akk[u][e] : 0.f;
          sAqk[Rr * kLS + i] = i <= Rr ? aqk[u][e] : 0.f;
        }
      }
    }
    lds_barrier();

    // ---- 3. Ti = (I + L)^{-1}: diagonal 16 x 16 blocks by forward
    //         substitution (one column per lane, waves 0-3), then the
    //         off-diagonal blocks Ti_IJ = -Ti_II sum_{K=J}^{I-1} L_IK Ti_KJ,
    //         level by level.
    // (I + L_bb)^{-1} for a strictly lower 16 x 16 block: L_bb^16 = 0, so
    // the inverse is exactly (I - L)(I + L^2)(I + L^4)(I + L^8). Wave w < 4
    // inverts block w with six fp32 block products; the temporaries live in
    // g's storage (dead after step 2) and only this wave touches them.
    if (w < 4) {
      float* tmp = rA + w * (4 * 16 * kTS);      // L2 | L4 | L8 | product
      float* L2 = tmp;
      float* L4 = tmp + 16 * kTS;
      float* L8 = tmp + 2 * 16 * kTS;
      float* X = tmp + 3 * 16 * kTS;
      const float* Lb = &sL[(16 * w) * kLS + 16 * w];
      auto put = [&](float* dst, int ld, floatx4 v4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(4 * g + e) * ld + r] = v4[e];
      };
      put(L2, kTS, blk16(zero4(), Lb, kLS, Lb, kLS, r, g));
      put(L4, kTS, blk16(zero4(), L2, kTS, L2, kTS, r, g));
      put(L8, kTS, blk16(zero4(), L4, kTS, L4, kTS, r, g));
      // A = (I - L) + (I - L) L2
      floatx4 a4 = zero4();
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int kk = 4 * s4 + g;
        const float av = (r == kk ? 1.f : 0.f) - Lb[r * kLS + kk];
        a4 = mma4(a4, av, L2[kk * kTS + r]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = 4 * g + e;
        a4[e] += (rr == r ? 1.f : 0.f) - Lb[rr * kLS + r];
      }
      put(X, kTS, a4);
      // B = A + A L4, then Ti_bb = B + B L8
      floatx4 b4 = blk16(zero4(), X, kTS, L4, kTS, r, g);
#pragma unroll
      for (int e = 0; e < 4; ++e) b4[e] += a4[e];
      put(X, kTS, b4);
      floatx4 x4 = blk16(zero4(), X, kTS, L8, kTS, r, g);
#pragma unroll
      for (int e = 0; e < 4; ++e) x4[e] += b4[e];
      put(&sTi[(16 * w) * kLS + 16 * w], kLS, x4);
    }
    lds_barrier();
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
      lds_barrier();
      if (w < 4 - d) {
        const int I = d + w, J = w;
        floatx4 acc = blk16(zero4(), &sTi[(16 * I) * kLS + 16 * I], kLS, &stmp[w * 16 * kTS], kTS, r, g);
#pragma unroll
        for (int e = 0; e < 4; ++e) sTi[(16 * I + 4 * g + e) * kLS + 16 * J + r] = -acc[e];
      }
      lds_barrier();
    }

    // ---- 4. P = A_qk Ti (lower triangular) into sL's storage; 20 block
    //         products over 7 waves: (3,0) | (3,1) | (2,0) | (3,2)+(0,0) |
    //         (2,1)+(1,1) | (1,0)+(2,2) | (3,3). Then bf16 copies of Ti, P.
    {
      auto plan = [&](int u, int& I, int& J) {
        switch (w) {
          case 0: I = u == 0 ? 3 : -1; J = 0; break;
          case 1: I = u == 0 ? 3 : -1; J = 1; break;
          case 2: I = u == 0 ? 2 : -1; J = 0; break;
          case 3: I = u == 0 ? 3 : 0; J = u == 0 ? 2 : 0; break;
          case 4: I = u == 0 ? 2 : 1; J = u == 0 ? 1 : 1; break;
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
    lds_barrier();
    // the next item's inputs are fetched while steps 5-6 run (issued here
    // rather than earlier to keep the registers they occupy off the peak)
    if (item + gridDim.x < n_items) {
      cp = chunk_pos(item + gridDim.x, H, cu, chunk_offset, n_seqs, T);
      load_chunk<E>(in, cp, t, q, k, v, log_alpha, beta, H);
    }
    const float* sP = sL;
    if constexpr (sizeof(E) == 2) {
      {
        const int i = t >> 3, c0 = (t & 7) * 8;   // 64 rows x 8 groups of 8
        float a8[8], b8[8];
        load8(&sTi[i * kLS + c0], a8);
        load8(&sP[i * kLS + c0], b8);
        Frag<bf16> fa8, fb8;
#pragma unroll
        for (int z = 0; z < 8; ++z) { fa8.set(z, a8[z]); fb8.set(z, b8[z]); }
        store8(&sTib[i * kBS + c0], fa8);
        store8(&sPb[i * kBS + c0], fb8);
      }
      lds_barrier();
    }
    // rows of Ti and P as operand fragments (bf16 copies or the fp32 originals)
    auto mat_frag = [&](bool isP, int R, int k0, Frag<E>& f) {
      if constexpr (sizeof(E) == 2) lds_frag((isP ? sPb : sTib) + R * kBS + k0, f);
      else lds_frag((isP ? sP : sTi) + R * kLS + k0, f);
    };

    // ---- 5. [-W^T | Qt^T] = (-B1)^T [Ti^T | P^T] + [0 | (Gamma*Q)^T] with
    //         B1 = Diag(beta)(Gamma*K) = Diag(beta) exp(g_s) Kr and
    //         Gamma*Q = exp(g_s) Qr. Wave w owns key channels [16 w, 16 w + 16).
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
        const float4 es = *reinterpret_cast<const float4*>(&sEs[(R >> 4) * kD + c4]);
        acc[nt][0] = es.x * qv[0];
        acc[nt][1] = es.y * qv[1];
        acc[nt][2] = es.z * qv[2];
        acc[nt][3] = es.w * qv[3];
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        Frag<E> fa;
        {
          const int i0 = 32 * kb + 8 * g;                 // standard order: one block
          const float es = -sEs[(i0 >> 4) * kD + cc];
#pragma unroll
          for (int e = 0; e < 8; ++e) fa.set(e, sb[i0 + e] * es * to_f(sK[(i0 + e) * RS + cc]));
        }
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          Frag<E> fb;
          mat_frag(nt >= 4, 16 * (nt & 3) + r, 32 * kb + 8 * g, fb);
          acc[nt] = mma(acc[nt], fa, fb);
        }
      }
      // these 16 channels are slots 0-3 (even m) or 4-7 (odd m) of the
      // sequential kernel's A-fragment (row tile nt, k-block m / 2)
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
        store_half_frag(XA + (nt * 4 + (m >> 1)) * kWave * 8, lane, m & 1, acc[nt]);
    }

    // ---- 6. U = Ti (beta V) (C-fragments, rows = token) and
    //         Ut^T = (beta V)^T P^T (C-fragments, rows = value column); the
    //         same (beta V) fragment is the B operand of one and the A operand
    //         of the other. Wave w owns value columns [16 w, 16 w + 16).
    {
      const int jt = w, j = 16 * jt + r;
      floatx4 acc[8];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) acc[mt] = zero4();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        Frag<E> fv;
        const int i0 = 32 * kb + 8 * g;
        if constexpr (kStageV) {
#pragma unroll
          for (int e = 0; e < 8; ++e) fv.v[e] = sV[(i0 + e) * RS + j];
        } else {
          auto row = [&](int x) -> int64_t { return ((tok0 + x) * H + h) * (int64_t)kD; };
#pragma unroll
          for (int e = 0; e < 8; ++e)
            fv.set(e, i0 + e < len ? sb[i0 + e] * to_f(v[row(i0 + e) + j]) : 0.f);
        }
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
          Frag<E> fm;
          mat_frag(mt >= 4, 16 * (mt & 3) + r, i0, fm);
          acc[mt] = mt < 4 ? mma(acc[mt], fm, fv) : mma(acc[mt], fv, fm);
        }
      }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) store_c4(UC + (jt * 8 + mt) * kWave * 4, lane, acc[mt]);
    }
    lds_barrier();   // every LDS read of this item precedes the next staging
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
    // persistent: one workgroup per CU (the kernel's LDS allows one), each
    // looping over (chunk, head) items
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
      (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int64_t items = n_slots * (int64_t)H;
    const unsigned grid = (unsigned)std::min<int64_t>(items, std::max(cus, 1));
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
