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

// Exact diagonal 16 x 16 blocks of A_kk and A_qk, for blocks whose decay is
// too strong for the factored form:
//   A_kk[i][j] = sum_c k_i[c] k_j[c] P_ij[c],  A_qk[i][j] = sum_c q_i[c] k_j[c] P_ij[c],
//   P_ij[c] = prod_{t=j+1..i} alpha_t[c] (j <= i; 1 on the diagonal),
// i.e. exp(g_i - g_j) formed as a product of decays <= 1, so nothing
// overflows whatever the gate. Lane (r, g) of the wave handles token i = r
// and reads its k, q and raw log alpha rows again (channels 16 ct + 4 g + e),
// so the caller keeps nothing extra live. Per 16-channel tile the wave
// stages alpha and k of its 16 tokens in LDS (`stage`, wave-private, 1 KiB
// of alpha + 16 x 16 E); every lane then walks the columns j = 15 .. 0 with
// a running product of its four channels. The sums over the lane's 32 channels are reduced over the
// four lanes of the row. Returns kk_t[e] = A_kk[i][4 g + e],
// qk_t[e] = A_qk[i][4 g + e] and kk_d[e] = A_kk[4 g + e][i], zero above the
// diagonal; tokens past the sequence end are identity tokens (k = q = 0,
// alpha = 1). With kNorm, rk and rq are the L2Norm scales of row i.
template <class E, bool kNorm>
__device__ __forceinline__ void exact_diag_block(const E* __restrict__ k_row,
                                                 const E* __restrict__ q_row,
                                                 const float* __restrict__ la_row, bool valid,
                                                 float rk, float rq, int r, int g, uint8_t* stage,
                                                 float (&kk_t)[4], float (&qk_t)[4],
                                                 float (&kk_d)[4]) {
  float* const sa = reinterpret_cast<float*>(stage);        // [16 tokens][16 channels]
  E* const sk = reinterpret_cast<E*>(stage + 16 * 16 * 4);   // [16 tokens][16 channels]
  float pkk[16], pqk[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) pkk[j] = pqk[j] = 0.f;
  const Frag16<E> zero = frag16<E>(zero4());
#pragma unroll 1
  for (int ct = 0; ct < 8; ++ct) {
    const int c0 = 16 * ct + 4 * g;
    const Frag16<E> ki = valid ? ld16(k_row + c0) : zero;
    const Frag16<E> qi = valid ? ld16(q_row + c0) : zero;
    const float4 l = *reinterpret_cast<const float4*>(la_row + c0);
    const float4 a = valid ? float4{exp_f(l.x), exp_f(l.y), exp_f(l.z), exp_f(l.w)}
                           : float4{1.f, 1.f, 1.f, 1.f};
    // the previous tile's reads are done before this tile's writes (LDS
    // operations of one wave complete in order; the clobbers keep the
    // compiler from moving accesses across)
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("" ::: "memory");
    *reinterpret_cast<float4*>(sa + r * 16 + 4 * g) = a;
    st16(sk + r * 16 + 4 * g, ki);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("" ::: "memory");
    float P[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int j = 15; j >= 0; --j) {
      if (j < 15) {
        const float4 an = *reinterpret_cast<const float4*>(sa + (j + 1) * 16 + 4 * g);
        const float av[4] = {an.x, an.y, an.z, an.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) P[e] = j < r ? P[e] * av[e] : P[e];
      }
      const Frag16<E> kj = ld16(sk + j * 16 + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float t = kj.get(e) * P[e];
        pkk[j] += ki.get(e) * t;
        pqk[j] += qi.get(e) * t;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) kk_t[e] = qk_t[e] = kk_d[e] = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float skk = sum_xor32(sum_xor16(pkk[j]));
    float sqk = sum_xor32(sum_xor16(pqk[j]));
    if constexpr (kNorm) {
      // L2Norm scales: row i's (rk, rq) and column j's rk (lane j + 16 g)
      const float rkj = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (j + 16 * g),
                                                                     __float_as_int(rk)));
      skk *= rk * rkj;
      sqk *= rq * rkj;
    }
    if (j > r) skk = sqk = 0.f;
    if (g == (j >> 2)) {
      kk_t[j & 3] = skk;
      qk_t[j & 3] = sqk;
    }
    // lane (j, g) takes A_kk[4 g + e][j] from lane (4 g + e, g)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = __int_as_float(
          __builtin_amdgcn_ds_bpermute(4 * ((4 * g + e) + 16 * g), __float_as_int(skk)));
      if (r == j) kk_d[e] = x;
    }
  }
}

template <class E, bool kNorm>
__global__ __launch_bounds__(kIntraThreads, sizeof(E) == 4 ? 2 : 1) void intra_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, int32_t* chunk_offset, int32_t* status, int32_t n_seqs,
    int64_t T, int32_t H, uint8_t* __restrict__ inter, int32_t single, int32_t W0) {
  // LDS, one region reused across phases:
  //   rows phase   sKf  Kf fragments of the four blocks [J][kb][lane][8]
  //                sF   per-block channel factors (five rows per block)
  //                sTot per-block sums of log alpha; sE = exp(sum), sEi = exp(-sum)
  //   tiles phase  sX   per block, 16 token-major accumulator tiles
  //                     [block][tile][lane][4]: beta Gamma K (tiles 0-7, key
  //                     channels) and beta V (8-15, value columns), each
  //                     replaced by W / U once solved
  //                sNL  -L_IJ (J < I) A-operand tiles [I][J]; sTI Ti_II^T tiles
  //                sB beta (read up to step 3, before the tiles phase
  //                overwrites the region)
  constexpr int kTile = kWave * 4;                        // elements per tile
  constexpr int kRowsBytes = 4 * 4 * kWave * 8 * (int)sizeof(E) + (5 + 3) * 4 * kD * 4;
  constexpr int kTilesBytes = (4 * 16 + 12 + 4) * kTile * (int)sizeof(E);
  // exact diagonal path: per wave, 16 x 16 alpha (fp32) and k (E) values,
  // placed after the rows-phase data
  constexpr int kStageBytes = 16 * 16 * (4 + (int)sizeof(E));
  static_assert(kRowsBytes + 4 * kStageBytes + kC * 4 <= kTilesBytes,
                "staging and sB fit the shared region");
  // (fp32 I/O: 80 KiB in all, so that two workgroups may share a CU)
  __shared__ __attribute__((aligned(16))) uint8_t smem[kRowsBytes > kTilesBytes ? kRowsBytes : kTilesBytes];
  float* const sB = reinterpret_cast<float*>(smem + kRowsBytes + 4 * kStageBytes);
  E* const sKf = reinterpret_cast<E*>(smem);
  float* const sF = reinterpret_cast<float*>(smem + 4 * 4 * kWave * 8 * sizeof(E));
  float* const sTot = sF + 4 * 5 * kD;
  float* const sE = sTot + 4 * kD;
  float* const sEi = sE + 4 * kD;
  E* const sX = reinterpret_cast<E*>(smem);
  E* const sNL = sX + 4 * 16 * kTile;
  E* const sTI = sNL + 12 * kTile;

  // Blocks run chunk-major from the last chunk slot down, all heads of a
  // chunk together: the carry kernel reads the chunks in ascending order, so
  // the blocks it needs first are the ones written last, still held in the
  // memory-side cache when it starts (1.19 -> 1.07 us per chunk of the carry
  // on the 8K workload with 32 heads).
  // The grid covers the window of chunk slots [W0, W0 + gridDim.x); blocks
  // are written to the window's part of the workspace.
  const int64_t lin = blockIdx.x + (int64_t)gridDim.x * blockIdx.y;
  const int bw = (int)(gridDim.x - 1 - lin / H), h = (int)(lin % H);
  const int b = W0 + bw;
  int total, first;
  int64_t seq_start, seq_end;
  if (single) {
    // one sequence: the chunk range and the cu_seqlens check need no chunk
    // map; the first block records them in the workspace as the map would
    const bool ok = cu == nullptr || (cu[0] == 0 && (int64_t)cu[1] == T);
    total = (int)((T + kC - 1) / kC);
    if (b == 0 && h == 0 && threadIdx.x == 0) {
      status[0] = ok ? 0 : 1;
      chunk_offset[0] = 0;
      chunk_offset[1] = total;
    }
    if (!ok) return;
    first = 0;
    seq_start = 0;
    seq_end = T;
  } else {
    if (status[0] != 0) return;
    total = chunk_offset[n_seqs];
    if (b >= total) return;
    int lo = 0, hi = n_seqs;  // chunk_offset[lo] <= b < chunk_offset[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (chunk_offset[mid] <= b) lo = mid; else hi = mid;
    }
    first = chunk_offset[lo];
    seq_start = cu ? cu[lo] : 0;
    seq_end = cu ? cu[lo + 1] : T;
  }
  if (b >= total) return;
  const int64_t tok0 = seq_start + (int64_t)(b - first) * kC;
  const int len = (int)min((int64_t)kC, seq_end - tok0);

  const int lane = threadIdx.x & 63;
  const int I = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // token block
  const int r = lane & 15, g = lane >> 4;
  const int i = 16 * I + r;
  const bool valid = i < len;
  auto row = [&](int x) -> int64_t { return ((tok0 + x) * H + h) * (int64_t)kD; };

  E* blk = reinterpret_cast<E*>(inter + ((int64_t)bw * H + h) * Inter<E>::kBytes);
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
  // optional L2Norm of the q and k rows: the row's 128 channels sit in the
  // four lanes r + 16 g; the scales are applied where the rows are first
  // used (in fp32); the exact diagonal path takes them from the lanes.
  float rk = 1.f, rq = 1.f;
  if constexpr (kNorm) {
    float kk = 0.f, qq = 0.f;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = kx[ct].get(e), c = qx[ct].get(e);
        kk += a * a;
        qq += c * c;
      }
    kk = sum_xor32(sum_xor16(kk));
    qq = sum_xor32(sum_xor16(qq));
    // hardware reciprocal square root (about 1 ulp), as the recurrent kernel
    rk = __builtin_amdgcn_rsqf(kk + kL2NormEps);
    rq = __builtin_amdgcn_rsqf(qq + kL2NormEps);
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
  bool wide = false;   // a channel decays by more than e^-44 over this block
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = lane + 64 * u;
    const float s = sTot[I * kD + c];
    sE[I * kD + c] = exp_f(s);
    sEi[I * kD + c] = exp_f(fminf(-s, 88.f));
    wide |= s < -44.f;
  }
  // Diagonal blocks whose factor exp(-block sum) could exceed e^44 are
  // computed per element instead (they replace the matrix-core tiles below);
  // done here, where little else is live. Staging area: the part of the
  // shared region the rows phase does not use.
  const bool exact = __builtin_amdgcn_ballot_w64(wide) != 0;
  float ex_kk[4], ex_qk[4], ex_kd[4];
  if (exact)
    exact_diag_block<E, kNorm>(k + ro, q + ro, log_alpha + ro, valid, rk, rq, r, g,
                               smem + kRowsBytes + I * kStageBytes, ex_kk, ex_qk, ex_kd);
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
        const float kv = kx[ct].get(e) * rk, fr = exp_f(la[ct][e]);
        kfI[kb].set(4 * hh + e, kv * exp_f(s[e] - la[ct][e]));
        Kr[ct].set(e, kv * fr);
        Qr[ct].set(e, qx[ct].get(e) * rq * fr);
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

  // v rows (identity tokens repeat the last valid row; beta = 0 zeroes them)
  Frag16<E> vx[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) vx[ct] = ld16(v + ro + 16 * ct + 4 * g);

  // A tiles. For J < I, A_kk[i][j] = sum_c (Kr_i D_IJ) Kf_j (same for A_qk
  // with Qr); the diagonal block uses D_II = exp(-block sum) >= 1, and where
  // that could exceed e^44 the block is recomputed exactly below. Lane (r, g)
  // accumulates akT[J][e] = A_kk[16I + r][16J + 4g + e],
  // aqT[J][e] = A_qk[16I + r][16J + 4g + e] and akD[e] = A_kk[16I + 4g + e][16I + r].
  floatx4 akT[4], aqT[4], akD = zero4();
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
        akT[J] = mma(akT[J], kfI[kb], fk);
        aqT[J] = mma(aqT[J], kfI[kb], fq);
        akD = mma(akD, fk, kfI[kb]);
      }
    }
  }

  // exact diagonal block (computed in step 1) in place of the factored one
  if (exact) {
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      if (J != I) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        akT[J][e] = ex_kk[e];
        aqT[J][e] = ex_qk[e];
        akD[e] = ex_kd[e];
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
  // A_qk (J <= I, masked on the diagonal) and its negation as B operands
  Frag16<E> aq[4], naq[4];
#pragma unroll
  for (int J = 0; J < 4; ++J) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = (J < I || 4 * g + e <= r) ? aqT[J][e] : 0.f;
      aq[J].set(e, x);
      naq[J].set(e, -x);
    }
  }

  // ---- 4. publish this block's operands of the solve: token-major beta
  //         Gamma K and beta V tiles (row pieces times the identity), -L_IJ
  //         and Ti_II^T. The rows-phase LDS is dead once every wave is here.
  lds_barrier();
  {
    E* const x = sX + (I * 16) * kTile + lane * 4;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      Frag16<E> vb;
#pragma unroll
      for (int e = 0; e < 4; ++e) vb.set(e, bt * vx[ct].get(e));
      st16(x + ct * kTile, frag16<E>(mma16(zero4(), Bx[ct], idf)));
      st16(x + (8 + ct) * kTile, frag16<E>(mma16(zero4(), vb, idf)));
    }
#pragma unroll
    for (int J = 0; J < 3; ++J) {
      if (J >= I) continue;
      Frag16<E> nl;
#pragma unroll
      for (int e = 0; e < 4; ++e) nl.set(e, -bt * akT[J][e]);
      st16(sNL + (I * 3 + J) * kTile + lane * 4, nl);
    }
    st16(sTI + I * kTile + lane * 4, tiT);
  }
  lds_barrier();

  // ---- 5. blocked forward substitution by tiles: wave w solves tiles
  //         4w .. 4w+3 of [W | U] for all four blocks in order,
  //           [W | U]_I = Ti_II ([B | V']_I - sum_{J<I} L_IJ [W | U]_J),
  //         keeping its own earlier blocks in registers (no barrier between
  //         blocks), and overwrites each [B | V'] tile with the result.
  {
    const int w = I;
    Frag16<E> sol[4][4];   // [block][tile]
#pragma unroll
    for (int Ib = 0; Ib < 4; ++Ib) {
      E* const x = sX + (Ib * 16 + 4 * w) * kTile + lane * 4;
      const Frag16<E> ti = ld16(sTI + Ib * kTile + lane * 4);
      floatx4 M[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const Frag16<E> b0 = ld16(x + t * kTile);
#pragma unroll
        for (int e = 0; e < 4; ++e) M[t][e] = b0.get(e);
      }
#pragma unroll
      for (int J = 0; J < 3; ++J) {
        if (J >= Ib) continue;
        const Frag16<E> nl = ld16(sNL + (Ib * 3 + J) * kTile + lane * 4);
#pragma unroll
        for (int t = 0; t < 4; ++t) M[t] = mma16(M[t], nl, sol[J][t]);
      }
      floatx4 wt[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const Frag16<E> mb = frag16<E>(M[t]);
        const floatx4 o = mma16(zero4(), ti, mb);     // token-major W / U tile
        sol[Ib][t] = frag16<E>(o);
        st16(x + t * kTile, sol[Ib][t]);
        if (w >= 2) store_c4(UC + ((4 * (w - 2) + t) * 8 + Ib) * kWave * 4, lane, o);
        else wt[t] = mma16(zero4(), mb, ti);          // W^T tile
      }
      if (w < 2) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          Frag<E> f;
#pragma unroll
          for (int e = 0; e < 4; ++e) { f.set(e, -wt[2 * kk][e]); f.set(4 + e, -wt[2 * kk + 1][e]); }
          store_frag(XA + (Ib * 4 + 2 * w + kk) * kWave * 8, lane, f);
        }
      }
    }
  }
  lds_barrier();

  // ---- 6. Qt_I^T = (Gamma Q_I)^T - sum_{J<=I} W_J^T A_qk,IJ^T and
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
      const E* src = sX + (J * 16 + hf * 8) * kTile + lane * 4;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) acc[ct] = mma16(acc[ct], ld16(src + ct * kTile), bop);
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

// ------------------------------------------------------------- windows
// The prefill runs over windows of chunk slots [W0, W1) (as many as the
// workspace holds blocks for), the intra-chunk kernel then the carry per
// window. A sequence whose chunks cross a window boundary leaves its state
// in the workspace's state area at the end of one window and picks it up
// at the start of the next: at most one sequence crosses each boundary, so
// the area holds one state per head, in two slots that alternate between
// windows (a window reads the slot the previous one wrote and writes the
// other).
// A sequence-head's state where a carry workgroup starts: the fp32 state
// the previous window left in the workspace, or the caller's h0 in the state
// type SE (float or bf16), or zeros.
template <class SE>
struct StateIn {
  const float* f;
  const SE* s;
  // S[mt][e] = state[16 mt + 4 g + e][j], the accumulator layout of a
  // 128 x 16 column tile (zeros when there is no state)
  __device__ void load(floatx4 (&S)[8], int g, int j) const {
    if (f) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[mt][e] = f[(16 * mt + 4 * g + e) * kD + j];
    } else if (s) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[mt][e] = to_f(s[(16 * mt + 4 * g + e) * kD + j]);
    } else {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) S[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  }
};
// Where it leaves the state: the next window's fp32 slot, or the caller's
// h_final in SE (rounded to nearest even for bf16), or nowhere.
template <class SE>
struct StateOut {
  float* f;
  SE* s;
  // row tiles [mt0, mt1) of the accumulator layout above
  template <int kMt0 = 0, int kMt1 = 8>
  __device__ void store(const floatx4 (&S)[8], int g, int j) const {
    if (f) {
#pragma unroll
      for (int mt = kMt0; mt < kMt1; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) f[(16 * mt + 4 * g + e) * kD + j] = S[mt][e];
    } else if (s) {
#pragma unroll
      for (int mt = kMt0; mt < kMt1; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[(16 * mt + 4 * g + e) * kD + j] = from_f<SE>(S[mt][e]);
    }
  }
};

struct WindowArgs {
  int32_t W0, W1;          // this window's chunk slots
  int32_t last;            // 1 for the last window of the call
  const float* resume;     // [H, 128, 128] state left by the previous window
  float* suspend;          // [H, 128, 128] state for the next window

  // The sequence's chunks [sb0, sb1) inside the window: [b0, b1). Returns
  // false when this window has nothing to do for the sequence. An empty
  // sequence (sb0 == sb1) is handled once, by the window holding slot sb0
  // (by the last window when sb0 is past every slot), which copies its
  // initial state to h_final.
  __device__ bool part(int sb0, int sb1, int& b0, int& b1) const {
    if (sb0 == sb1) {
      b0 = b1 = sb0;
      return (sb0 >= W0 && sb0 < W1) || (last && sb0 >= W1);
    }
    b0 = max(sb0, W0);
    b1 = min(sb1, W1);
    return b0 < b1;
  }
  // State at chunk b0: h0 (or NULL for zeros) at the sequence's first
  // chunk, else the state the previous window left.
  template <class SE>
  __device__ StateIn<SE> state_in(int sb0, int b0, const SE* h0, int pair, int h) const {
    if (b0 > sb0) return {resume + (int64_t)h * kD * kD, nullptr};
    return {nullptr, h0 ? h0 + (int64_t)pair * kD * kD : nullptr};
  }
  // Where the state after chunk b1 - 1 goes: h_final (or nowhere) after the
  // sequence's last chunk, else the next window's state slot.
  template <class SE>
  __device__ StateOut<SE> state_out(int sb1, int b1, SE* h_final, int pair, int h) const {
    if (b1 < sb1) return {suspend + (int64_t)h * kD * kD, nullptr};
    return {nullptr, h_final ? h_final + (int64_t)pair * kD * kD : nullptr};
  }
};

// ------------------------------------------------------- sequential carry
// One workgroup per (sequence, head, 16-column tile of the state), four
// waves (or per two tiles when there are many pairs; see carry_kernel).
// Per chunk:
//   state wave    X = U + [-W] S            pseudo-value (rows = token)
//                 S = Diag(gamma_C) S + K'^T X
//   output wave   O^T = Ut^T + S^T Qt^T     (rows = value column)
//   loader waves  stream the state wave's operands into an LDS ring; one
//                 of them also stores the output wave's O tiles
// Wave 3 (a loader) also touches one word per 128-byte line of this
// workgroup's share of the block kTouchAhead chunks ahead (an eighth six
// chunks ahead, or a quarter four ahead with two tiles; buffer->LDS loads
// into a scratch slot, no registers), so
// the loaders and the output wave find the blocks in L2 rather than waiting
// on HBM.
// The state never leaves the state wave's registers; its accumulator tiles
// feed the next products directly in the split K order. At the end of each
// chunk the state wave also publishes the new state as bf16 operand
// fragments in one of two LDS buffers, which the output wave uses in the
// next chunk, so one workgroup barrier per chunk orders everything and only
// 32 of the 48 products per chunk sit on the sequential path.
//
// bf16 intermediates: the loaders keep chunks b+2 and b+3 of [-W], K'^T,
// the tiles' U and gamma_C in flight (buffer->LDS DMA into a three-slot
// ring, each loader below the hardware's outstanding-load limit); a state
// wave reads chunk b+1's fragments into a second register set while it
// computes chunk b, so chunk b's slot is free for chunk b+3 during chunk b;
// the output wave loads its Qt fragments and Ut^T from global memory two
// chunks ahead. (fp32 intermediates have their own carry, carry_f32_kernel.)
constexpr int kRing = 3;
constexpr int kCarryThreads = 256;
constexpr int64_t kCarryRound = 256;   // carry workgroups resident at once (one per CU)
// Chunks between the L2 touch of a block and its use: six for one tile per
// workgroup, four for two (the two-tile form runs on batches with many
// pairs; measured on the 16-sequence packed batch, 3,967-3,988 us against
// 4,059-4,101 with six; the 8K workload's one-tile carry loses with four,
// 310-323 against 296-318 us).
template <int kTiles>
constexpr int kTouchAhead = kTiles == 1 ? 6 : 4;

// Workgroup barrier without a memory fence: no wave waits on another's
// global memory traffic, and LDS hand-offs are fenced by lgkmcnt where
// written.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Staged bytes per chunk: [-W] and K'^T fragments (32 KiB), each tile's U
// (2 KiB), gamma_C (512 B, in a 1 KiB slot), 1 KiB per DMA instruction.
constexpr int kStageW = kXAElems / 2 * 2;
constexpr int kStageKT = kKTElems * 2;
constexpr int kStageU = 4 * kWave * 4 * 2;

// State wave operands of one chunk.
template <class E>
struct StateOps {
  Frag<E> fw[4][4];   // [-W] fragments [token tile][k-slice]
  Frag<E> fk[8][2];   // K'^T fragments [channel tile][k-slice]
  Frag16<E> u[4];     // U accumulator tiles, in the I/O type
  floatx4 gm[8];      // gamma_C of the rows 16 mt + 4 g .. + 3
};
template <class E>
__device__ __forceinline__ void load_state_ops(StateOps<E>& p, const E* XW, const E* KT,
                                               const E* UA, const float* GC, int lane) {
  const int g = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) p.u[mt] = ld16(UA + (mt * kWave + lane) * 4);
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) p.gm[mt] = *reinterpret_cast<const floatx4*>(GC + 16 * mt + 4 * g);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) load_frag(XW + (mt * 4 + kb) * kWave * 8, lane, p.fw[mt][kb]);
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) load_frag(KT + (mt * 2 + kb) * kWave * 8, lane, p.fk[mt][kb]);
}

// State wave, one chunk: S <- Diag(gamma) S + K'^T (U + [-W] S), with the
// fragments of S (fs) in registers on entry and of the new S on exit.
template <class E>
__device__ __forceinline__ void carry_state(floatx4 (&S)[8], Frag<E> (&fs)[4],
                                            const StateOps<E>& p) {
  floatx4 X[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) X[mt] = zero4();
  // pseudo-value tiles 0, 1 first: they feed the first half of the update
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) X[mt] = mma(X[mt], p.fw[mt][kb], fs[kb]);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int mt = 2; mt < 4; ++mt) X[mt] = mma(X[mt], p.fw[mt][kb], fs[kb]);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) X[mt][e] += p.u[mt].get(e);
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) S[mt] *= p.gm[mt];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    Frag<E> fv;
#pragma unroll
    for (int e = 0; e < 4; ++e) { fv.set(e, X[2 * kb][e]); fv.set(4 + e, X[2 * kb + 1][e]); }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) S[mt] = mma(S[mt], p.fk[mt][kb], fv);
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int e = 0; e < 4; ++e) { fs[kb].set(e, S[2 * kb][e]); fs[kb].set(4 + e, S[2 * kb + 1][e]); }
}

// Output wave operands of one chunk: Qt fragments and the Ut^T of the
// workgroup's kTiles column tiles.
template <class E, int kTiles>
struct OutOps {
  Frag<E> fq[4][4];
  Frag16<E> ut[kTiles][4];   // kept in the I/O type until used: no wait at load time
};
template <class E, int kTiles>
__device__ __forceinline__ void load_out_ops(OutOps<E, kTiles>& p, const E* blk, int jt0,
                                             int lane) {
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      load_frag(blk + Inter<E>::kXA + ((4 + nt) * 4 + kb) * kWave * 8, lane, p.fq[nt][kb]);
#pragma unroll
  for (int t = 0; t < kTiles; ++t)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      p.ut[t][nt] = ld16(blk + Inter<E>::kUC + (((jt0 + t) * 8 + 4 + nt) * kWave + lane) * 4);
}

// Output wave, one chunk and column tile t: O^T = Ut^T + S^T Qt^T; lane
// (i = 16 nt + r, j = j0 + 4 g .. +3) holds four consecutive outputs of one
// token. They go to LDS in the I/O type; a loader wave stores them to
// global memory in the next chunk.
template <class E, int kTiles>
__device__ __forceinline__ void carry_out(const OutOps<E, kTiles>& p, int t,
                                          const Frag<E> (&fs)[4], E* sOb, int lane) {
  floatx4 X[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) X[nt] = zero4();
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) X[nt] = mma(X[nt], fs[kb], p.fq[nt][kb]);
  // Ut^T joins after the products: converting it earlier would make the
  // scheduler wait on the newest prefetch
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int e = 0; e < 4; ++e) X[nt][e] += p.ut[t][nt].get(e);
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) st16(sOb + (nt * kWave + lane) * 4, frag16<E>(X[nt]));
}

// Stores one chunk's O tile (16 columns) for the valid tokens. A loader wave
// issues these stores after its wait for the ring, so they have a whole
// chunk to complete before its next wait (one counter tracks loads and
// stores here); in the state wave, whose step sets the chunk's pace, the
// four stores cost about a fifth of the step.
template <class E>
__device__ __forceinline__ void store_out(const Frag16<E> (&x)[4], E* __restrict__ o,
                                          int64_t tok0, int len, int H, int h, int lane, int j0) {
  const int g = lane >> 4;
  E* const base = o + ((tok0 + (lane & 15)) * H + h) * kD + j0 + 4 * g;
  const int64_t step16 = (int64_t)16 * H * kD;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
    if (16 * nt + (lane & 15) < len) st16(base + nt * step16, x[nt]);
}

// One workgroup per (sequence, head, group of kTiles column tiles).
//   kTiles = 1: waves 0 state, 1 output, 2 and 3 loaders (2 moves [-W] and
//               U and stores O, 3 moves K'^T and gamma_C and touches L2);
//   kTiles = 2: waves 0 and 1 state (one tile each, sharing the staged
//               [-W] and K'^T), 2 output (both tiles), 3 the only loader
//               (and stores O).
// Two tiles per workgroup halve the L2 traffic per column tile at the cost
// of a longer chain per chunk; they pay when there are more (sequence,
// head) pairs than one round of one-tile workgroups fills.
template <class E, int kTiles, class SE>
__global__ __launch_bounds__(kCarryThreads) void carry_kernel(
    const uint8_t* inter,   // not restrict: prefetch loads stay ahead of the barriers
    const int32_t* __restrict__ cu,
    const int32_t* __restrict__ chunk_offset, const int32_t* __restrict__ status,
    const SE* h0, SE* h_final,   // not restrict: h_final may be h0 (in place)
    E* __restrict__ o, int32_t n_seqs, int64_t T, int32_t H, int32_t single,
    WindowArgs win) {
  static_assert(kTiles == 1 || kTiles == 2, "one or two column tiles per workgroup");
  static_assert(sizeof(E) == 2, "bf16 intermediates (fp32 ones: carry_f32_kernel)");
  constexpr int kGroups = 8 / kTiles;                 // workgroups per (sequence, head)
  constexpr int kUOff = kStageW + kStageKT;           // slot offset of the U tiles
  constexpr int kGOff = kUOff + kTiles * kStageU;     // slot offset of gamma_C
  constexpr int kBuf = kGOff + 1024;
  constexpr int kSBuf = 4 * kWave * 8;                // one published state
  constexpr int kOBuf = 4 * kWave * 4;                // one O tile
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kRing * kBuf];
  __shared__ __attribute__((aligned(16))) E sS[kTiles * 2 * kSBuf];   // published states
  __shared__ __attribute__((aligned(16))) int32_t sTouch[kWave];       // L2 touch sink
  __shared__ __attribute__((aligned(16))) E sO[kTiles * 2 * kOBuf];   // output tiles

  // XCD-aware order: consecutive ids go round-robin over the 8 XCDs; give the
  // workgroups of one (sequence, head) the same id % 8 so they share an L2.
  const int id = blockIdx.x;
  const int pair = (id & 7) + 8 * ((id >> 3) / kGroups);
  const int jg = (id >> 3) % kGroups;
  if (pair >= n_seqs * H) return;
  // one sequence (the full call skips the chunk map): check cu_seqlens here
  if (single ? (cu != nullptr && (cu[0] != 0 || (int64_t)cu[1] != T)) : status[0] != 0) return;
  const int n = pair / H, h = pair % H;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int64_t seq_start = cu ? cu[n] : 0, seq_end = cu ? cu[n + 1] : T;
  // the sequence's chunks [sb0, sb1), of which [b0, b1) fall in this window
  const int sb0 = single ? 0 : chunk_offset[n];
  const int sb1 = single ? (int)((T + kC - 1) / kC) : chunk_offset[n + 1];
  int b0, b1;
  if (!win.part(sb0, sb1, b0, b1)) return;   // whole workgroup: no barrier reached
  auto block_of = [&](int b) {
    return inter + ((int64_t)(b - win.W0) * H + h) * Inter<E>::kBytes;
  };
  auto slot = [&](int b) { return lds + ((b - b0) % kRing) * kBuf; };

  // loader roles: kTiles = 1 splits a chunk's transfers over waves 2 and 3
  const bool moves_w = kTiles == 1 ? w == 2 : w == 3;     // [-W] and U
  const bool moves_kt = w == 3;                           // K'^T, gamma_C, touches
  auto issue = [&](int b) {
    const uint8_t* src = block_of(b);
    uint8_t* dst = slot(b);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)src, 0, (int)Inter<E>::kBytes, 0x00020000);
    if (moves_w) {
#pragma unroll
      for (int i = 0; i < kStageW / 1024; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(dst + i * 1024), 16, lane * 16,
            (int)(Inter<E>::kXA * sizeof(E)) + i * 1024, 0, 0);
      // U of the group's tiles (tile jt's U is the first half of its 4 KiB
      // in the block; Ut^T follows it)
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
        const int uc = (int)(Inter<E>::kUC * sizeof(E)) + (jg * kTiles + t) * 8 * kWave * 4 * 2;
#pragma unroll
        for (int i = 0; i < kStageU / 1024; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs, (__attribute__((address_space(3))) void*)(dst + kUOff + t * kStageU + i * 1024),
              16, lane * 16, uc + i * 1024, 0, 0);
      }
    }
    if (moves_kt) {
#pragma unroll
      for (int i = 0; i < kStageKT / 1024; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(dst + kStageW + i * 1024), 16,
            lane * 16, (int)(Inter<E>::kKT * sizeof(E)) + i * 1024, 0, 0);
      // gamma_C: 512 bytes; lanes >= 32 read past the block and get zeros
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(dst + kGOff),
          16, lane * 16, (int)Inter<E>::kGCByte, 0, 0);
    }
  };
  // DMA instructions per chunk of each loader
  constexpr int kDMAw = kTiles == 1 ? (kStageW + kStageU) / 1024
                                    : (kStageW + kStageKT + kTiles * kStageU) / 1024 + 1;
  constexpr int kDMAkt = kTiles == 1 ? kStageKT / 1024 + 1 : kDMAw;
  // L2 touch of chunk b by wave 3: one word per 128-byte line of lines
  // [jg * kShare, (jg + 1) * kShare) of the block
  constexpr int kLines = (int)((Inter<E>::kBytes + 127) / 128);
  constexpr int kShare = (kLines + kGroups - 1) / kGroups;
  constexpr int kTouchOps = (kShare + kWave - 1) / kWave;
  auto touch = [&](int b) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)block_of(b), 0, (int)Inter<E>::kBytes, 0x00020000);
#pragma unroll
    for (int u = 0; u < kTouchOps; ++u) {
      const int line = min(jg * kShare + u * kWave + lane, kLines - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)sTouch, 4, line * 128, 0, 0, 0);
    }
  };
  // kTiles = 1, iteration b: after issuing chunk b+3 (dma) and touching
  // chunk b+6 (tch), wait until chunk b+2 has landed. The memory counter
  // retires in order, so the wait allows exactly the instructions issued
  // after chunk b+2's: the previous iteration's touch (prev), this
  // iteration's DMA and touch. Fewer allowed instructions only wait longer.
  auto loader_wait = [&](bool dma, bool tch, bool prev) {
    if (!dma) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else if (w == 2) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDMAw) : "memory");
    } else if (tch) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDMAkt + 2 * kTouchOps) : "memory");
    } else if (prev) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDMAkt + kTouchOps) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDMAkt) : "memory");
    }
  };

  // O of chunk b (all tiles of the group), written to LDS by the output wave
  // in step b and visible after that step's barrier; stored by a loader
  // after its ring wait in the next step (or after the last step).
  auto store_o = [&](int b) {
    const int64_t tok0 = seq_start + (int64_t)(b - sb0) * kC;
    const int len = (int)min((int64_t)kC, seq_end - tok0);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      const E* src = sO + (t * 2 + ((b - b0) & 1)) * kOBuf;
      Frag16<E> x[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) x[nt] = ld16(src + (nt * kWave + lane) * 4);
      store_out<E>(x, o, tok0, len, H, h, lane, 16 * (jg * kTiles + t));
    }
    // the reads are done before the barrier after which the output wave
    // rewrites this buffer, also where no lane stores
    __builtin_amdgcn_s_waitcnt(0xC07F);
  };

  // Each role runs its own loop; all execute two barriers before the first
  // chunk and one per chunk.
  if (w < kTiles) {
    // state wave of column tile jt
    const int jt = jg * kTiles + w;
    const int j = 16 * jt + (lane & 15);
    E* const sSw = sS + w * 2 * kSBuf;
    auto publish = [&](const Frag<E> (&fs)[4], int b) {
      E* dst = sSw + ((b - b0) & 1) * kSBuf;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) store8(dst + (kb * kWave + lane) * 8, fs[kb]);
    };
    // operand sources of chunk b in the LDS ring
    auto w_src = [&](int b) { return reinterpret_cast<const E*>(slot(b)); };
    auto kt_src = [&](int b) { return reinterpret_cast<const E*>(slot(b) + kStageW); };
    auto u_src = [&](int b) {
      return reinterpret_cast<const E*>(slot(b) + kUOff + w * kStageU);
    };
    auto gc_src = [&](int b) { return reinterpret_cast<const float*>(slot(b) + kGOff); };
    floatx4 S[8];
    Frag<E> fs[4];
    win.state_in(sb0, b0, h0, pair, h).load(S, g, j);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) { fs[kb].set(e, S[2 * kb][e]); fs[kb].set(4 + e, S[2 * kb + 1][e]); }
    publish(fs, b0);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    ring_barrier();
    StateOps<E> sa, sb;   // alternating chunks
    auto fetch = [&](StateOps<E>& p, int b) {
      load_state_ops(p, w_src(b), kt_src(b), u_src(b), gc_src(b), lane);
    };
    if (b0 < b1) fetch(sa, b0);
    // chunk b0's slot is read before the loaders reuse it for chunk b0 + 3
    __builtin_amdgcn_s_waitcnt(0xC07F);
    ring_barrier();
    auto step = [&](int b, StateOps<E>& cur, StateOps<E>& nxt) {
      fetch(nxt, min(b + 1, b1 - 1));
      carry_state<E>(S, fs, cur);
      // one prefetch read per product: a wave stalls once 16 LDS reads are
      // outstanding, which would hold the products back
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
      }
      publish(fs, b + 1);
      __builtin_amdgcn_s_waitcnt(0xC07F);
      ring_barrier();
    };
    // pairs of chunks, then the odd one: every loop back edge follows both
    // register sets' loads, so the compiler's counter waits stay exact
    int b = b0;
    for (; b + 1 < b1; b += 2) {
      step(b, sa, sb);
      step(b + 1, sb, sa);
    }
    if (b < b1) step(b, sa, sb);
    win.state_out(sb1, b1, h_final, pair, h).store(S, g, j);
  } else if (w == kTiles) {
    // output wave of the group's tiles
    auto step = [&](int b, OutOps<E, kTiles>& out) {
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
        Frag<E> fsb[4];
        const E* src = sS + (t * 2 + ((b - b0) & 1)) * kSBuf;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) lds_frag(src + (kb * kWave + lane) * 8, fsb[kb]);
        carry_out<E, kTiles>(out, t, fsb, sO + (t * 2 + ((b - b0) & 1)) * kOBuf, lane);
      }
      // unconditional (clamped) so every path issues the same loads and the
      // compiler's counter waits stay exact
      load_out_ops(out, reinterpret_cast<const E*>(block_of(min(b + 2, b1 - 1))), jg * kTiles,
                   lane);
      __builtin_amdgcn_s_waitcnt(0xC07F);   // O tiles written
      ring_barrier();
    };
    if (b0 < b1) {
      OutOps<E, kTiles> oa, ob;   // alternating chunks, loaded two chunks ahead
      load_out_ops(oa, reinterpret_cast<const E*>(block_of(b0)), jg * kTiles, lane);
      load_out_ops(ob, reinterpret_cast<const E*>(block_of(min(b0 + 1, b1 - 1))), jg * kTiles,
                   lane);
      ring_barrier();
      ring_barrier();
      // pairs of chunks, then the odd one: every loop back edge follows both
      // register sets' loads
      int b = b0;
      for (; b + 1 < b1; b += 2) {
        step(b, oa);
        step(b + 1, ob);
      }
      if (b < b1) step(b, oa);
    } else {
      ring_barrier();
      ring_barrier();
    }
  } else if (kTiles == 1) {
    // two loaders
    for (int b = b0; b < b0 + 3 && b < b1; ++b) issue(b);
    loader_wait(b0 + 2 < b1, false, false);   // chunks b0, b0 + 1 landed
    if (w == 3)
      for (int b = b0 + 3; b < b0 + kTouchAhead<kTiles> && b < b1; ++b) touch(b);
    ring_barrier();
    ring_barrier();
    // Wave 2 issues chunk b-1's O stores after its wait, so at its next wait
    // they sit between two chunks' DMA. That wait allows only the newer
    // chunk's DMA to stay outstanding, which holds whether or not stores
    // retire in order with loads: loads retire in order among themselves,
    // and the allowance leaves no room for a store.
    for (int b = b0; b < b1; ++b) {
      const bool dma = b + 3 < b1;
      const bool tch = w == 3 && b + kTouchAhead<kTiles> < b1;
      const bool prev = w == 3 && b + kTouchAhead<kTiles> - 1 < b1;
      if (dma) issue(b + 3);
      if (tch) touch(b + kTouchAhead<kTiles>);
      loader_wait(dma, tch, prev);
      if (w == 2 && b > b0) store_o(b - 1);
      ring_barrier();
    }
    if (w == 2 && b0 < b1) store_o(b1 - 1);
  } else {
    // one loader, kDMAw = 37 transfers per chunk: at most one chunk's
    // transfers are in flight (the counter holds 63), so iteration b first
    // waits for chunk b+2, issued in iteration b-1 and followed there only
    // by that iteration's touch, and then issues chunk b+3.
    if (b0 < b1) {
      issue(b0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (b0 + 1 < b1) issue(b0 + 1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // chunks b0, b0 + 1 landed
      if (b0 + 2 < b1) issue(b0 + 2);
      for (int b = b0 + 3; b < b0 + kTouchAhead<kTiles> && b < b1; ++b) touch(b);
    }
    ring_barrier();
    ring_barrier();
    for (int b = b0; b < b1; ++b) {
      if (b > b0 && b + kTouchAhead<kTiles> - 1 < b1)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kTouchOps) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (b + 3 < b1) issue(b + 3);
      if (b + kTouchAhead<kTiles> < b1) touch(b + kTouchAhead<kTiles>);
      // after the issues: the next wait allows only the touch, so these
      // stores never let a DMA transfer count as landed
      if (b > b0) store_o(b - 1);
      ring_barrier();
    }
    if (b0 < b1) store_o(b1 - 1);
  }
}

// ------------------------------------------------------- carry, fp32 I/O
// The carry for fp32 intermediates (fp32 I/O). A chunk's state operands
// take 69 KiB in fp32, so the ring has two slots and the loaders stay one
// chunk ahead. fp32 products run at a sixteenth of the bf16 rate (eight
// 16x16x4 products per fragment), so the chain is bound by the products:
// 256 per chunk for the state and 128 for the output of one column tile,
// about 12 k cycles on one SIMD. They are spread over four state and four
// output waves, with the same products in the same order per tile as one
// wave would issue (so the results do not depend on the split). One
// workgroup per (sequence, head, 16-column tile), ten waves:
//   waves 0 .. 3  state: wave s computes the pseudo-value rows 16 s .. +15
//           (over all 128 state rows), the rows are swapped through LDS at a
//           second barrier per chunk, and wave s updates the state rows
//           32 s .. 32 s + 31 and publishes them; each reads the others'
//           rows back for the next chunk
//   waves 4 .. 7  output: O^T = Ut^T + S^T Qt^T for tokens 16 (w-4) .. +15,
//           Qt and Ut held in registers one chunk ahead; each stores its O
//           rows itself, issuing the next chunk's loads first so that its
//           load waits never include its stores
//   waves 8, 9  loaders: [-W] and U; K'^T, gamma_C and the L2 touches
// Every wave executes one barrier before the first chunk and two per
// chunk (the state waves swap pseudo-value rows between them).
constexpr int kF32UOff = 2 * 32768;            // slot offsets (bytes)
constexpr int kF32GOff = kF32UOff + 4096;
constexpr int kF32Buf = kF32GOff + 1024;       // 69 KiB
constexpr int kF32States = 4;                  // state waves (and output waves)
constexpr int kF32Threads = (2 * kF32States + 2) * kWave;

template <class SE>
__global__ __launch_bounds__(kF32Threads) void carry_f32_kernel(
    const uint8_t* inter, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ chunk_offset, const int32_t* __restrict__ status,
    const SE* h0, SE* h_final,   // not restrict: h_final may be h0 (in place)
    float* __restrict__ o, int32_t n_seqs, int64_t T, int32_t H, int32_t single,
    WindowArgs win) {
  typedef float E;
  constexpr int kNS = kF32States;
  constexpr int kXT = 4 / kNS;           // pseudo-value tiles per state wave
  constexpr int kST = 8 / kNS;           // state row tiles per state wave
  constexpr int kSF = 4 / kNS;           // state fragments per state wave
  static_assert(kNS == 2 || kNS == 4, "two or four state waves");
  constexpr int kSBuf = 4 * kWave * 8;   // one published state (fp32 fragments)
  constexpr int kXBuf = kWave * 4;       // one pseudo-value tile
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kF32Buf];
  __shared__ __attribute__((aligned(16))) float sS[2 * kSBuf];
  __shared__ __attribute__((aligned(16))) float sX[4 * kXBuf];
  __shared__ __attribute__((aligned(16))) int32_t sTouch[kWave];

  const int id = blockIdx.x;
  const int pair = (id & 7) + 8 * ((id >> 3) / 8);
  const int jt = (id >> 3) % 8;
  if (pair >= n_seqs * H) return;
  if (single ? (cu != nullptr && (cu[0] != 0 || (int64_t)cu[1] != T)) : status[0] != 0) return;
  const int n = pair / H, h = pair % H;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int64_t seq_start = cu ? cu[n] : 0, seq_end = cu ? cu[n + 1] : T;
  const int sb0 = single ? 0 : chunk_offset[n];
  const int sb1 = single ? (int)((T + kC - 1) / kC) : chunk_offset[n + 1];
  int b0, b1;
  if (!win.part(sb0, sb1, b0, b1)) return;   // whole workgroup: no barrier reached
  auto block_of = [&](int b) {
    return inter + ((int64_t)(b - win.W0) * H + h) * Inter<E>::kBytes;
  };
  auto slot = [&](int b) { return lds + ((b - b0) & 1) * kF32Buf; };

  // the state wave index is a template constant so that every register
  // array index stays static
  auto state_role = [&](auto hsc) {
    constexpr int hs = decltype(hsc)::value;
    const int j = 16 * jt + (lane & 15);
    floatx4 S[8];
    Frag<E> fs[4];
    win.state_in(sb0, b0, h0, pair, h).load(S, g, j);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) { fs[kb].set(e, S[2 * kb][e]); fs[kb].set(4 + e, S[2 * kb + 1][e]); }
    // fragments kb = kSF hs .. kSF hs + kSF - 1 hold this wave's state rows
    auto publish = [&](int b) {
      float* dst = sS + ((b - b0) & 1) * kSBuf;
#pragma unroll
      for (int q = 0; q < kSF; ++q) {
        const int kb = kSF * hs + q;
        if (b > b0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            fs[kb].set(e, S[2 * kb][e]);
            fs[kb].set(4 + e, S[2 * kb + 1][e]);
          }
        }
        store8(dst + (kb * kWave + lane) * 8, fs[kb]);
      }
    };
    publish(b0);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    ring_barrier();
    for (int b = b0; b < b1; ++b) {
      if (b > b0) {
        // the other waves' state rows, published in the previous step
        const float* src = sS + ((b - b0) & 1) * kSBuf;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          if (kb / kSF != hs) lds_frag(src + (kb * kWave + lane) * 8, fs[kb]);
      }
      const uint8_t* sl = slot(b);
      const float* XW = reinterpret_cast<const float*>(sl);
      const float* KT = reinterpret_cast<const float*>(sl + 32768);
      const float* UA = reinterpret_cast<const float*>(sl + kF32UOff);
      const float* GC = reinterpret_cast<const float*>(sl + kF32GOff);
      // this wave's pseudo-value rows: the same products in the same order
      // as the bf16 carry's carry_state
      floatx4 X[4];
#pragma unroll
      for (int q = 0; q < kXT; ++q) {
        const int mt = kXT * hs + q;
        X[mt] = zero4();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          Frag<E> a;
          lds_frag(XW + ((mt * 4 + kb) * kWave + lane) * 8, a);
          X[mt] = mma(X[mt], a, fs[kb]);
        }
        const Frag16<E> u = ld16(UA + (mt * kWave + lane) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) X[mt][e] += u.get(e);
        st16(sX + (mt * kWave + lane) * 4, frag16<E>(X[mt]));
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);
      ring_barrier();
      // the other waves' pseudo-value rows
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (mt / kXT == hs) continue;
        const Frag16<E> x = ld16(sX + (mt * kWave + lane) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) X[mt][e] = x.get(e);
      }
      // this wave's state rows
#pragma unroll
      for (int q = 0; q < kST; ++q) {
        const int mt = kST * hs + q;
        S[mt] *= *reinterpret_cast<const floatx4*>(GC + 16 * mt + 4 * g);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        Frag<E> fv;
#pragma unroll
        for (int e = 0; e < 4; ++e) { fv.set(e, X[2 * kb][e]); fv.set(4 + e, X[2 * kb + 1][e]); }
#pragma unroll
        for (int q = 0; q < kST; ++q) {
          const int mt = kST * hs + q;
          Frag<E> a;
          lds_frag(KT + ((mt * 2 + kb) * kWave + lane) * 8, a);
          S[mt] = mma(S[mt], a, fv);
        }
      }
      publish(b + 1);
      __builtin_amdgcn_s_waitcnt(0xC07F);
      ring_barrier();
    }
    // this wave's state rows: tiles kST hs .. kST hs + kST - 1
    win.state_out(sb1, b1, h_final, pair, h).template store<kST * hs, kST * hs + kST>(S, g, j);
  };
  // output wave ho: O tiles nt = kXT ho .. kXT ho + kXT - 1
  auto output_role = [&](int ho) {
    Frag<E> fq[kXT][4];
    Frag16<E> ut[kXT];
    auto load_ops = [&](int b) {
      const E* blk = reinterpret_cast<const E*>(block_of(b));
#pragma unroll
      for (int q = 0; q < kXT; ++q) {
        const int nt = kXT * ho + q;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          load_frag(blk + Inter<E>::kXA + ((4 + nt) * 4 + kb) * kWave * 8, lane, fq[q][kb]);
        ut[q] = ld16(blk + Inter<E>::kUC + ((jt * 8 + 4 + nt) * kWave + lane) * 4);
      }
    };
    if (b0 < b1) load_ops(b0);
    ring_barrier();
    for (int b = b0; b < b1; ++b) {
      Frag<E> fsb[4];
      const float* src = sS + ((b - b0) & 1) * kSBuf;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) lds_frag(src + (kb * kWave + lane) * 8, fsb[kb]);
      floatx4 X[kXT];
#pragma unroll
      for (int q = 0; q < kXT; ++q) X[q] = zero4();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int q = 0; q < kXT; ++q) X[q] = mma(X[q], fsb[kb], fq[q][kb]);
      Frag16<E> ob[kXT];
#pragma unroll
      for (int q = 0; q < kXT; ++q) {
#pragma unroll
        for (int e = 0; e < 4; ++e) X[q][e] += ut[q].get(e);
        ob[q] = frag16<E>(X[q]);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);
      ring_barrier();   // the state waves' pseudo-value swap
      // next chunk's operands first, then this chunk's stores
      load_ops(min(b + 1, b1 - 1));
      const int64_t tok0 = seq_start + (int64_t)(b - sb0) * kC;
      const int len = (int)min((int64_t)kC, seq_end - tok0);
      E* const base = o + ((tok0 + (lane & 15)) * H + h) * kD + 16 * jt + 4 * g;
#pragma unroll
      for (int q = 0; q < kXT; ++q) {
        const int nt = kXT * ho + q;
        if (16 * nt + (lane & 15) < len) st16(base + (int64_t)16 * nt * H * kD, ob[q]);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);
      ring_barrier();
    }
  };
  const int wl = w - 2 * kNS;   // loader index
  if (w < kNS) {
    switch (w) {
      case 0: state_role(std::integral_constant<int, 0>{}); break;
      case 1: state_role(std::integral_constant<int, 1>{}); break;
      case 2: if constexpr (kNS > 2) state_role(std::integral_constant<int, 2 % kNS>{}); break;
      default: if constexpr (kNS > 3) state_role(std::integral_constant<int, 3 % kNS>{}); break;
    }
  } else if (w < 2 * kNS) {
    output_role(w - kNS);
  } else {
    // loaders: chunk b + 1 into the other slot while chunk b is computed
    constexpr int kLines = (int)((Inter<E>::kBytes + 127) / 128);
    constexpr int kShare = (kLines + 7) / 8;
    constexpr int kTouchOps = (kShare + kWave - 1) / kWave;
    auto issue = [&](int b) {
      const uint8_t* src = block_of(b);
      uint8_t* dst = slot(b);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)src, 0, (int)Inter<E>::kBytes, 0x00020000);
      if (wl == 0) {
#pragma unroll
        for (int i = 0; i < 32; ++i)   // [-W]: the first half of [-W ; Qt]
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs, (__attribute__((address_space(3))) void*)(dst + i * 1024), 16, lane * 16,
              i * 1024, 0, 0);
        const int uc = (int)(Inter<E>::kUC * sizeof(E)) + jt * 8 * kWave * 4 * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i)    // U of this tile
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs, (__attribute__((address_space(3))) void*)(dst + kF32UOff + i * 1024), 16,
              lane * 16, uc + i * 1024, 0, 0);
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs, (__attribute__((address_space(3))) void*)(dst + 32768 + i * 1024), 16,
              lane * 16, (int)(Inter<E>::kKT * sizeof(E)) + i * 1024, 0, 0);
        // gamma_C: 512 bytes; lanes >= 32 read past the block and get zeros
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(dst + kF32GOff), 16, lane * 16,
            (int)Inter<E>::kGCByte, 0, 0);
      }
    };
    auto touch = [&](int b) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)block_of(b), 0, (int)Inter<E>::kBytes, 0x00020000);
#pragma unroll
      for (int u = 0; u < kTouchOps; ++u) {
        const int line = min(jt * kShare + u * kWave + lane, kLines - 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)sTouch, 4, line * 128, 0, 0, 0);
      }
    };
    if (b0 < b1) issue(b0);
    if (wl == 1 && b0 + 1 < b1) touch(b0 + 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    ring_barrier();
    for (int b = b0; b < b1; ++b) {
      if (b + 1 < b1) issue(b + 1);
      const bool tch = wl == 1 && b + 2 < b1;
      if (tch) touch(b + 2);
      // chunk b + 1 landed; this iteration's touch may stay in flight (the
      // counter retires in order and the touch was issued last): waiting
      // for it too held the loader for its HBM round trip every chunk
      // (fp32 8K call 643 -> 606 us)
      if (tch)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kTouchOps) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      ring_barrier();   // the state waves' pseudo-value swap
      ring_barrier();
    }
  }
}

// ------------------------------------------------- carry for short sequences
// One workgroup of eight waves per (sequence, head), for batches of short
// sequences, where the pipelined carry pays its fixed cost (state load, ring
// fill and drain in a workgroup that fills a CU) for one or two chunks. Per
// chunk the eight waves stage the operands all column tiles share ([-W ; Qt]
// and K'^T, 48 KiB, and gamma_C) in LDS with buffer->LDS transfers, a
// seventh of them each; wave t loads column tile t's state and its U and
// Ut^T rows itself and computes the tile with the same products in the same
// order as the pipelined carry (O = Ut + Qt S from the state at the chunk
// start, then the state update), reading each fragment from LDS just before
// its product, so the results are bit-identical to it. Each block is read
// from memory once per chunk (the one-wave-per-tile form read its shared
// part eight times through the CUs' memory pipelines), and at most 128
// registers and 50 KiB of LDS let two or three workgroups share a CU.
constexpr int kShortThreads = 8 * kWave;
constexpr int kShortShared = kStageW * 2 + kStageKT;   // [-W ; Qt] and K'^T bytes
constexpr int kShortXfers = kShortShared / 1024 + 1;   // and gamma_C

template <class E, class SE>
__global__ __launch_bounds__(kShortThreads, 2) void carry_short_kernel(
    const uint8_t* __restrict__ inter, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ chunk_offset, const int32_t* __restrict__ status,
    const SE* h0, SE* h_final,   // not restrict: h_final may be h0 (in place)
    E* __restrict__ o, int32_t n_seqs, int64_t T, int32_t H, WindowArgs win) {
  static_assert(sizeof(E) == 2, "bf16 intermediates");
  static_assert(Inter<E>::kXA == 0 && Inter<E>::kKT * sizeof(E) == kStageW * 2,
                "[-W ; Qt] and K'^T open the block, in this order");
  __shared__ __attribute__((aligned(1024))) uint8_t sm[kShortShared + 1024];
  const E* const sXA = reinterpret_cast<const E*>(sm);
  const E* const sKT = reinterpret_cast<const E*>(sm + kStageW * 2);
  const float* const sGC = reinterpret_cast<const float*>(sm + kShortShared);

  const int pair = blockIdx.x;
  if (pair >= n_seqs * H || status[0] != 0) return;
  const int n = pair / H, h = pair % H;
  const int lane = threadIdx.x & 63;
  const int jt = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // column tile
  const int g = lane >> 4;
  const int j = 16 * jt + (lane & 15);
  const int64_t seq_start = cu ? cu[n] : 0, seq_end = cu ? cu[n + 1] : T;
  const int sb0 = chunk_offset[n], sb1 = chunk_offset[n + 1];
  int b0, b1;
  if (!win.part(sb0, sb1, b0, b1)) return;   // whole workgroup: no barrier reached

  floatx4 S[8];
  Frag<E> fs[4];
  win.state_in(sb0, b0, h0, pair, h).load(S, g, j);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int e = 0; e < 4; ++e) { fs[kb].set(e, S[2 * kb][e]); fs[kb].set(4 + e, S[2 * kb + 1][e]); }

  for (int b = b0; b < b1; ++b) {
    const uint8_t* blk8 = inter + ((int64_t)(b - win.W0) * H + h) * Inter<E>::kBytes;
    const E* blk = reinterpret_cast<const E*>(blk8);
    {
      // transfers x = jt, jt + 8, ...: 1 KiB pieces of [-W ; Qt] and K'^T,
      // then gamma_C (512 bytes; lanes >= 32 read past the block and get
      // zeros)
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)blk8, 0, (int)Inter<E>::kBytes, 0x00020000);
      for (int x = jt; x < kShortXfers; x += 8) {
        const int so = x < kShortXfers - 1 ? x * 1024 : (int)Inter<E>::kGCByte;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(sm + x * 1024), 16, lane * 16, so, 0,
            0);
      }
    }
    // this tile's U and Ut^T rows
    Frag16<E> u[4], ut[4];
    const E* UA = blk + Inter<E>::kUC + jt * 8 * kWave * 4;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      u[mt] = ld16(UA + (mt * kWave + lane) * 4);
      ut[mt] = ld16(UA + ((4 + mt) * kWave + lane) * 4);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // O^T = Ut^T + S^T Qt^T from the state at the chunk start (the
    // pipelined carry's carry_out, with Qt from LDS)
    floatx4 X[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) X[nt] = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        Frag<E> fq;
        load_frag(sXA + ((4 + nt) * 4 + kb) * kWave * 8, lane, fq);
        X[nt] = mma(X[nt], fs[kb], fq);
      }
    Frag16<E> ob[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
      for (int e = 0; e < 4; ++e) X[nt][e] += ut[nt].get(e);
      ob[nt] = frag16<E>(X[nt]);
    }
    // S <- Diag(gamma) S + K'^T (U + [-W] S) (the pipelined carry's
    // carry_state, with the fragments from LDS)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) X[mt] = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        Frag<E> fw;
        load_frag(sXA + (mt * 4 + kb) * kWave * 8, lane, fw);
        X[mt] = mma(X[mt], fw, fs[kb]);
      }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int mt = 2; mt < 4; ++mt) {
        Frag<E> fw;
        load_frag(sXA + (mt * 4 + kb) * kWave * 8, lane, fw);
        X[mt] = mma(X[mt], fw, fs[kb]);
      }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) X[mt][e] += u[mt].get(e);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
      S[mt] *= *reinterpret_cast<const floatx4*>(sGC + 16 * mt + 4 * g);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      Frag<E> fv;
#pragma unroll
      for (int e = 0; e < 4; ++e) { fv.set(e, X[2 * kb][e]); fv.set(4 + e, X[2 * kb + 1][e]); }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        Frag<E> fk;
        load_frag(sKT + (mt * 2 + kb) * kWave * 8, lane, fk);
        S[mt] = mma(S[mt], fk, fv);
      }
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) { fs[kb].set(e, S[2 * kb][e]); fs[kb].set(4 + e, S[2 * kb + 1][e]); }
    const int64_t tok0 = seq_start + (int64_t)(b - sb0) * kC;
    store_out<E>(ob, o, tok0, (int)min((int64_t)kC, seq_end - tok0), H, h, lane, 16 * jt);
    // every wave has read this chunk's operands before the next transfers
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  win.state_out(sb1, b1, h_final, pair, h).store(S, g, j);
}

// ------------------------------------------------------------- launchers
size_t inter_block_bytes(bool bf16_io) {
  return bf16_io ? Inter<bf16>::kBytes : Inter<float>::kBytes;
}


// phases: bit 0 chunk map, bit 1 intra-chunk, bit 2 carry (all three, in
// order on one stream, make one prefill call). The chunk slots [0, n_slots)
// run in windows of win_slots: per window the intra-chunk kernel, then the
// carry. state_area holds two [H, 128, 128] float32 states for sequences
// crossing a window boundary.
hipError_t launch_chunk_fwd(int phases, bool bf16_io, bool l2norm, bool bf16_state,
                            const void* q, const void* k, const void* v,
                            const float* log_alpha, const float* beta, const void* h0,
                            const int32_t* cu, int32_t n_seqs, int64_t T, int32_t H,
                            int64_t n_slots, int64_t win_slots, void* o, void* h_final,
                            int32_t* status, int32_t* chunk_offset, float* state_area,
                            uint8_t* inter, hipStream_t stream) {
  hipError_t err = hipSuccess;
  // A full call on one sequence needs no chunk map: the two kernels derive
  // the chunk range from T and check cu_seqlens themselves.
  const int32_t single = phases == 7 && n_seqs == 1 && T > 0;
  if ((phases & 1) && !single) {
    chunk_map_kernel<<<1, 256, 0, stream>>>(cu, n_seqs, T, n_slots, chunk_offset, status);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int64_t pairs = (int64_t)n_seqs * H;
  // Two column tiles per workgroup once one-tile workgroups (eight per pair)
  // would not all be resident at once (one per CU on the 256-CU MI355X): on
  // the 16-sequence packed batch the carry drops from 2.70 to 2.02 ms; a
  // single round of one-tile workgroups keeps the shorter chain (1.06 against
  // 1.28 us per chunk on the 8K workload).
  const bool two = bf16_io && pairs * 8 > kCarryRound;
  const int64_t nblocks = ((pairs + 7) / 8) * 8 * (two ? 4 : 8);   // column-tile groups
  // batches of short sequences: one workgroup per pair, no pipeline (the
  // single-sequence call always pipelines). It runs a sequence's chunks one
  // after another at about 3.5 us each where the pipelined carry takes about
  // 1 us, but reads each block once and packs two workgroups per CU. Measured
  // at 32 heads (whole call): 256 x 64 tokens 817 -> 706 us, 32 x 256
  // 347 -> 278 us, 16 x 512 307 -> 261 us, 8 x 2048 589 -> 558 us; with few
  // pairs or long sequences it loses (4 x 2048 277 -> 338 us, 2 x 4096
  // 271 -> 463 us). The choice sees only the mean length: a batch that mixes
  // one long sequence with many short ones runs the long one unpipelined.
  const bool short_seqs = bf16_io && !single && n_seqs > 0 &&
                          (T <= 2 * kC * n_seqs || (T <= 4 * kC * n_seqs && pairs >= kCarryRound));
  const int64_t n_windows = n_slots > 0 ? (n_slots + win_slots - 1) / win_slots : 1;
  const int64_t state_floats = (int64_t)H * kD * kD;
  for (int64_t w = 0; w < n_windows; ++w) {
    const int64_t W0 = w * win_slots, W1 = std::min(W0 + win_slots, n_slots);
    if ((phases & 2) && T > 0 && W1 > W0) {
      dim3 grid((unsigned)(W1 - W0), (unsigned)H);
#define KDA_INTRA(E, NORM)                                                                  \
  intra_kernel<E, NORM><<<grid, kIntraThreads, 0, stream>>>(                                \
      (const E*)q, (const E*)k, (const E*)v, log_alpha, beta, cu, chunk_offset, status, \
      n_seqs, T, H, inter, single, (int32_t)W0)
      if (bf16_io) {
        if (l2norm) KDA_INTRA(bf16, true); else KDA_INTRA(bf16, false);
      } else {
        if (l2norm) KDA_INTRA(float, true); else KDA_INTRA(float, false);
      }
#undef KDA_INTRA
      err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
    if (!(phases & 4)) continue;
    WindowArgs win;
    win.W0 = (int32_t)W0;
    win.W1 = (int32_t)W1;
    win.last = w == n_windows - 1;
    win.resume = state_area + ((w + 1) & 1) * state_floats;
    win.suspend = state_area + (w & 1) * state_floats;
    // h0 and h_final in the state type SE (the carry keeps fp32 inside)
    auto carry = [&](auto se) {
      typedef decltype(se) SE;
      const SE* h0s = static_cast<const SE*>(h0);
      SE* hfs = static_cast<SE*>(h_final);
      if (short_seqs)
        carry_short_kernel<bf16, SE><<<(unsigned)pairs, kShortThreads, 0, stream>>>(
            inter, cu, chunk_offset, status, h0s, hfs, (bf16*)o, n_seqs, T, H, win);
      else if (two)
        carry_kernel<bf16, 2, SE><<<(unsigned)nblocks, kCarryThreads, 0, stream>>>(
            inter, cu, chunk_offset, status, h0s, hfs, (bf16*)o, n_seqs, T, H, single, win);
      else if (bf16_io)
        carry_kernel<bf16, 1, SE><<<(unsigned)nblocks, kCarryThreads, 0, stream>>>(
            inter, cu, chunk_offset, status, h0s, hfs, (bf16*)o, n_seqs, T, H, single, win);
      else
        carry_f32_kernel<SE><<<(unsigned)nblocks, kF32Threads, 0, stream>>>(
            inter, cu, chunk_offset, status, h0s, hfs, (float*)o, n_seqs, T, H, single, win);
    };
    if (bf16_state) carry(bf16{}); else carry(0.f);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace kda
