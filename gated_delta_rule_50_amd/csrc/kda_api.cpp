// Host side of the C ABI declared in include/kda.h: argument validation,
// workspace sizing and launch sequencing. No compute happens here; every
// step of the operator runs in the HIP kernels.
#include <algorithm>
#include <cstring>
#include <initializer_list>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda.h"

namespace kda {
hipError_t launch_chunk_fwd(int phases, bool bf16_io, bool l2norm, bool bf16_state,
                            const void* q, const void* k, const void* v,
                            const float* log_alpha, const float* beta, const void* h0,
                            const int32_t* cu, int32_t n_seqs, int64_t T, int32_t H,
                            int64_t n_slots, int64_t win_slots, void* o, void* h_final,
                            int32_t* status, int32_t* chunk_offset, float* state_area,
                            uint8_t* inter, hipStream_t stream);
size_t inter_block_bytes(bool bf16_io);
hipError_t launch_recurrent_fwd(bool bf16_io, bool bf16_state, bool l2norm, const void* q,
                                const void* k, const void* v, const float* log_alpha,
                                const float* beta, const void* h0, const int32_t* cu,
                                int64_t seq_len, int64_t T, int32_t H, int64_t pairs,
                                void* o, void* h_final, hipStream_t stream);
hipError_t launch_rmsnorm_gate(bool bf16_io, const void* o, const void* g, const float* w,
                               float eps, int64_t rows, void* y, hipStream_t stream);
hipError_t launch_check_inputs(bool bf16_io, const void* q, const void* k, const void* v,
                               const float* log_alpha, const float* beta, const int32_t* cu,
                               int32_t n_seqs, int64_t T, int32_t H, int32_t* flags,
                               hipStream_t stream);
}  // namespace kda

namespace {

constexpr int64_t kChunk = KDA_CHUNK;
constexpr int64_t kDim = KDA_HEAD_DIM;

struct Range {
  uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
  Range() = default;
  Range(const void* p, int64_t bytes)
      : lo((uintptr_t)p), hi((uintptr_t)p + (uintptr_t)(p ? bytes : 0)) {}
  bool empty() const { return hi <= lo; }
};

bool overlap(const Range& a, const Range& b) {
  return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi;
}

// Enum arguments as integers. A C caller may pass any int; reading the
// value through its object representation keeps an out-of-range one from
// being an invalid load of the enum type.
template <class Enum>
int raw(const Enum& e) {
  static_assert(sizeof(Enum) == sizeof(int), "C enums are int-sized");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

bool valid_io(int io) { return io == KDA_IO_F32 || io == KDA_IO_BF16; }

// Tensor pointers the kernels read or write with 16-byte vectors must be
// 16-byte aligned; NULL passes.
bool aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if ((uintptr_t)p & 15u) return false;
  return true;
}
bool aligned4(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if ((uintptr_t)p & 3u) return false;
  return true;
}

int64_t io_bytes(int io) { return io == KDA_IO_BF16 ? 2 : 4; }

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Chunk slots the prefill launch is sized for: sum_n ceil(L_n / 64) is at
// most ceil(T / 64) + N - 1 for any split of T tokens into N sequences.
int64_t chunk_slots(int64_t n_seqs, int64_t T) {
  return (T + kChunk - 1) / kChunk + n_seqs - 1;
}

// Workspace layout: status word, chunk offsets, two [H, 128, 128] float32
// states for sequences crossing a window boundary, then the intermediate
// blocks of one window of chunk slots ([slot - W0][head]).
int64_t state_offset(int64_t n_seqs) { return 256 + round_up(4 * (n_seqs + 1), 256); }
int64_t inter_offset(int64_t n_seqs, int64_t heads) {
  return state_offset(n_seqs) + 2 * heads * kDim * kDim * 4;
}
int64_t block_bytes(int io) { return (int64_t)kda::inter_block_bytes(io == KDA_IO_BF16); }

// Blocks of the window kda_chunk_fwd_workspace_bytes sizes for: the whole
// call when its blocks take at most this much, else as many chunk slots as
// fit (the 8K x 32-head bf16 call is one window). Windows run one after the
// other over the chunk slots in sequence order, which costs one sequence
// nothing but serialises the sequences of a packed batch (a window of 512
// MiB holds one or two of the 16-sequence batch's): packed batches get a
// larger window, so such batches stay one window. fp32 blocks take twice
// the bytes of bf16 ones, so their cap is doubled to hold as many chunk
// slots (the fp32 8K x 32-head call as one window: 638-684 against
// 659-686 us in two; 65,536 tokens in windows of 198 slots 4.80 ms against
// 4.97-5.00 in windows of 99).
constexpr int64_t kWindowBytes = (int64_t)512 << 20;
constexpr int64_t kPackedWindowBytes = (int64_t)8 << 30;

bool valid_sizes(int64_t n_seqs, int64_t T, int64_t heads, int io) {
  return n_seqs >= 1 && T >= 0 && heads >= 1 && heads <= 65535 && valid_io(io) &&
         chunk_slots(n_seqs, T) <= INT32_MAX;
}

// Recommended size (0 when the sizes are unusable).
size_t workspace_bytes(int64_t n_seqs, int64_t T, int64_t heads, int io) {
  if (!valid_sizes(n_seqs, T, heads, io)) return 0;
  const int64_t slots = chunk_slots(n_seqs, T);
  const int64_t per_slot = heads * block_bytes(io);
  const int64_t cap =
      n_seqs > 1 ? kPackedWindowBytes : (io == KDA_IO_F32 ? 2 : 1) * kWindowBytes;
  const int64_t win = std::min(slots, std::max<int64_t>(1, cap / per_slot));
  return (size_t)(inter_offset(n_seqs, heads) + win * per_slot);
}

// Smallest usable size: a window of one chunk slot (0 when unusable).
size_t workspace_min_bytes(int64_t n_seqs, int64_t T, int64_t heads, int io) {
  if (!valid_sizes(n_seqs, T, heads, io)) return 0;
  const int64_t slots = chunk_slots(n_seqs, T);
  return (size_t)(inter_offset(n_seqs, heads) + (slots > 0 ? heads * block_bytes(io) : 0));
}

}  // namespace

extern "C" {

size_t kda_chunk_fwd_workspace_bytes(int32_t n_seqs, int64_t total_tokens, int32_t heads,
                                     int32_t dk, int32_t dv, kda_io_dtype io_arg) {
  const int io = raw(io_arg);
  if (dk != kDim || dv != kDim) return 0;
  return workspace_bytes(n_seqs, total_tokens, heads, io);
}

size_t kda_chunk_fwd_workspace_min_bytes(int32_t n_seqs, int64_t total_tokens, int32_t heads,
                                         int32_t dk, int32_t dv, kda_io_dtype io_arg) {
  const int io = raw(io_arg);
  if (dk != kDim || dv != kDim) return 0;
  return workspace_min_bytes(n_seqs, total_tokens, heads, io);
}

}  // extern "C"

namespace {

// Validates the prefill arguments and launches the phases selected by the
// bit mask `phases` (bit 0: chunk map, bit 1: intra-chunk, bit 2: carry).
kda_status chunk_fwd_impl(int phases, const void* q, const void* k, const void* v,
                          const float* log_alpha, const float* beta, const void* h0,
                          const int32_t* cu_seqlens, int32_t n_seqs, int64_t total_tokens,
                          int32_t heads, int32_t dk, int32_t dv, int io,
                          uint32_t flags, void* o, void* h_final, void* workspace,
                          size_t workspace_bytes_given, void* stream) {
  const int64_t T = total_tokens;
  if (T < 0 || n_seqs < 1 || heads < 1) return KDA_ERR_SHAPE;
  if (dk != kDim || dv != kDim || !valid_io(io) || heads > 65535) return KDA_ERR_UNSUPPORTED;
  if (flags & ~(uint32_t)(KDA_FLAG_QK_L2NORM | KDA_FLAG_STATE_BF16)) return KDA_ERR_UNSUPPORTED;
  if (cu_seqlens == nullptr && n_seqs != 1) return KDA_ERR_NULL;
  if (cu_seqlens != nullptr && T > INT32_MAX) return KDA_ERR_SHAPE;
  // the carry grid has up to eight workgroups per (sequence, head) pair
  if ((int64_t)n_seqs * heads > ((int64_t)1 << 27)) return KDA_ERR_SHAPE;
  if (T > 0 && (!q || !k || !v || !log_alpha || !beta || !o)) return KDA_ERR_NULL;
  if (!aligned16({q, k, v, log_alpha, h0, o, h_final}) || !aligned4({beta, cu_seqlens}))
    return KDA_ERR_ALIGN;
  const size_t need = workspace_min_bytes(n_seqs, T, heads, io);
  if (need == 0) return KDA_ERR_SHAPE;
  if (!workspace || workspace_bytes_given < need || ((uintptr_t)workspace & 255u))
    return KDA_ERR_WORKSPACE;
  // window of chunk slots: as many as the given workspace holds blocks for
  const int64_t slots = chunk_slots(n_seqs, T);
  const int64_t per_slot = (int64_t)heads * block_bytes(io);
  const int64_t fit = ((int64_t)std::min<size_t>(workspace_bytes_given, (size_t)INT64_MAX) -
                       inter_offset(n_seqs, heads)) / per_slot;
  const int64_t win = std::min(slots, fit);
  // a single phase launch covers every chunk only when one window does
  if (phases != 7 && win < slots) return KDA_ERR_WORKSPACE;
  const int64_t used = inter_offset(n_seqs, heads) + win * per_slot;

  const int64_t th = T * heads;
  const int64_t eb = io_bytes(io);
  const Range rq(q, th * kDim * eb), rk(k, th * kDim * eb), rv(v, th * kDim * eb);
  const Range rla(log_alpha, th * kDim * 4), rb(beta, th * 4);
  const Range ro(o, th * kDim * eb);
  const int64_t state_bytes =
      (int64_t)n_seqs * heads * kDim * kDim * ((flags & KDA_FLAG_STATE_BF16) ? 2 : 4);
  const Range rh0(h0, state_bytes), rhf(h_final, state_bytes);
  const Range rcu(cu_seqlens, 4 * ((int64_t)n_seqs + 1));
  const Range rws(workspace, used);
  for (const Range* in : {&rq, &rk, &rv, &rla, &rb, &rh0, &rcu, &rws})
    if (overlap(ro, *in)) return KDA_ERR_ALIAS;
  for (const Range* in : {&rq, &rk, &rv, &rla, &rb, &ro, &rcu, &rws})
    if (overlap(rhf, *in)) return KDA_ERR_ALIAS;
  if (overlap(rhf, rh0) && rhf.lo != rh0.lo) return KDA_ERR_ALIAS;
  for (const Range* in : {&rq, &rk, &rv, &rla, &rb, &rh0, &rcu})
    if (overlap(rws, *in)) return KDA_ERR_ALIAS;

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* status = reinterpret_cast<int32_t*>(ws);
  int32_t* chunk_offset = reinterpret_cast<int32_t*>(ws + 256);
  float* state_area = reinterpret_cast<float*>(ws + state_offset(n_seqs));
  uint8_t* inter = ws + inter_offset(n_seqs, heads);
  const hipError_t err = kda::launch_chunk_fwd(
      phases, io == KDA_IO_BF16, (flags & KDA_FLAG_QK_L2NORM) != 0,
      (flags & KDA_FLAG_STATE_BF16) != 0, q, k, v, log_alpha, beta, h0, cu_seqlens, n_seqs,
      T, heads, slots, std::max<int64_t>(win, 1), o, h_final, status, chunk_offset,
      state_area, inter, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" {

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v,
                         const float* log_alpha, const float* beta, const void* h0,
                         const int32_t* cu_seqlens, int32_t n_seqs, int64_t total_tokens,
                         int32_t heads, int32_t dk, int32_t dv, kda_io_dtype io,
                         uint32_t flags, void* o, void* h_final, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return chunk_fwd_impl(7, q, k, v, log_alpha, beta, h0, cu_seqlens, n_seqs, total_tokens,
                        heads, dk, dv, raw(io), flags, o, h_final, workspace, workspace_bytes,
                        stream);
}

kda_status kda_chunk_fwd_phase(int32_t phase, const void* q, const void* k, const void* v,
                               const float* log_alpha, const float* beta, const void* h0,
                               const int32_t* cu_seqlens, int32_t n_seqs,
                               int64_t total_tokens, int32_t heads, int32_t dk, int32_t dv,
                               kda_io_dtype io, uint32_t flags, void* o, void* h_final,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (phase < 0 || phase > 2) return KDA_ERR_SHAPE;
  return chunk_fwd_impl(1 << phase, q, k, v, log_alpha, beta, h0, cu_seqlens, n_seqs,
                        total_tokens, heads, dk, dv, raw(io), flags, o, h_final, workspace,
                        workspace_bytes, stream);
}

kda_status kda_decode_step(const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta, float* S_inout,
                           int32_t n_seqs, int32_t heads, int32_t dk, int32_t dv,
                           kda_io_dtype io_arg, void* o, void* stream) {
  const int io = raw(io_arg);
  if (n_seqs < 0 || heads < 1) return KDA_ERR_SHAPE;
  if (dk != kDim || dv != kDim || !valid_io(io)) return KDA_ERR_UNSUPPORTED;
  if (n_seqs == 0) return KDA_OK;
  if (!q || !k || !v || !log_alpha || !beta || !S_inout || !o) return KDA_ERR_NULL;
  if (!aligned16({q, k, v, log_alpha, S_inout, o}) || !aligned4({beta})) return KDA_ERR_ALIGN;
  const int64_t pairs = (int64_t)n_seqs * heads;
  if (pairs > ((int64_t)1 << 29)) return KDA_ERR_SHAPE;  // grid of 4 waves per pair
  const int64_t eb = io_bytes(io);
  const Range rq(q, pairs * kDim * eb), rk(k, pairs * kDim * eb), rv(v, pairs * kDim * eb);
  const Range rla(log_alpha, pairs * kDim * 4), rb(beta, pairs * 4);
  const Range rs(S_inout, pairs * kDim * kDim * 4), ro(o, pairs * kDim * eb);
  for (const Range* in : {&rq, &rk, &rv, &rla, &rb, &ro})
    if (overlap(rs, *in)) return KDA_ERR_ALIAS;
  for (const Range* in : {&rq, &rk, &rv, &rla, &rb})
    if (overlap(ro, *in)) return KDA_ERR_ALIAS;
  // one token per sequence through the fused recurrent kernel, state in place
  const hipError_t err = kda::launch_recurrent_fwd(
      io == KDA_IO_BF16, false, false, q, k, v, log_alpha, beta, S_inout, nullptr, 1, n_seqs,
      heads, pairs, o, S_inout, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_recurrent_fwd(const void* q, const void* k, const void* v,
                             const float* log_alpha, const float* beta, const void* h0,
                             const int32_t* cu_seqlens, int32_t n_seqs, int64_t total_tokens,
                             int32_t heads, int32_t dk, int32_t dv, kda_io_dtype io_arg,
                             kda_state_dtype state_arg, uint32_t flags, void* o,
                             void* h_final, void* stream) {
  const int io = raw(io_arg), state_dtype = raw(state_arg);
  const int64_t T = total_tokens;
  if (T < 0 || n_seqs < 0 || heads < 1) return KDA_ERR_SHAPE;
  if (dk != kDim || dv != kDim || !valid_io(io)) return KDA_ERR_UNSUPPORTED;
  if (state_dtype != KDA_STATE_F32 && state_dtype != KDA_STATE_BF16) return KDA_ERR_UNSUPPORTED;
  if (flags & ~(uint32_t)KDA_FLAG_QK_L2NORM) return KDA_ERR_UNSUPPORTED;
  if (n_seqs == 0) return T == 0 ? KDA_OK : KDA_ERR_SHAPE;
  if (cu_seqlens == nullptr && T % n_seqs != 0) return KDA_ERR_SHAPE;
  if (cu_seqlens != nullptr && T > INT32_MAX) return KDA_ERR_SHAPE;
  const int64_t pairs = (int64_t)n_seqs * heads;
  if (pairs > ((int64_t)1 << 29)) return KDA_ERR_SHAPE;  // grid of 4 waves per pair
  if (T > 0 && (!q || !k || !v || !log_alpha || !beta || !o)) return KDA_ERR_NULL;
  if (!aligned16({q, k, v, log_alpha, h0, o, h_final}) || !aligned4({beta, cu_seqlens}))
    return KDA_ERR_ALIGN;

  const int64_t th = T * heads;
  const int64_t eb = io_bytes(io);
  const Range rq(q, th * kDim * eb), rk(k, th * kDim * eb), rv(v, th * kDim * eb);
  const Range rla(log_alpha, th * kDim * 4), rb(beta, th * 4);
  const Range ro(o, th * kDim * eb);
  const int64_t state_bytes = pairs * kDim * kDim * (state_dtype == KDA_STATE_BF16 ? 2 : 4);
  const Range rh0(h0, state_bytes), rhf(h_final, state_bytes);
  const Range rcu(cu_seqlens, 4 * ((int64_t)n_seqs + 1));
  for (const Range* in : {&rq, &rk, &rv, &rla, &rb, &rh0, &rcu, &rhf})
    if (overlap(ro, *in)) return KDA_ERR_ALIAS;
  for (const Range* in : {&rq, &rk, &rv, &rla, &rb, &rcu})
    if (overlap(rhf, *in)) return KDA_ERR_ALIAS;
  if (overlap(rhf, rh0) && rhf.lo != rh0.lo) return KDA_ERR_ALIAS;

  const hipError_t err = kda::launch_recurrent_fwd(
      io == KDA_IO_BF16, state_dtype == KDA_STATE_BF16, (flags & KDA_FLAG_QK_L2NORM) != 0, q,
      k, v, log_alpha, beta, h0, cu_seqlens, cu_seqlens ? 0 : T / n_seqs, T, heads, pairs, o,
      h_final, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_rmsnorm_gate(const void* o, const void* gate, const float* weight, float eps,
                            int64_t rows, int32_t dv, kda_io_dtype io_arg, void* y,
                            void* stream) {
  const int io = raw(io_arg);
  if (rows < 0 || !(eps >= 0.f) || eps > 3.0e38f) return KDA_ERR_SHAPE;
  if (dv != kDim || !valid_io(io)) return KDA_ERR_UNSUPPORTED;
  if (rows == 0) return KDA_OK;
  if (rows > ((int64_t)1 << 36)) return KDA_ERR_SHAPE;
  if (!o || !gate || !y) return KDA_ERR_NULL;
  if (!aligned16({o, gate, weight, y})) return KDA_ERR_ALIGN;
  const int64_t bytes = rows * kDim * io_bytes(io);
  const Range ro(o, bytes), rg(gate, bytes), rw(weight, kDim * 4), ry(y, bytes);
  if (overlap(ry, ro) && ry.lo != ro.lo) return KDA_ERR_ALIAS;
  if (overlap(ry, rg) || overlap(ry, rw)) return KDA_ERR_ALIAS;
  const hipError_t err = kda::launch_rmsnorm_gate(io == KDA_IO_BF16, o, gate, weight, eps, rows,
                                                  y, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_check_inputs(const void* q, const void* k, const void* v, const float* log_alpha,
                            const float* beta, const int32_t* cu_seqlens, int32_t n_seqs,
                            int64_t total_tokens, int32_t heads, int32_t dk, int32_t dv,
                            kda_io_dtype io_arg, int32_t* flags, void* stream) {
  const int io = raw(io_arg);
  const int64_t T = total_tokens;
  if (T < 0 || heads < 1 || (cu_seqlens != nullptr && n_seqs < 1)) return KDA_ERR_SHAPE;
  if (dk != kDim || dv != kDim || !valid_io(io) || heads > 65535) return KDA_ERR_UNSUPPORTED;
  if (cu_seqlens != nullptr && T > INT32_MAX) return KDA_ERR_SHAPE;
  if (T > ((int64_t)1 << 40) / heads) return KDA_ERR_SHAPE;
  if (!flags) return KDA_ERR_NULL;
  if (T > 0 && (!q || !k || !v || !log_alpha || !beta)) return KDA_ERR_NULL;
  if (!aligned16({q, k, v, log_alpha}) || !aligned4({beta, cu_seqlens, flags}))
    return KDA_ERR_ALIGN;
  const int64_t th = T * heads, eb = io_bytes(io);
  const Range rf(flags, 4);
  const Range rq(q, th * kDim * eb), rk(k, th * kDim * eb), rv(v, th * kDim * eb);
  const Range rla(log_alpha, th * kDim * 4), rb(beta, th * 4);
  const Range rcu(cu_seqlens, cu_seqlens ? 4 * ((int64_t)n_seqs + 1) : 0);
  for (const Range* in : {&rq, &rk, &rv, &rla, &rb, &rcu})
    if (overlap(rf, *in)) return KDA_ERR_ALIAS;
  const hipError_t err = kda::launch_check_inputs(
      io == KDA_IO_BF16, q, k, v, log_alpha, beta, cu_seqlens, cu_seqlens ? n_seqs : 0, T,
      heads, flags, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

const char* kda_status_string(kda_status s) {
  switch (raw(s)) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_SHAPE: return "a size is negative or inconsistent";
    case KDA_ERR_UNSUPPORTED: return "unsupported head size or dtype (d_k = d_v = 128 only)";
    case KDA_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case KDA_ERR_ALIAS: return "an output overlaps an input it must not";
    case KDA_ERR_HIP: return "the HIP runtime reported a launch error";
    case KDA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned (beta, cu_seqlens: 4)";
    case KDA_ERR_SCRATCH:
      return "the call needs more workspace than the allocation-free entry point holds";
  }
  return "unknown status";
}

int32_t kda_version(void) { return 200; }

}  // extern "C"
