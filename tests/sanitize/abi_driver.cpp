// Drives the C ABI's host side (gated_delta_rule_50_amd/csrc/kda_api.cpp)
// in a build under AddressSanitizer and UndefinedBehaviorSanitizer. The
// kernel launchers are replaced by stubs that count calls, so valid calls
// run through every check and into the launch sequencing without a GPU.
// All tensor pointers are fake addresses: the host side never dereferences
// them. Exits non-zero on a wrong status or launch count.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include "kda.h"

namespace kda {
int g_chunk = 0, g_rec = 0, g_epi = 0, g_chk = 0;
int64_t g_win = -1;   // window size of the last chunk launch
hipError_t launch_chunk_fwd(int, bool, bool, bool, const void*, const void*, const void*,
                            const float*, const float*, const void*, const int32_t*, int32_t,
                            int64_t, int32_t, int64_t, int64_t win_slots, void*, void*, int32_t*,
                            int32_t*, float*, uint8_t*, hipStream_t) {
  ++g_chunk;
  g_win = win_slots;
  return hipSuccess;
}
// per chunk-head block: [-W ; Qt], K'^T, [U ; Ut] in the I/O type, gamma_C fp32
size_t inter_block_bytes(bool bf16_io) { return (16384 + 8192 + 16384) * (bf16_io ? 2 : 4) + 512; }
hipError_t launch_recurrent_fwd(bool, bool, bool, const void*, const void*, const void*,
                                const float*, const float*, const void*, const int32_t*, int64_t,
                                int64_t, int32_t, int64_t, void*, void*, hipStream_t) {
  ++g_rec;
  return hipSuccess;
}
hipError_t launch_rmsnorm_gate(bool, const void*, const void*, const float*, float, int64_t, void*,
                               hipStream_t) {
  ++g_epi;
  return hipSuccess;
}
hipError_t launch_check_inputs(bool, const void*, const void*, const void*, const float*,
                               const float*, const int32_t*, int32_t, int64_t, int32_t, int32_t*,
                               hipStream_t) {
  ++g_chk;
  return hipSuccess;
}
}  // namespace kda

static int fails = 0;
static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
    ++fails;
  }
}
static void* at(uintptr_t off) { return reinterpret_cast<void*>((uintptr_t)0x7F0000000000ull + off); }

int main() {
  const uintptr_t MB = 1 << 20;
  const int T = 100, H = 2;
  const size_t ws = kda_chunk_fwd_workspace_bytes(1, T, H, 128, 128, KDA_IO_BF16);
  const size_t ws_min = kda_chunk_fwd_workspace_min_bytes(1, T, H, 128, 128, KDA_IO_BF16);
  auto prefill = [&](const void* q, const void* o, const float* h0, float* hf, const void* wsp,
                     size_t wsb, int32_t n, const int32_t* cu, int64_t t, uint32_t flags) {
    return (int)kda_chunk_fwd(q, at(1 * 64 * MB), at(2 * 64 * MB), (const float*)at(3 * 64 * MB),
                              (const float*)at(4 * 64 * MB), h0, cu, n, t, H, 128, 128,
                              KDA_IO_BF16, flags, const_cast<void*>(o), hf,
                              const_cast<void*>(wsp), wsb, nullptr);
  };
  const float* h0 = (const float*)at(5 * 64 * MB);
  float* hf = (float*)at(8 * 64 * MB);
  const void* o = at(7 * 64 * MB);
  const void* w = at(9 * 64 * MB);
  expect(prefill(at(0), o, h0, hf, w, ws, 1, nullptr, T, 0), KDA_OK, "prefill valid");
  expect(prefill(at(0), o, nullptr, nullptr, w, ws, 1, nullptr, 0, 0), KDA_OK, "prefill T=0");
  expect(prefill(nullptr, o, h0, hf, w, ws, 1, nullptr, T, 0), KDA_ERR_NULL, "prefill q NULL");
  expect(prefill(at(8), o, h0, hf, w, ws, 1, nullptr, T, 0), KDA_ERR_ALIGN, "prefill misaligned");
  expect(prefill(at(0), o, h0, hf, w, ws_min - 1, 1, nullptr, T, 0), KDA_ERR_WORKSPACE,
         "workspace");
  expect(prefill(at(0), o, h0, hf, w, ws_min, 1, nullptr, T, 0), KDA_OK, "one-slot window");
  if (kda::g_win != 1) ++fails;
  expect(prefill(at(0), o, h0, hf, w, ws, 1, nullptr, T, 0), KDA_OK, "one window");
  if (kda::g_win != 2) ++fails;
  expect((int)kda_chunk_fwd_phase(1, at(0), at(64 * MB), at(128 * MB),
                                  (const float*)at(192 * MB), (const float*)at(256 * MB), h0,
                                  nullptr, 1, T, H, 128, 128, KDA_IO_BF16, 0,
                                  const_cast<void*>(o), hf, const_cast<void*>(w), ws_min, nullptr),
         KDA_ERR_WORKSPACE, "phase with a partial window");
  expect(prefill(at(0), at(4096), h0, hf, w, ws, 1, nullptr, T, 0), KDA_ERR_ALIAS, "o over q");
  expect(prefill(at(0), o, h0, hf, w, ws, 1, nullptr, T, 4), KDA_ERR_UNSUPPORTED, "flag");
  expect(prefill(at(0), o, h0, hf, w, ws, 1, nullptr, T, 2), KDA_OK, "bf16 state flag");
  expect(prefill(at(0), o, h0, hf, w, ws, 1, nullptr, -1, 0), KDA_ERR_SHAPE, "T < 0");
  expect(prefill(at(0), o, h0, hf, w, ws, 1 << 27, (const int32_t*)at(6 * 64 * MB), T, 0),
         KDA_ERR_SHAPE, "pairs");   // 2^27 sequences x 2 heads
  expect((int)kda_chunk_fwd(at(0), at(64 * MB), at(128 * MB), (const float*)at(192 * MB),
                            (const float*)at(256 * MB), h0, nullptr, 1, T, H, 128, 128,
                            (kda_io_dtype)5, 0, const_cast<void*>(o), hf, const_cast<void*>(w),
                            ws, nullptr), KDA_ERR_UNSUPPORTED, "io dtype 5");
  if (kda_chunk_fwd_workspace_bytes(1, T, H, 128, 128, (kda_io_dtype)-3) != 0) ++fails;
  for (int ph = 0; ph < 3; ++ph)
    expect((int)kda_chunk_fwd_phase(ph, at(0), at(64 * MB), at(128 * MB),
                                    (const float*)at(192 * MB), (const float*)at(256 * MB), h0,
                                    nullptr, 1, T, H, 128, 128, KDA_IO_BF16, 0,
                                    const_cast<void*>(o), hf, const_cast<void*>(w), ws, nullptr),
           KDA_OK, "phase");
  expect((int)kda_chunk_fwd_phase(3, at(0), at(64 * MB), at(128 * MB), (const float*)at(192 * MB),
                                  (const float*)at(256 * MB), h0, nullptr, 1, T, H, 128, 128,
                                  KDA_IO_BF16, 0, const_cast<void*>(o), hf,
                                  const_cast<void*>(w), ws, nullptr),
         KDA_ERR_SHAPE, "phase 3");
  // decode
  float* S = (float*)at(64 * MB);
  expect((int)kda_decode_step(at(0), at(MB), at(2 * MB), (const float*)at(3 * MB),
                              (const float*)at(4 * MB), S, 4, 2, 128, 128, KDA_IO_BF16,
                              at(5 * MB), nullptr), KDA_OK, "decode valid");
  expect((int)kda_decode_step(at(0), at(MB), at(2 * MB), (const float*)at(3 * MB),
                              (const float*)at(4 * MB), (float*)at(1024), 4, 2, 128, 128,
                              KDA_IO_BF16, at(5 * MB), nullptr), KDA_ERR_ALIAS, "decode alias");
  // recurrent
  expect((int)kda_recurrent_fwd(at(0), at(MB), at(2 * MB), (const float*)at(3 * MB),
                                (const float*)at(4 * MB), at(64 * MB), nullptr, 4, 8, 2, 128, 128,
                                KDA_IO_BF16, KDA_STATE_BF16, KDA_FLAG_QK_L2NORM, at(5 * MB),
                                at(64 * MB), nullptr), KDA_OK, "recurrent valid");
  expect((int)kda_recurrent_fwd(at(0), at(MB), at(2 * MB), (const float*)at(3 * MB),
                                (const float*)at(4 * MB), at(64 * MB), nullptr, 4, 9, 2, 128, 128,
                                KDA_IO_BF16, KDA_STATE_F32, 0, at(5 * MB), at(64 * MB), nullptr),
         KDA_ERR_SHAPE, "recurrent T % N");
  expect((int)kda_recurrent_fwd(at(0), at(MB), at(2 * MB), (const float*)at(3 * MB),
                                (const float*)at(4 * MB), at(64 * MB), nullptr, 4, 8, 2, 128, 128,
                                KDA_IO_BF16, (kda_state_dtype)7, 0, at(5 * MB), at(64 * MB),
                                nullptr), KDA_ERR_UNSUPPORTED, "state dtype 7");
  expect((int)kda_decode_step(at(0), at(MB), at(2 * MB), (const float*)at(3 * MB),
                              (const float*)at(4 * MB), S, 4, 2, 128, 128, (kda_io_dtype)9,
                              at(5 * MB), nullptr), KDA_ERR_UNSUPPORTED, "decode io 9");
  // epilogue
  expect((int)kda_rmsnorm_gate(at(0), at(MB), (const float*)at(2 * MB), 1e-6f, 64, 128,
                               KDA_IO_BF16, at(0), nullptr), KDA_OK, "epilogue in place");
  expect((int)kda_rmsnorm_gate(at(0), at(MB), (const float*)at(2 * MB), -1.f, 64, 128,
                               KDA_IO_BF16, at(3 * MB), nullptr), KDA_ERR_SHAPE, "epilogue eps");
  // input check
  int32_t* fl = (int32_t*)at(10 * 64 * MB);
  const int32_t* cu = (const int32_t*)at(6 * 64 * MB);
  expect((int)kda_check_inputs(at(0), at(MB), at(2 * MB), (const float*)at(3 * MB),
                               (const float*)at(4 * MB), cu, 3, 8, 2, 128, 128, KDA_IO_BF16, fl,
                               nullptr), KDA_OK, "check valid");
  expect((int)kda_check_inputs(at(0), at(MB), at(2 * MB), (const float*)at(3 * MB),
                               (const float*)at(4 * MB), nullptr, 0, 0, 2, 128, 128, KDA_IO_F32,
                               fl, nullptr), KDA_OK, "check T=0");
  expect((int)kda_check_inputs(at(0), at(MB), at(2 * MB), (const float*)at(3 * MB),
                               (const float*)at(4 * MB), cu, 3, 8, 2, 128, 128, KDA_IO_BF16,
                               (int32_t*)at(MB + 64), nullptr), KDA_ERR_ALIAS, "check alias");
  expect((int)kda_check_inputs(at(0), at(MB), at(2 * MB), (const float*)at(3 * MB),
                               (const float*)at(4 * MB), cu, 3, 8, 2, 128, 128, (kda_io_dtype)4,
                               fl, nullptr), KDA_ERR_UNSUPPORTED, "check io 4");
  for (int st = -1; st < 9; ++st)
    if (kda_status_string((kda_status)st) == nullptr) ++fails;
  if (kda::g_chunk != 8 || kda::g_rec != 2 || kda::g_epi != 1 || kda::g_chk != 2) {
    fprintf(stderr, "launch counts %d %d %d %d\n", kda::g_chunk, kda::g_rec, kda::g_epi,
            kda::g_chk);
    ++fails;
  }
  if (!fails) printf("abi driver ok\n");
  return fails ? 1 : 0;
}
