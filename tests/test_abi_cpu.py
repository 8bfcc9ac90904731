"""C ABI checks that need no GPU: the library loads, exports every entry point
include/kda.h declares, and rejects bad arguments before launching anything.

All pointers here are fake addresses; the argument checks never dereference
them, and every call below returns before the first HIP call.
"""
import ctypes
import re
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "kda.h"
LIB = ROOT / "gated_delta_rule_50_amd" / "libkda.so"

OK, NULL, SHAPE, UNSUP, WS, ALIAS, HIPERR, ALIGN, SCRATCH = range(9)
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def lib():
    if not LIB.exists():
        pytest.skip("libkda.so not built (run python -m gated_delta_rule_50_amd.build)")
    L = ctypes.CDLL(str(LIB))
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.kda_chunk_fwd_workspace_bytes.argtypes = [i32, i64, i32, i32, i32, ctypes.c_int]
    L.kda_chunk_fwd_workspace_bytes.restype = sz
    L.kda_chunk_fwd_workspace_min_bytes.argtypes = [i32, i64, i32, i32, i32, ctypes.c_int]
    L.kda_chunk_fwd_workspace_min_bytes.restype = sz
    L.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                ctypes.c_int, ctypes.c_uint32, vp, vp, vp, sz, vp]
    L.kda_chunk_fwd.restype = ctypes.c_int
    L.kda_chunk_fwd_phase.argtypes = [i32] + L.kda_chunk_fwd.argtypes
    L.kda_chunk_fwd_phase.restype = ctypes.c_int
    L.kda_chunk_fwd_noalloc.argtypes = L.kda_chunk_fwd.argtypes[:16] + [vp]
    L.kda_chunk_fwd_noalloc.restype = ctypes.c_int
    L.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_int,
                                  vp, vp]
    L.kda_decode_step.restype = ctypes.c_int
    L.kda_recurrent_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_uint32, vp, vp, vp]
    L.kda_recurrent_fwd.restype = ctypes.c_int
    L.kda_rmsnorm_gate.argtypes = [vp, vp, vp, ctypes.c_float, i64, i32, ctypes.c_int, vp, vp]
    L.kda_rmsnorm_gate.restype = ctypes.c_int
    L.kda_check_inputs.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                   ctypes.c_int, vp, vp]
    L.kda_check_inputs.restype = ctypes.c_int
    L.kda_status_string.argtypes = [ctypes.c_int]
    L.kda_status_string.restype = ctypes.c_char_p
    L.kda_version.restype = i32
    return L


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("kda_chunk_fwd", "kda_decode_step", "kda_chunk_fwd_workspace_bytes",
                     "kda_recurrent_fwd", "kda_status_string"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_binding_names_match_header():
    from gated_delta_rule_50_amd import kda
    assert sorted(kda.EXPORTS) == declared_functions()


def test_status_strings_and_version(lib):
    for s in range(8):
        assert lib.kda_status_string(s)
    assert lib.kda_status_string(99) == b"unknown status"
    assert lib.kda_version() >= 200


# ------------------------------------------------------------ workspace size
def _block_bytes(io):
    e = 2 if io == BF16 else 4
    return 40960 * e + 128 * 4


@pytest.mark.parametrize("io", [F32, BF16])
@pytest.mark.parametrize("N,T,H", [(1, 0, 1), (1, 1, 1), (1, 8192, 32), (16, 135000, 32),
                                   (3, 64, 2), (300, 100000, 4), (1, 1 << 20, 32),
                                   (1, 1 << 24, 64), (16, 1 << 22, 32)])
def test_workspace_formula(lib, io, N, T, H):
    """Recommended size: the whole call's blocks up to 512 MiB of them for one
    bf16 sequence (1 GiB in fp32: as many chunk slots; 8 GiB for a packed
    batch), else that much (it stops growing with T); smallest: one chunk
    slot."""
    slots = (T + 63) // 64 + N - 1
    inter = 256 + (4 * (N + 1) + 255) // 256 * 256 + 2 * H * 128 * 128 * 4
    per_slot = H * _block_bytes(io)
    cap = ((1024 << 20) if io == F32 else (512 << 20)) if N == 1 else (8 << 30)
    win = min(slots, max(1, cap // per_slot))
    assert lib.kda_chunk_fwd_workspace_bytes(N, T, H, 128, 128, io) == inter + win * per_slot
    assert lib.kda_chunk_fwd_workspace_min_bytes(N, T, H, 128, 128, io) == \
        inter + (per_slot if slots > 0 else 0)
    assert lib.kda_chunk_fwd_workspace_bytes(N, T, H, 128, 128, io) <= inter + cap + per_slot


def test_workspace_for_a_long_call_is_bounded(lib):
    """A million-token call needs no more workspace than a 16K-token one."""
    big = lib.kda_chunk_fwd_workspace_bytes(1, 1 << 20, 32, 128, 128, BF16)
    mid = lib.kda_chunk_fwd_workspace_bytes(1, 1 << 14, 32, 128, 128, BF16)
    assert big == mid < (600 << 20)


def test_workspace_invalid(lib):
    for f in (lib.kda_chunk_fwd_workspace_bytes, lib.kda_chunk_fwd_workspace_min_bytes):
        assert f(0, 10, 1, 128, 128, BF16) == 0
        assert f(1, -1, 1, 128, 128, BF16) == 0
        assert f(1, 10, 70000, 128, 128, BF16) == 0
        assert f(1, 10, 1, 128, 64, BF16) == 0
    assert lib.kda_chunk_fwd_workspace_bytes(0, 10, 1, 128, 128, BF16) == 0
    assert lib.kda_chunk_fwd_workspace_bytes(1, -1, 1, 128, 128, BF16) == 0
    assert lib.kda_chunk_fwd_workspace_bytes(1, 10, 0, 128, 128, BF16) == 0
    assert lib.kda_chunk_fwd_workspace_bytes(1, 10, 1, 64, 128, BF16) == 0
    assert lib.kda_chunk_fwd_workspace_bytes(1, 10, 1, 128, 128, 7) == 0


# ------------------------------------------------------ prefill validation
BASE = 0x7F0000000000          # fake, 256-byte aligned, never dereferenced
MB = 1 << 20


def prefill_args(lib, T=100, H=2, N=1, io=BF16, **over):
    e = 2 if io == BF16 else 4
    th = T * H
    a = dict(q=BASE, k=BASE + 1 * 64 * MB, v=BASE + 2 * 64 * MB, log_alpha=BASE + 3 * 64 * MB,
             beta=BASE + 4 * 64 * MB, h0=BASE + 5 * 64 * MB,
             cu=(BASE + 6 * 64 * MB) if N != 1 else None, N=N, T=T, H=H, dk=128, dv=128,
             io=io, flags=0, o=BASE + 7 * 64 * MB, h_final=BASE + 8 * 64 * MB,
             ws=BASE + 9 * 64 * MB, ws_bytes=None, stream=None)
    a.update(over)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = lib.kda_chunk_fwd_workspace_bytes(a["N"] if a["N"] > 0 else 1,
                                                          max(a["T"], 0), max(a["H"], 1),
                                                          128, 128, io) or 0
    assert th * 128 * e < 64 * MB
    return a


def call_prefill(lib, a, phase=None):
    args = (a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["h0"], a["cu"], a["N"],
            a["T"], a["H"], a["dk"], a["dv"], a["io"], a["flags"], a["o"], a["h_final"], a["ws"],
            a["ws_bytes"], a["stream"])
    if phase is None:
        return lib.kda_chunk_fwd(*args)
    return lib.kda_chunk_fwd_phase(phase, *args)


@pytest.mark.parametrize("over,expect", [
    (dict(T=-1), SHAPE),
    (dict(N=0), SHAPE),
    (dict(H=0), SHAPE),
    (dict(dk=64), UNSUP),
    (dict(dv=256), UNSUP),
    (dict(io=5), UNSUP),
    (dict(H=70000), UNSUP),
    (dict(flags=4), UNSUP),
    (dict(flags=0x80000000), UNSUP),
    (dict(q=None), NULL),
    (dict(beta=None), NULL),
    (dict(o=None), NULL),
    (dict(N=2, cu=None), NULL),
    (dict(ws=None), WS),
    (dict(ws_bytes=100), WS),
    (dict(ws=BASE + 9 * 64 * MB + 128), WS),
])
def test_prefill_argument_errors(lib, over, expect):
    a = prefill_args(lib)
    a.update(over)
    assert call_prefill(lib, a) == expect


@pytest.mark.parametrize("name,off", [("q", 8), ("k", 2), ("v", 4), ("log_alpha", 4),
                                      ("h0", 8), ("o", 8), ("h_final", 4), ("beta", 2)])
def test_prefill_misaligned_pointer(lib, name, off):
    a = prefill_args(lib)
    assert call_prefill(lib, dict(a, **{name: a[name] + off})) == ALIGN
    assert call_prefill(lib, dict(a, N=2, cu=BASE + 6 * 64 * MB + 2)) == ALIGN


def test_alignment_checked_on_every_entry_point(lib):
    assert call_decode(lib, q=BASE + 8) == ALIGN
    assert call_decode(lib, S=BASE + 64 * MB + 4) == ALIGN
    assert call_decode(lib, beta=BASE + 4 * MB + 2) == ALIGN
    assert call_recurrent(lib, h0=BASE + 64 * MB + 8) == ALIGN
    assert call_recurrent(lib, cu=BASE + 6 * MB + 1) == ALIGN
    assert call_recurrent(lib, o=BASE + 5 * MB + 8) == ALIGN
    assert call_epilogue(lib, w=BASE + 2 * MB + 4) == ALIGN
    assert call_epilogue(lib, y=BASE + 3 * MB + 8) == ALIGN
    # 16-byte multiples pass the check (and then fail on the alias test)
    assert call_epilogue(lib, y=BASE + 16) == ALIAS


def test_prefill_alias_errors(lib):
    a = prefill_args(lib)
    assert call_prefill(lib, dict(a, o=a["q"] + 4096)) == ALIAS          # o inside q
    assert call_prefill(lib, dict(a, h_final=a["o"])) == ALIAS            # h_final = o
    assert call_prefill(lib, dict(a, h_final=a["h0"] + 1024)) == ALIAS    # partial overlap
    assert call_prefill(lib, dict(a, ws=a["k"])) == ALIAS                 # workspace over k
    assert call_prefill(lib, dict(a, o=a["ws"] + 256)) == ALIAS           # o inside workspace


def test_prefill_state_size_follows_state_flag(lib):
    # 1 x 2 states are 128 KiB in fp32 and 64 KiB with KDA_FLAG_STATE_BF16;
    # o starting just before either end overlaps h0 (calls that pass every
    # check would launch, so only rejected calls appear here)
    a = prefill_args(lib)
    assert call_prefill(lib, dict(a, o=a["h0"] + 128 * 1024 - 256)) == ALIAS
    assert call_prefill(lib, dict(a, flags=2, o=a["h0"] + 64 * 1024 - 256)) == ALIAS
    assert call_prefill(lib, dict(a, flags=3, h_final=a["h0"] + 32 * 1024)) == ALIAS


def test_prefill_invalid_phase(lib):
    a = prefill_args(lib)
    assert call_prefill(lib, a, phase=3) == SHAPE
    assert call_prefill(lib, a, phase=-1) == SHAPE


def test_prefill_pair_limit(lib):
    # 2^20 sequences x 256 heads: more (sequence, head) pairs than the carry grid takes
    a = prefill_args(lib, N=2)
    assert call_prefill(lib, dict(a, N=1 << 20, H=256, T=1 << 20)) == SHAPE


def test_prefill_large_T_needs_int32_cu(lib):
    a = prefill_args(lib, N=2)
    a["T"] = 1 << 31
    assert call_prefill(lib, a) == SHAPE


# ------------------------------------------------------- decode validation
def call_decode(lib, **over):
    a = dict(q=BASE, k=BASE + MB, v=BASE + 2 * MB, la=BASE + 3 * MB, beta=BASE + 4 * MB,
             S=BASE + 64 * MB, N=4, H=2, dk=128, dv=128, io=BF16, o=BASE + 5 * MB, stream=None)
    a.update(over)
    return lib.kda_decode_step(a["q"], a["k"], a["v"], a["la"], a["beta"], a["S"], a["N"],
                               a["H"], a["dk"], a["dv"], a["io"], a["o"], a["stream"])


def test_decode_argument_errors(lib):
    assert call_decode(lib, N=-1) == SHAPE
    assert call_decode(lib, H=0) == SHAPE
    assert call_decode(lib, dk=96) == UNSUP
    assert call_decode(lib, io=3) == UNSUP
    assert call_decode(lib, q=None) == NULL
    assert call_decode(lib, S=None) == NULL
    assert call_decode(lib, S=BASE + 1024) == ALIAS           # state over q
    assert call_decode(lib, o=BASE + 64 * MB + 4096) == ALIAS  # o inside the state
    assert call_decode(lib, o=BASE + 3 * MB + 64) == ALIAS    # o over log_alpha


def test_decode_empty_batch_is_a_noop(lib):
    # returns before any HIP call
    assert call_decode(lib, N=0, q=None, S=None, o=None) == OK


# ---------------------------------------------------- recurrent validation
def call_recurrent(lib, **over):
    a = dict(q=BASE, k=BASE + MB, v=BASE + 2 * MB, la=BASE + 3 * MB, beta=BASE + 4 * MB,
             h0=BASE + 64 * MB, cu=None, N=4, T=8, H=2, dk=128, dv=128, io=BF16, st=F32,
             flags=0, o=BASE + 5 * MB, hf=BASE + 64 * MB, stream=None)
    a.update(over)
    return lib.kda_recurrent_fwd(a["q"], a["k"], a["v"], a["la"], a["beta"], a["h0"], a["cu"],
                                 a["N"], a["T"], a["H"], a["dk"], a["dv"], a["io"], a["st"],
                                 a["flags"], a["o"], a["hf"], a["stream"])


def test_recurrent_argument_errors(lib):
    assert call_recurrent(lib, T=-1) == SHAPE
    assert call_recurrent(lib, N=-1) == SHAPE
    assert call_recurrent(lib, H=0) == SHAPE
    assert call_recurrent(lib, T=9) == SHAPE                    # 9 tokens over 4 sequences
    assert call_recurrent(lib, N=0) == SHAPE                    # tokens but no sequence
    assert call_recurrent(lib, N=1 << 28, T=1 << 28, H=4) == SHAPE   # grid limit
    assert call_recurrent(lib, cu=BASE + 6 * MB, T=1 << 31) == SHAPE
    assert call_recurrent(lib, dk=64) == UNSUP
    assert call_recurrent(lib, io=2) == UNSUP
    assert call_recurrent(lib, st=2) == UNSUP
    assert call_recurrent(lib, flags=2) == UNSUP
    assert call_recurrent(lib, v=None) == NULL
    assert call_recurrent(lib, o=None) == NULL
    assert call_recurrent(lib, o=BASE + 2 * MB + 512) == ALIAS      # o over v
    assert call_recurrent(lib, o=BASE + 64 * MB + 4096) == ALIAS    # o inside the state
    assert call_recurrent(lib, hf=BASE + 3 * MB) == ALIAS           # h_final over log_alpha
    assert call_recurrent(lib, hf=BASE + 64 * MB + 2048) == ALIAS   # partial overlap of h0


def test_recurrent_state_size_follows_state_dtype(lib):
    # 4 x 2 states are 512 KiB in fp32 and 256 KiB in bf16; o starting just
    # before either end overlaps (calls that pass every check would launch, so
    # only rejected calls appear here)
    assert call_recurrent(lib, st=F32, hf=None, o=BASE + 64 * MB + 512 * 1024 - 16) == ALIAS
    assert call_recurrent(lib, st=BF16, hf=None, o=BASE + 64 * MB + 256 * 1024 - 16) == ALIAS


def test_recurrent_empty_batch_is_a_noop(lib):
    assert call_recurrent(lib, N=0, T=0, q=None, h0=None, o=None, hf=None) == OK


# ------------------------------------------------------ epilogue validation
def call_epilogue(lib, **over):
    a = dict(o=BASE, g=BASE + MB, w=BASE + 2 * MB, eps=1e-6, rows=64, dv=128, io=BF16,
             y=BASE + 3 * MB, stream=None)
    a.update(over)
    return lib.kda_rmsnorm_gate(a["o"], a["g"], a["w"], a["eps"], a["rows"], a["dv"], a["io"],
                                a["y"], a["stream"])


def test_epilogue_argument_errors(lib):
    assert call_epilogue(lib, rows=-1) == SHAPE
    assert call_epilogue(lib, eps=-1e-6) == SHAPE
    assert call_epilogue(lib, eps=float("nan")) == SHAPE
    assert call_epilogue(lib, eps=float("inf")) == SHAPE
    assert call_epilogue(lib, rows=(1 << 36) + 16) == SHAPE
    assert call_epilogue(lib, dv=64) == UNSUP
    assert call_epilogue(lib, io=9) == UNSUP
    assert call_epilogue(lib, o=None) == NULL
    assert call_epilogue(lib, g=None) == NULL
    assert call_epilogue(lib, y=None) == NULL
    assert call_epilogue(lib, y=BASE + 256) == ALIAS            # partial overlap of o
    assert call_epilogue(lib, y=BASE + MB - 256) == ALIAS       # over the gate
    assert call_epilogue(lib, y=BASE + 2 * MB - 1024) == ALIAS  # over the weight
    assert call_epilogue(lib, rows=0, o=None, g=None, y=None) == OK


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    from gated_delta_rule_50_amd import kda
    x = torch.zeros(4, 2, 128)
    with pytest.raises(ValueError):
        kda.decode_step(x, x, x, x, torch.zeros(4, 2), torch.zeros(4, 2, 128, 128))


def test_probe_library_rejects_bad_arguments():
    """The achievable-rate probes (bench.py's ceilings) load, export their
    entry points and refuse bad arguments before any launch."""
    path = ROOT / "probes" / "libkda_probes.so"
    if not path.exists():
        pytest.skip("libkda_probes.so not built")
    P = ctypes.CDLL(str(path))
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    P.kdab_read.argtypes = [vp, i64, vp, i32, vp]
    P.kdab_copy.argtypes = [vp, vp, i64, i32, i32, vp]
    P.kdab_rmw.argtypes = [vp, i64, i32, vp]
    P.kdab_mfma.argtypes = [vp, i64, i32, vp]
    P.kdab_valu.argtypes = [vp, i64, i32, vp]
    a, b, s = 0x10000, 0x20000000, 0x30000
    assert P.kdab_read(None, 1024, s, 64, None) == -1            # null buffer
    assert P.kdab_read(a + 4, 1024, s, 64, None) == -1           # misaligned
    assert P.kdab_read(a, 1000, s, 64, None) == -1               # not a multiple of 16
    assert P.kdab_read(a, 1024, None, 64, None) == -1            # no sink
    assert P.kdab_read(a, 1024, s, 0, None) == -1                # empty grid
    assert P.kdab_copy(a, a + 512, 1024, 1, 64, None) == -1      # overlapping
    assert P.kdab_copy(a, b, -16, 1, 64, None) == -1
    assert P.kdab_rmw(a, 0, 64, None) == -1
    assert P.kdab_mfma(s, 0, 64, None) == -1                     # no iterations
    assert P.kdab_valu(s, 10, (1 << 20) + 1, None) == -1         # grid too large


def test_check_inputs_rejects_bad_arguments(lib):
    """kda_check_inputs validates its arguments before any launch (fake
    addresses, never dereferenced)."""
    T, H = 10, 2
    q, k, v = 0x100000, 0x200000, 0x300000
    la, b, cu, fl = 0x400000, 0x500000, 0x600000, 0x700000
    call = lib.kda_check_inputs
    assert call(q, k, v, la, b, cu, 3, T, H, 128, 128, BF16, None, None) == NULL
    assert call(q, None, v, la, b, cu, 3, T, H, 128, 128, BF16, fl, None) == NULL
    assert call(q, k, v, la, b, cu, 3, -1, H, 128, 128, BF16, fl, None) == SHAPE
    assert call(q, k, v, la, b, cu, 0, T, H, 128, 128, BF16, fl, None) == SHAPE
    assert call(q, k, v, la, b, cu, 3, T, 0, 128, 128, BF16, fl, None) == SHAPE
    assert call(q, k, v, la, b, cu, 3, T, H, 64, 128, BF16, fl, None) == UNSUP
    assert call(q, k, v, la, b, cu, 3, T, H, 128, 128, 5, fl, None) == UNSUP
    assert call(q + 8, k, v, la, b, cu, 3, T, H, 128, 128, BF16, fl, None) == ALIGN
    assert call(q, k, v, la, b, cu, 3, T, H, 128, 128, BF16, fl + 2, None) == ALIGN
    assert call(q, k, v, la, b, cu, 3, T, H, 128, 128, BF16, q + 64, None) == ALIAS
    assert call(q, k, v, la, b, cu, 3, T, H, 128, 128, BF16, cu + 4, None) == ALIAS
    assert call(q, k, v, la, b, cu, 3, 1 << 40, H, 128, 128, BF16, fl, None) == SHAPE


def _host_prefill_args(T=130, H=3, N=2):
    torch = pytest.importorskip("torch")
    z = lambda *s, dt=torch.float32: torch.zeros(*s, dtype=dt)  # noqa: E731
    return dict(q=z(T, H, 128), k=z(T, H, 128), v=z(T, H, 128), log_alpha=z(T, H, 128),
                beta=z(T, H), h0=z(N, H, 128, 128),
                cu_seqlens=torch.tensor([0, 60, T], dtype=torch.int32),
                o=z(T, H, 128), h_final=z(N, H, 128, 128))


# one mis-shaped tensor per case: (argument, bad shape)
PREFILL_BAD = [("q", (130, 3, 64)), ("v", (130, 2, 128)), ("log_alpha", (129, 3, 128)),
               ("beta", (130,)), ("beta", (130, 3, 1)), ("h0", (3, 128, 128)),
               ("h0", (1, 3, 128, 128)), ("h_final", (2, 3, 128, 64)), ("o", (130, 3, 127)),
               ("cu_seqlens", (2, 2))]


@pytest.mark.parametrize("name,shape", PREFILL_BAD)
def test_binding_rejects_misshaped_prefill_tensor(name, shape):
    """Every tensor the prefill kernels index by (T, H, N, 128) is checked for
    its exact shape before anything reaches the library."""
    torch = pytest.importorskip("torch")
    from gated_delta_rule_50_amd import kda
    a = _host_prefill_args()
    a[name] = torch.zeros(*shape, dtype=a[name].dtype)
    with pytest.raises(ValueError, match="shape"):
        kda.Prefill(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["h0"],
                    a["cu_seqlens"], o=a["o"], h_final=a["h_final"])
    with pytest.raises(ValueError, match="shape"):
        kda.Recurrent(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["h0"],
                      a["cu_seqlens"], o=a["o"], h_final=a["h_final"])


def test_binding_shape_check_passes_good_shapes():
    """With every shape right, host tensors fail on the device check instead."""
    torch = pytest.importorskip("torch")
    from gated_delta_rule_50_amd import kda
    a = _host_prefill_args()
    for ctor in (kda.Prefill, kda.Recurrent):
        with pytest.raises(ValueError, match="GPU tensor"):
            ctor(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["h0"],
                 a["cu_seqlens"], o=a["o"], h_final=a["h_final"])
    with pytest.raises(ValueError, match="GPU tensor"):
        kda.check_inputs(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["cu_seqlens"])


@pytest.mark.parametrize("name,shape", [("q", (4, 2, 64)), ("v", (4, 3, 128)),
                                        ("log_alpha", (5, 2, 128)), ("beta", (4,)),
                                        ("S", (4, 2, 128, 64)), ("S", (2, 128, 128)),
                                        ("o", (4, 2, 100))])
def test_binding_rejects_misshaped_decode_tensor(name, shape):
    torch = pytest.importorskip("torch")
    from gated_delta_rule_50_amd import kda
    z = lambda *s: torch.zeros(*s)  # noqa: E731
    a = dict(q=z(4, 2, 128), k=z(4, 2, 128), v=z(4, 2, 128), log_alpha=z(4, 2, 128),
             beta=z(4, 2), S=z(4, 2, 128, 128), o=z(4, 2, 128))
    a[name] = z(*shape)
    with pytest.raises(ValueError, match="shape"):
        kda.decode_step(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["S"], o=a["o"])


@pytest.mark.parametrize("name,shape", [("gate", (10, 2, 128)), ("weight", (64,)),
                                        ("weight", (1, 128)), ("y", (10, 128)),
                                        ("o", (10, 3, 64))])
def test_binding_rejects_misshaped_epilogue_tensor(name, shape):
    torch = pytest.importorskip("torch")
    from gated_delta_rule_50_amd import kda
    a = dict(o=torch.zeros(10, 3, 128), gate=torch.zeros(10, 3, 128),
             weight=torch.zeros(128), y=torch.zeros(10, 3, 128))
    a[name] = torch.zeros(*shape)
    with pytest.raises(ValueError, match="shape"):
        kda.rmsnorm_gate(a["o"], a["gate"], a["weight"], y=a["y"])


@pytest.mark.parametrize("name,shape", [("q", (6, 2, 128, 1)), ("beta", (6, 3)),
                                        ("log_alpha", (6, 2, 64)), ("flags", (2,))])
def test_binding_rejects_misshaped_check_inputs_tensor(name, shape):
    torch = pytest.importorskip("torch")
    from gated_delta_rule_50_amd import kda
    z = lambda *s, dt=torch.float32: torch.zeros(*s, dtype=dt)  # noqa: E731
    a = dict(q=z(6, 2, 128), k=z(6, 2, 128), v=z(6, 2, 128), log_alpha=z(6, 2, 128),
             beta=z(6, 2), flags=z(1, dt=torch.int32))
    a[name] = z(*shape, dt=a[name].dtype)
    with pytest.raises(ValueError, match="shape"):
        kda.check_inputs(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], flags=a["flags"])


def test_noalloc_refuses_calls_beyond_its_array(lib):
    """kda_chunk_fwd_noalloc refuses, before any HIP call, a call whose
    smallest workspace (one chunk slot) exceeds its fixed array (fake
    addresses, never touched)."""
    cap = 128 << 20
    T, H = 64, 1024
    assert lib.kda_chunk_fwd_workspace_min_bytes(1, T, H, 128, 128, BF16) > cap
    assert lib.kda_chunk_fwd_workspace_min_bytes(1, 1 << 24, 32, 128, 128, BF16) <= cap
    p = [0x100000 * (i + 1) for i in range(9)]
    st = lib.kda_chunk_fwd_noalloc(p[0], p[1], p[2], p[3], p[4], None, None, 1, T, H, 128,
                                   128, BF16, 0, p[5], p[6], None)
    assert st == SCRATCH
    assert lib.kda_status_string(SCRATCH).decode().startswith("the call needs more workspace")


def test_workspace_below_minimum_and_phase_windows(lib):
    """Below the smallest size the call is refused; a phase launch needs
    every chunk slot in one window."""
    a = prefill_args(lib, T=1000, H=2)
    mn = lib.kda_chunk_fwd_workspace_min_bytes(1, 1000, 2, 128, 128, BF16)
    assert call_prefill(lib, dict(a, ws_bytes=mn - 1)) == WS
    for ph in (1, 2):
        assert call_prefill(lib, dict(a, ws_bytes=mn), phase=ph) == WS


def test_mode_switch_thresholds():
    """kda.forward's crossover: for bf16 I/O 16 tokens for one sequence and
    32 for more; for fp32 I/O 32 below 256 (sequence, head) pairs, 64 from
    256, 512 from 512 (the measurements are in kda.py)."""
    import torch
    from gated_delta_rule_50_amd import kda
    assert kda.recurrent_max_len(torch.bfloat16, 1, 32) == 16
    assert kda.recurrent_max_len(torch.bfloat16, 1, 1) == 16
    for n, h in ((2, 1), (2, 32), (16, 32), (256, 32)):
        assert kda.recurrent_max_len(torch.bfloat16, n, h) == 32
    assert [kda.recurrent_max_len(torch.float32, n, 32) for n in (1, 7, 8, 15, 16, 256)] \
        == [32, 32, 64, 64, 512, 512]
    assert kda.recurrent_max_len(torch.float32, 1, 16) == 32
