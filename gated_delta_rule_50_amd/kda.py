"""Thin Python binding of libkda.so (the C ABI in include/kda.h).

Argument marshalling only: torch tensors supply device memory and the
current HIP stream; every step of the operator runs in the HIP kernels. If
the library is not built the calls raise instead of falling back to anything.

Streams: the functions that take stream= allocate what they allocate (o,
h_final, the workspace) with that stream current, so torch's caching
allocator hands the memory on only in that stream's order. The classes
allocate on the stream current at construction; a caller that runs them on
another stream keeps the object alive until that stream's work is done.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch

LIB_PATH = Path(__file__).resolve().parent / "libkda.so"

KDA_OK, KDA_ERR_NULL, KDA_ERR_SHAPE, KDA_ERR_UNSUPPORTED = 0, 1, 2, 3
KDA_ERR_WORKSPACE, KDA_ERR_ALIAS, KDA_ERR_HIP, KDA_ERR_ALIGN, KDA_ERR_SCRATCH = 4, 5, 6, 7, 8
KDA_IO_F32, KDA_IO_BF16 = 0, 1
KDA_STATE_F32, KDA_STATE_BF16 = 0, 1
KDA_FLAG_QK_L2NORM = 1
KDA_FLAG_STATE_BF16 = 2
KDA_BAD_QKV, KDA_BAD_GATE, KDA_BAD_BETA, KDA_BAD_CU = 1, 2, 4, 8
CHUNK = 64
HEAD_DIM = 128

EXPORTS = ("kda_chunk_fwd_workspace_bytes", "kda_chunk_fwd_workspace_min_bytes",
           "kda_chunk_fwd", "kda_chunk_fwd_phase", "kda_chunk_fwd_noalloc", "kda_decode_step", "kda_recurrent_fwd", "kda_rmsnorm_gate",
           "kda_check_inputs", "kda_status_string", "kda_version")
# bytes of the fixed device array kda_chunk_fwd_noalloc uses as its workspace
NOALLOC_SCRATCH_BYTES = 128 << 20

_LIB = None


class KDAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """Loads libkda.so once; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m gated_delta_rule_50_amd.build` first")
        L = ctypes.CDLL(str(LIB_PATH))
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
        L.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                      ctypes.c_int, vp, vp]
        L.kda_decode_step.restype = ctypes.c_int
        L.kda_recurrent_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_uint32, vp, vp,
                                        vp]
        L.kda_recurrent_fwd.restype = ctypes.c_int
        L.kda_rmsnorm_gate.argtypes = [vp, vp, vp, ctypes.c_float, i64, i32, ctypes.c_int, vp,
                                       vp]
        L.kda_rmsnorm_gate.restype = ctypes.c_int
        L.kda_check_inputs.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                       ctypes.c_int, vp, vp]
        L.kda_check_inputs.restype = ctypes.c_int
        L.kda_status_string.argtypes = [ctypes.c_int]
        L.kda_status_string.restype = ctypes.c_char_p
        L.kda_version.restype = i32
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return lib().kda_status_string(int(status)).decode()


def _io(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return KDA_IO_BF16
    if dtype == torch.float32:
        return KDA_IO_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {dtype}")


def _state(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return KDA_STATE_BF16
    if dtype == torch.float32:
        return KDA_STATE_F32
    raise TypeError(f"states must be bfloat16 or float32, got {dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, dtype=None, device=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _shape(t, name, shape):
    """Raises ValueError unless t (when given) has exactly `shape`. Checked
    before anything else: the kernels index every buffer by T, H, N and the
    head size, so a mis-shaped tensor would be read or written past its end."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _head_rows(k, name="k"):
    """(rows, H) of a [rows, H, 128] tensor, or ValueError."""
    if k.dim() != 3 or k.shape[2] != HEAD_DIM:
        raise ValueError(f"{name} has shape {tuple(k.shape)}, expected [T, H, {HEAD_DIM}]")
    return int(k.shape[0]), int(k.shape[1])


def _stream(stream, device):
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def chunk_fwd_workspace_bytes(n_seqs: int, total_tokens: int, heads: int,
                              io_dtype: torch.dtype) -> int:
    return int(lib().kda_chunk_fwd_workspace_bytes(n_seqs, total_tokens, heads,
                                                   HEAD_DIM, HEAD_DIM, _io(io_dtype)))


def chunk_fwd_workspace_min_bytes(n_seqs: int, total_tokens: int, heads: int,
                                  io_dtype: torch.dtype) -> int:
    return int(lib().kda_chunk_fwd_workspace_min_bytes(n_seqs, total_tokens, heads,
                                                       HEAD_DIM, HEAD_DIM, _io(io_dtype)))


def alloc_workspace(n_seqs, total_tokens, heads, io_dtype, device, nbytes=None) -> torch.Tensor:
    """A 256-byte aligned uint8 device buffer of the recommended size (or
    nbytes: any size from chunk_fwd_workspace_min_bytes up works; a smaller
    workspace runs the prefill in more windows of chunk slots)."""
    if nbytes is None:
        nbytes = chunk_fwd_workspace_bytes(n_seqs, total_tokens, heads, io_dtype)
    if nbytes == 0:
        raise ValueError("invalid sizes for the prefill workspace")
    raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-raw.data_ptr()) % 256
    return raw[off:off + nbytes]


class Prefill:
    """Device buffers of one prefill call, marshalled once for repeated use.

    q, k [T, H, 128], v [T, H, 128] (bf16 or fp32, one dtype); log_alpha
    [T, H, 128] fp32; beta [T, H] fp32; h0 [N, H, 128, 128] in state_dtype
    (float32, or bfloat16: the serving format; the state is carried in fp32
    inside the call and rounded once into h_final) or None; cu_seqlens int32
    [N + 1] on the device or None (one sequence). h_final may be passed as h0
    to continue in place. qk_l2norm normalises q and k inside the kernel.
    """

    def __init__(self, q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, *, o=None,
                 h_final=None, want_final=True, workspace=None, qk_l2norm=False,
                 noalloc=False, state_dtype=torch.float32):
        dev = k.device
        self.T, self.H = _head_rows(k)
        if cu_seqlens is not None and cu_seqlens.dim() != 1:
            raise ValueError(f"cu_seqlens has shape {tuple(cu_seqlens.shape)}, expected [N + 1]")
        self.N = 1 if cu_seqlens is None else int(cu_seqlens.shape[0]) - 1
        T, H, N, D = self.T, self.H, self.N, HEAD_DIM
        for t, n in ((q, "q"), (v, "v"), (log_alpha, "log_alpha"), (o, "o")):
            _shape(t, n, (T, H, D))
        _shape(beta, "beta", (T, H))
        _shape(h0, "h0", (N, H, D, D))
        _shape(h_final, "h_final", (N, H, D, D))
        self.io = _io(k.dtype)
        for t, n in ((q, "q"), (k, "k"), (v, "v")):
            _check(t, n, k.dtype, dev)
        _check(log_alpha, "log_alpha", torch.float32, dev)
        _check(beta, "beta", torch.float32, dev)
        flags = (KDA_FLAG_QK_L2NORM if qk_l2norm else 0) | (
            KDA_FLAG_STATE_BF16 if _state(state_dtype) == KDA_STATE_BF16 else 0)
        _check(h0, "h0", state_dtype, dev)
        _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
        if o is None:
            o = torch.empty((self.T, self.H, v.shape[2]), dtype=k.dtype, device=dev)
        _check(o, "o", k.dtype, dev)
        if h_final is None and want_final:
            h_final = torch.empty((self.N, self.H, k.shape[2], v.shape[2]),
                                  dtype=state_dtype, device=dev)
        _check(h_final, "h_final", state_dtype, dev)
        if noalloc and workspace is not None:
            raise ValueError("noalloc calls take no workspace")
        if workspace is None and not noalloc:
            workspace = alloc_workspace(self.N, self.T, self.H, k.dtype, dev)
        _check(workspace, "workspace", torch.uint8, dev)
        self.device = dev
        self.noalloc = noalloc
        self.o, self.h_final, self.workspace = o, h_final, workspace
        self._keep = (q, k, v, log_alpha, beta, h0, cu_seqlens)
        self._args = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(h0),
                      _ptr(cu_seqlens), self.N, self.T, self.H, int(k.shape[2]),
                      int(v.shape[2]), self.io, flags, _ptr(o), _ptr(h_final))
        if not noalloc:
            self._args += (_ptr(workspace), workspace.numel())

    def run(self, stream=None):
        if self.noalloc:
            st = lib().kda_chunk_fwd_noalloc(*self._args, _stream(stream, self.device))
            if st != KDA_OK:
                raise KDAError(st, "kda_chunk_fwd_noalloc")
        else:
            st = lib().kda_chunk_fwd(*self._args, _stream(stream, self.device))
            if st != KDA_OK:
                raise KDAError(st, "kda_chunk_fwd")
        return self.o, self.h_final

    def run_phase(self, phase: int, stream=None):
        if self.noalloc:
            raise ValueError("the phase entry point takes a caller workspace")
        st = lib().kda_chunk_fwd_phase(int(phase), *self._args, _stream(stream, self.device))
        if st != KDA_OK:
            raise KDAError(st, f"kda_chunk_fwd_phase({phase})")


def chunk_fwd(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, *, o=None,
              h_final=None, want_final=True, workspace=None, qk_l2norm=False,
              state_dtype=torch.float32, stream=None):
    """Chunked prefill (see Prefill for shapes). Returns (o, h_final or None)."""
    with torch.cuda.stream(stream):
        return Prefill(q, k, v, log_alpha, beta, h0, cu_seqlens, o=o, h_final=h_final,
                       want_final=want_final, workspace=workspace, qk_l2norm=qk_l2norm,
                       state_dtype=state_dtype).run(stream)


def chunk_fwd_noalloc(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, *, o=None,
                      h_final=None, want_final=True, qk_l2norm=False,
                      state_dtype=torch.float32, stream=None):
    """chunk_fwd through kda_chunk_fwd_noalloc: the workspace is the
    library's fixed per-GPU array, so the call itself allocates nothing
    (pass o, and h_final or want_final=False, to allocate nothing here
    either). Calls overlapping on one GPU race on that array."""
    with torch.cuda.stream(stream):
        return Prefill(q, k, v, log_alpha, beta, h0, cu_seqlens, o=o, h_final=h_final,
                       want_final=want_final, qk_l2norm=qk_l2norm, noalloc=True,
                       state_dtype=state_dtype).run(stream)


class Decode:
    """Device buffers of one decode step (kda_decode_step), marshalled once.

    q, k, v [N, H, 128] (bf16 or fp32, one dtype); log_alpha [N, H, 128]
    fp32; beta [N, H] fp32; S [N, H, 128, 128] fp32, updated in place by
    every run. A serving loop that writes each new token into the same
    q/k/v/log_alpha/beta buffers binds them once and pays one library call
    per token in run(); the shape, dtype and device checks happen here.
    """

    def __init__(self, q, k, v, log_alpha, beta, S, *, o=None):
        dev = k.device
        N, H = _head_rows(k)
        for t, n in ((q, "q"), (v, "v"), (log_alpha, "log_alpha"), (o, "o")):
            _shape(t, n, (N, H, HEAD_DIM))
        _shape(beta, "beta", (N, H))
        _shape(S, "S", (N, H, HEAD_DIM, HEAD_DIM))
        io = _io(k.dtype)
        for t, n in ((q, "q"), (k, "k"), (v, "v")):
            _check(t, n, k.dtype, dev)
        _check(log_alpha, "log_alpha", torch.float32, dev)
        _check(beta, "beta", torch.float32, dev)
        _check(S, "S", torch.float32, dev)
        if o is None:
            o = torch.empty((N, H, v.shape[2]), dtype=k.dtype, device=dev)
        _check(o, "o", k.dtype, dev)
        self.device, self.o, self.S = dev, o, S
        self._keep = (q, k, v, log_alpha, beta)
        self._args = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S), N, H,
                      int(k.shape[2]), int(v.shape[2]), io, _ptr(o))
        self._fn = lib().kda_decode_step

    def run(self, stream=None):
        st = self._fn(*self._args, _stream(stream, self.device))
        if st != KDA_OK:
            raise KDAError(st, "kda_decode_step")
        return self.o


def decode_step(q, k, v, log_alpha, beta, S, *, o=None, stream=None):
    """One recurrent step; S [N, H, 128, 128] fp32 is updated in place.

    q, k, v [N, H, 128] (bf16 or fp32); log_alpha [N, H, 128] fp32;
    beta [N, H] fp32. Returns o [N, H, 128]. (Decode binds the buffers once
    for repeated steps.)
    """
    with torch.cuda.stream(stream):
        return Decode(q, k, v, log_alpha, beta, S, o=o).run(stream)


class Recurrent:
    """Device buffers of one fused recurrent call (kda_recurrent_fwd).

    Same tensors as Prefill, without a workspace. With cu_seqlens None the
    batch holds n_seqs sequences of T / n_seqs tokens each ([N, L, H, 128]
    flattened to [T, H, 128]). h0 / h_final are [N, H, 128, 128] in
    state_dtype (float32 or bfloat16); h_final may be h0 (in-place update).
    qk_l2norm normalises q and k inside the kernel.
    """

    def __init__(self, q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, *, n_seqs=None,
                 state_dtype=torch.float32, qk_l2norm=False, o=None, h_final=None,
                 want_final=True):
        dev = k.device
        self.T, self.H = _head_rows(k)
        if cu_seqlens is not None:
            if cu_seqlens.dim() != 1:
                raise ValueError(f"cu_seqlens has shape {tuple(cu_seqlens.shape)}, "
                                 "expected [N + 1]")
            self.N = int(cu_seqlens.shape[0]) - 1
        else:
            self.N = 1 if n_seqs is None else int(n_seqs)
        T, H, N, D = self.T, self.H, self.N, HEAD_DIM
        for t, n in ((q, "q"), (v, "v"), (log_alpha, "log_alpha"), (o, "o")):
            _shape(t, n, (T, H, D))
        _shape(beta, "beta", (T, H))
        _shape(h0, "h0", (N, H, D, D))
        _shape(h_final, "h_final", (N, H, D, D))
        self.io = _io(k.dtype)
        for t, n in ((q, "q"), (k, "k"), (v, "v")):
            _check(t, n, k.dtype, dev)
        _check(log_alpha, "log_alpha", torch.float32, dev)
        _check(beta, "beta", torch.float32, dev)
        _check(h0, "h0", state_dtype, dev)
        _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
        if o is None:
            o = torch.empty((self.T, self.H, v.shape[2]), dtype=k.dtype, device=dev)
        _check(o, "o", k.dtype, dev)
        if h_final is None and want_final:
            h_final = torch.empty((self.N, self.H, k.shape[2], v.shape[2]), dtype=state_dtype,
                                  device=dev)
        _check(h_final, "h_final", state_dtype, dev)
        self.device = dev
        self.o, self.h_final = o, h_final
        self._keep = (q, k, v, log_alpha, beta, h0, cu_seqlens)
        self._args = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(h0),
                      _ptr(cu_seqlens), self.N, self.T, self.H, int(k.shape[2]),
                      int(v.shape[2]), self.io, _state(state_dtype),
                      KDA_FLAG_QK_L2NORM if qk_l2norm else 0, _ptr(o), _ptr(h_final))

    def run(self, stream=None):
        st = lib().kda_recurrent_fwd(*self._args, _stream(stream, self.device))
        if st != KDA_OK:
            raise KDAError(st, "kda_recurrent_fwd")
        return self.o, self.h_final


def recurrent_fwd(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, *, n_seqs=None,
                  state_dtype=torch.float32, qk_l2norm=False, o=None, h_final=None,
                  want_final=True, stream=None):
    """Fused token-by-token forward (see Recurrent). Returns (o, h_final or None)."""
    with torch.cuda.stream(stream):
        return Recurrent(q, k, v, log_alpha, beta, h0, cu_seqlens, n_seqs=n_seqs,
                         state_dtype=state_dtype, qk_l2norm=qk_l2norm, o=o, h_final=h_final,
                         want_final=want_final).run(stream)


def rmsnorm_gate(o, gate, weight=None, eps=1e-6, *, y=None, stream=None):
    """Output epilogue y = sigmoid(gate) * RMSNorm(o) * weight per (token, head)
    row of 128 channels. o, gate [..., 128] in one I/O dtype; weight [128]
    float32 or None; y may be o (in place). Returns y."""
    dev = o.device
    if o.dim() < 1 or o.shape[-1] != HEAD_DIM:
        raise ValueError(f"o has shape {tuple(o.shape)}, expected [..., {HEAD_DIM}]")
    _shape(gate, "gate", o.shape)
    _shape(weight, "weight", (HEAD_DIM,))
    _shape(y, "y", o.shape)
    io = _io(o.dtype)
    _check(o, "o", None, dev)
    _check(gate, "gate", o.dtype, dev)
    _check(weight, "weight", torch.float32, dev)
    if y is None:
        with torch.cuda.stream(stream):
            y = torch.empty_like(o)
    _check(y, "y", o.dtype, dev)
    dv = int(o.shape[-1])
    rows = o.numel() // max(dv, 1)
    st = lib().kda_rmsnorm_gate(_ptr(o), _ptr(gate), _ptr(weight), float(eps), rows, dv, io,
                                _ptr(y), _stream(stream, dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_rmsnorm_gate")
    return y


def check_inputs(q, k, v, log_alpha, beta, cu_seqlens=None, *, flags=None, stream=None):
    """Debug check of the documented preconditions (finite q, k, v, beta;
    log_alpha finite and <= 0; cu_seqlens rising from 0 to T) on the device.
    Same tensors as chunk_fwd, or the decode step's ([N, H, 128] as T = N).
    With flags (a device int32 tensor of one element) the check is enqueued
    and flags receives the OR of the KDA_BAD_* bits; without, the bits are
    returned as an int (which waits for the stream)."""
    dev = k.device
    T, H = _head_rows(k)
    for t, n in ((q, "q"), (v, "v"), (log_alpha, "log_alpha")):
        _shape(t, n, (T, H, HEAD_DIM))
    _shape(beta, "beta", (T, H))
    if cu_seqlens is not None and cu_seqlens.dim() != 1:
        raise ValueError(f"cu_seqlens has shape {tuple(cu_seqlens.shape)}, expected [N + 1]")
    _shape(flags, "flags", (1,))
    _io(k.dtype)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, k.dtype, dev)
    _check(log_alpha, "log_alpha", torch.float32, dev)
    _check(beta, "beta", torch.float32, dev)
    _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
    with torch.cuda.stream(stream):   # out and its read-back on the check's stream
        out = torch.empty(1, dtype=torch.int32, device=dev) if flags is None else flags
        _check(out, "flags", torch.int32, dev)
        n = 0 if cu_seqlens is None else int(cu_seqlens.shape[0]) - 1
        st = lib().kda_check_inputs(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                    _ptr(cu_seqlens), n, T, H, int(k.shape[2]),
                                    int(v.shape[2]), _io(k.dtype), _ptr(out),
                                    _stream(stream, dev))
        if st != KDA_OK:
            raise KDAError(st, "kda_check_inputs")
        return out if flags is not None else int(out.item())


# Longest sequence routed to the recurrent kernel. The pages' serving notes
# switch at 64 new tokens; on MI355X (32 heads, fp32 states, whole calls) the
# chunked path with its short-sequence carry is faster from 40 tokens on for
# 64 and 256 sequences (L = 40: 177 against 186 us and 671 against 706 us)
# and from 32 on for 16 sequences, and the recurrent one up to 32 for 64 and
# 256 sequences (154 against 170 us, 597 against 639 us), so the switch sits
# at 32 for bf16 I/O. A single sequence (a single prompt) takes the chunked
# path's one-sequence launch, which skips the chunk map: there the recurrent
# kernel wins only up to about 20 tokens (32 heads: 16 tokens 17.2 against
# 19.6 us, 24 tokens 23.0 against 19.8, 32 tokens 28.8 against 19.9; 16
# heads alike), so one bf16 sequence switches at 16.
RECURRENT_MAX_LEN = 32
RECURRENT_MAX_LEN_ONE_SEQ = 16
# fp32 I/O: the chunked path's fp32 products run at a sixteenth of the bf16
# rate and it has no short-sequence carry, so with many (sequence, head)
# pairs the recurrent kernel stays faster much longer. Measured (32 heads,
# recurrent against chunked): 512 pairs, 16 x 512 tokens 703 against 728
# us (16 x 1024: 1320 against 1317); 2048 pairs, 64 x 1024 4223 against
# 4862; 8192 pairs, 256 x 512 7732 against 10461; 256 pairs, 8 x 64 70
# against 79 but 8 x 128 125 against 115; 128 pairs, 4 x 64 57 against 57;
# 32 pairs, 1 x 64 51 against 35.
RECURRENT_MAX_LEN_F32 = ((512, 512), (256, 64))   # (at least this many pairs, max length)


def recurrent_max_len(io_dtype: torch.dtype, n_seqs: int, heads: int) -> int:
    """Longest sequence that kda.forward sends to the recurrent kernel for a
    batch of n_seqs sequences of `heads` heads in this I/O dtype."""
    if io_dtype == torch.float32:
        for min_pairs, max_len in RECURRENT_MAX_LEN_F32:
            if n_seqs * heads >= min_pairs:
                return max_len
        return RECURRENT_MAX_LEN
    return RECURRENT_MAX_LEN_ONE_SEQ if n_seqs == 1 else RECURRENT_MAX_LEN


def forward(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, *, max_seqlen, n_seqs=None,
            qk_l2norm=False, o=None, h_final=None, state_dtype=torch.float32, stream=None):
    """Mode switch after the "L2 Deep Distill" page's serving notes: batches
    whose sequences have at most recurrent_max_len(...) new tokens (32 for
    bf16 I/O, 16 for one bf16 sequence; for fp32 I/O up to 512 with many
    (sequence, head) pairs) go
    through the fused recurrent kernel, longer ones through the chunked
    prefill. max_seqlen is the longest sequence in the batch (the caller
    knows it; cu_seqlens stays on the device). Same tensors as chunk_fwd,
    states in state_dtype (float32 or bfloat16) on both paths; with
    cu_seqlens None, n_seqs sequences of T / n_seqs tokens each. Returns
    (o, h_final)."""
    N = int(cu_seqlens.shape[0]) - 1 if cu_seqlens is not None else int(n_seqs or 1)
    if max_seqlen <= recurrent_max_len(k.dtype, N, int(k.shape[1])):
        return recurrent_fwd(q, k, v, log_alpha, beta, h0, cu_seqlens, n_seqs=n_seqs,
                             state_dtype=state_dtype, qk_l2norm=qk_l2norm, o=o,
                             h_final=h_final, stream=stream)
    if cu_seqlens is None and N != 1:
        # fixed-length batch: the chunked path takes its sequence offsets
        T = int(k.shape[0])
        if N < 1 or T % N != 0:
            raise ValueError(f"{T} tokens do not split into {N} sequences of equal length")
        with torch.cuda.stream(stream):
            cu_seqlens = torch.arange(N + 1, dtype=torch.int32, device=k.device) * (T // N)
    return chunk_fwd(q, k, v, log_alpha, beta, h0, cu_seqlens, o=o, h_final=h_final,
                     qk_l2norm=qk_l2norm, state_dtype=state_dtype, stream=stream)
