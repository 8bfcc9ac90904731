"""Thin Python binding of libkda.so (the C ABI in include/kda.h).

Argument marshalling only: torch tensors supply device memory and the
current HIP stream; every step of the operator runs in the HIP kernels. If
the library is not built the calls raise instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch

LIB_PATH = Path(__file__).resolve().parent / "libkda.so"

KDA_OK, KDA_ERR_NULL, KDA_ERR_SHAPE, KDA_ERR_UNSUPPORTED = 0, 1, 2, 3
KDA_ERR_WORKSPACE, KDA_ERR_ALIAS, KDA_ERR_HIP, KDA_ERR_ALIGN = 4, 5, 6, 7
KDA_IO_F32, KDA_IO_BF16 = 0, 1
KDA_STATE_F32, KDA_STATE_BF16 = 0, 1
KDA_FLAG_QK_L2NORM = 1
KDA_BAD_QKV, KDA_BAD_GATE, KDA_BAD_BETA, KDA_BAD_CU = 1, 2, 4, 8
CHUNK = 64
HEAD_DIM = 128

EXPORTS = ("kda_chunk_fwd_workspace_bytes", "kda_chunk_fwd", "kda_chunk_fwd_phase",
           "kda_decode_step", "kda_recurrent_fwd", "kda_rmsnorm_gate", "kda_check_inputs",
           "kda_status_string", "kda_version")

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
        L.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                    ctypes.c_int, ctypes.c_uint32, vp, vp, vp, sz, vp]
        L.kda_chunk_fwd.restype = ctypes.c_int
        L.kda_chunk_fwd_phase.argtypes = [i32] + L.kda_chunk_fwd.argtypes
        L.kda_chunk_fwd_phase.restype = ctypes.c_int
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


def _stream(stream, device):
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def chunk_fwd_workspace_bytes(n_seqs: int, total_tokens: int, heads: int,
                              io_dtype: torch.dtype) -> int:
    return int(lib().kda_chunk_fwd_workspace_bytes(n_seqs, total_tokens, heads,
                                                   HEAD_DIM, HEAD_DIM, _io(io_dtype)))


def alloc_workspace(n_seqs, total_tokens, heads, io_dtype, device) -> torch.Tensor:
    """A 256-byte aligned uint8 device buffer of the required size."""
    nbytes = chunk_fwd_workspace_bytes(n_seqs, total_tokens, heads, io_dtype)
    if nbytes == 0:
        raise ValueError("invalid sizes for the prefill workspace")
    raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-raw.data_ptr()) % 256
    return raw[off:off + nbytes]


class Prefill:
    """Device buffers of one prefill call, marshalled once for repeated use.

    q, k [T, H, 128], v [T, H, 128] (bf16 or fp32, one dtype); log_alpha
    [T, H, 128] fp32; beta [T, H] fp32; h0 [N, H, 128, 128] fp32 or None;
    cu_seqlens int32 [N + 1] on the device or None (one sequence). h_final
    may be passed as h0 to continue in place. qk_l2norm normalises q and k
    inside the kernel.
    """

    def __init__(self, q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, *, o=None,
                 h_final=None, want_final=True, workspace=None, qk_l2norm=False):
        dev = k.device
        self.io = _io(k.dtype)
        self.T, self.H = int(k.shape[0]), int(k.shape[1])
        self.N = 1 if cu_seqlens is None else int(cu_seqlens.shape[0]) - 1
        for t, n in ((q, "q"), (k, "k"), (v, "v")):
            _check(t, n, k.dtype, dev)
        _check(log_alpha, "log_alpha", torch.float32, dev)
        _check(beta, "beta", torch.float32, dev)
        _check(h0, "h0", torch.float32, dev)
        _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
        if o is None:
            o = torch.empty((self.T, self.H, v.shape[2]), dtype=k.dtype, device=dev)
        _check(o, "o", k.dtype, dev)
        if h_final is None and want_final:
            h_final = torch.empty((self.N, self.H, k.shape[2], v.shape[2]),
                                  dtype=torch.float32, device=dev)
        _check(h_final, "h_final", torch.float32, dev)
        if workspace is None:
            workspace = alloc_workspace(self.N, self.T, self.H, k.dtype, dev)
        _check(workspace, "workspace", torch.uint8, dev)
        self.device = dev
        self.o, self.h_final, self.workspace = o, h_final, workspace
        self._keep = (q, k, v, log_alpha, beta, h0, cu_seqlens)
        self._args = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(h0),
                      _ptr(cu_seqlens), self.N, self.T, self.H, int(k.shape[2]),
                      int(v.shape[2]), self.io, KDA_FLAG_QK_L2NORM if qk_l2norm else 0,
                      _ptr(o), _ptr(h_final), _ptr(workspace), workspace.numel())

    def run(self, stream=None):
        st = lib().kda_chunk_fwd(*self._args, _stream(stream, self.device))
        if st != KDA_OK:
            raise KDAError(st, "kda_chunk_fwd")
        return self.o, self.h_final

    def run_phase(self, phase: int, stream=None):
        st = lib().kda_chunk_fwd_phase(int(phase), *self._args, _stream(stream, self.device))
        if st != KDA_OK:
            raise KDAError(st, f"kda_chunk_fwd_phase({phase})")


def chunk_fwd(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, *, o=None,
              h_final=None, want_final=True, workspace=None, qk_l2norm=False, stream=None):
    """Chunked prefill (see Prefill for shapes). Returns (o, h_final or None)."""
    return Prefill(q, k, v, log_alpha, beta, h0, cu_seqlens, o=o, h_final=h_final,
                   want_final=want_final, workspace=workspace,
                   qk_l2norm=qk_l2norm).run(stream)


def decode_step(q, k, v, log_alpha, beta, S, *, o=None, stream=None):
    """One recurrent step; S [N, H, 128, 128] fp32 is updated in place.

    q, k, v [N, H, 128] (bf16 or fp32); log_alpha [N, H, 128] fp32;
    beta [N, H] fp32. Returns o [N, H, 128].
    """
    dev = k.device
    io = _io(k.dtype)
    N, H = int(k.shape[0]), int(k.shape[1])
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, k.dtype, dev)
    _check(log_alpha, "log_alpha", torch.float32, dev)
    _check(beta, "beta", torch.float32, dev)
    _check(S, "S", torch.float32, dev)
    if o is None:
        o = torch.empty((N, H, v.shape[2]), dtype=k.dtype, device=dev)
    _check(o, "o", k.dtype, dev)
    st = lib().kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                               _ptr(S), N, H, int(k.shape[2]), int(v.shape[2]), io,
                               _ptr(o), _stream(stream, dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_decode_step")
    return o


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
        self.io = _io(k.dtype)
        self.T, self.H = int(k.shape[0]), int(k.shape[1])
        if cu_seqlens is not None:
            self.N = int(cu_seqlens.shape[0]) - 1
        else:
            self.N = 1 if n_seqs is None else int(n_seqs)
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
    return Recurrent(q, k, v, log_alpha, beta, h0, cu_seqlens, n_seqs=n_seqs,
                     state_dtype=state_dtype, qk_l2norm=qk_l2norm, o=o, h_final=h_final,
                     want_final=want_final).run(stream)


def rmsnorm_gate(o, gate, weight=None, eps=1e-6, *, y=None, stream=None):
    """Output epilogue y = sigmoid(gate) * RMSNorm(o) * weight per (token, head)
    row of 128 channels. o, gate [..., 128] in one I/O dtype; weight [128]
    float32 or None; y may be o (in place). Returns y."""
    dev = o.device
    io = _io(o.dtype)
    _check(o, "o", None, dev)
    _check(gate, "gate", o.dtype, dev)
    _check(weight, "weight", torch.float32, dev)
    if gate.shape != o.shape:
        raise ValueError(f"gate shape {tuple(gate.shape)} != o shape {tuple(o.shape)}")
    if y is None:
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
    _io(k.dtype)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, k.dtype, dev)
    _check(log_alpha, "log_alpha", torch.float32, dev)
    _check(beta, "beta", torch.float32, dev)
    _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
    out = torch.empty(1, dtype=torch.int32, device=dev) if flags is None else flags
    _check(out, "flags", torch.int32, dev)
    T, H = int(k.shape[0]), int(k.shape[1])
    n = 0 if cu_seqlens is None else int(cu_seqlens.shape[0]) - 1
    st = lib().kda_check_inputs(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                _ptr(cu_seqlens), n, T, H, int(k.shape[2]), int(v.shape[2]),
                                _io(k.dtype), _ptr(out), _stream(stream, dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_check_inputs")
    return out if flags is not None else int(out.item())


# Longest sequence routed to the recurrent kernel. The pages' serving notes
# switch at 64 new tokens; on MI355X the two paths cost the same at 48 (256
# or 64 sequences x 32 heads, fp32 states) and the chunked one is 12-23 %
# faster from 56 to 64, so the switch sits at the measured crossover.
RECURRENT_MAX_LEN = 48


def forward(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, *, max_seqlen, n_seqs=None,
            qk_l2norm=False, o=None, h_final=None, stream=None):
    """Mode switch after the "L2 Deep Distill" page's serving notes: batches
    whose sequences have at most RECURRENT_MAX_LEN new tokens go through the
    fused recurrent kernel, longer ones through the chunked prefill. max_seqlen is the longest sequence in the batch (the
    caller knows it; cu_seqlens stays on the device). Same tensors as
    chunk_fwd (fp32 states). Returns (o, h_final)."""
    if max_seqlen <= RECURRENT_MAX_LEN:
        return recurrent_fwd(q, k, v, log_alpha, beta, h0, cu_seqlens, n_seqs=n_seqs,
                             qk_l2norm=qk_l2norm, o=o, h_final=h_final, stream=stream)
    if cu_seqlens is None and (n_seqs or 1) != 1:
        raise ValueError("the chunked path needs cu_seqlens for more than one sequence")
    return chunk_fwd(q, k, v, log_alpha, beta, h0, cu_seqlens, o=o, h_final=h_final,
                     qk_l2norm=qk_l2norm, stream=stream)
