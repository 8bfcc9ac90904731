"""Seeded synthetic workloads for the KDA forward operator.

This module only draws inputs: it holds none of the operator's arithmetic.
Both the HIP path (through the tests and the benchmark) and the fp64 oracle
consume what it produces.

Value distributions follow the pages' KDA heads ("Kimi Linear: An Expressive,
Efficient Attention Architecture", paper-graph-ui review, section "Neural
Parameterization"): 128-dim heads, L2-normalised q and k, beta = sigmoid(.),
alpha in (0, 1] per channel, supplied here as its natural log.

Recipe (numpy PCG64, ``default_rng(seed)``), in draw order:
  lengths (the seeded variable-length batch: integers uniform in [lo, hi],
  both ends included) -> q -> k -> v -> beta -> log_alpha -> h0.
  q, k  ~ N(0,1) float32, L2-normalised per (token, head) in fp64, then
        rounded to the I/O dtype (bf16: round-to-nearest-even). With
        qk="raw" the normalisation is skipped (inputs for the operator's
        in-kernel L2Norm); the draws are the same.
  v     ~ N(0,1) float32, rounded to the I/O dtype.
  beta  = sigmoid(z), z ~ N(0,1), float32.
  log_alpha = log(sigmoid(z)) / 16 = -softplus(-z)/16, z ~ N(0,1), computed
        in fp64, stored float32. "split" decay: channels [0, dk/2) use that
        draw; channels [dk/2, dk) draw uniform [-1.0, -0.25] (strong decay).
        "extreme" decay: as "split" with channels [dk/2, dk) uniform in
        [-4.0, -3.0], so a 16-token block's decay on those channels
        exceeds e^-44 (decays the chunk kernels evaluate per element).
  h0    ~ N(0, std^2) float32 when std is given, else zeros (None).
Large draws go in fixed row blocks, so results depend only on the seed.
The draws stay in one sequential stream per batch; the elementwise and
per-row arithmetic after them (normalisation, rounding, the log-sigmoid)
runs on row blocks in a thread pool, which gives the same values as one
thread.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

D = 128          # key / value head dimension of the pages' KDA heads
CHUNK = 64       # chunk length of the chunkwise algorithm
_BLOCK = 1 << 14  # rows per generation block


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 (ties to even), returned as float32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are exactly bf16."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _to_io(x: np.ndarray, io: str) -> np.ndarray:
    return round_bf16(x) if io == "bf16" else x.astype(np.float32)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _normal_f32(rng, shape, post=None):
    """N(0,1) float32 draws in row blocks of the first axis. post(blk), if
    given, transforms each drawn block in place on the thread pool while the
    next blocks are drawn."""
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(shape[0], int(np.prod(shape[1:], dtype=np.int64)))
    if post is None:
        for s in range(0, shape[0], _BLOCK):
            e = min(s + _BLOCK, shape[0])
            flat[s:e] = rng.standard_normal(flat[s:e].shape, dtype=np.float32)
        return out
    with ThreadPoolExecutor(max_workers=_workers()) as ex:
        pending = []
        for s in range(0, shape[0], _BLOCK):
            e = min(s + _BLOCK, shape[0])
            flat[s:e] = rng.standard_normal(flat[s:e].shape, dtype=np.float32)
            pending.append(ex.submit(post, out[s:e]))
            if len(pending) > 2 * _workers():
                pending.pop(0).result()
        for f in pending:
            f.result()
    return out


def _round_block(io):
    def rnd(blk):
        if io == "bf16":
            blk[...] = round_bf16(blk)
    return rnd


def _unit_rows(rng, shape, io, normalise=True):
    """N(0,1) rows normalised along the last axis in fp64, rounded to io."""
    if not normalise:
        return _normal_f32(rng, shape, _round_block(io))

    def norm(blk):
        x = blk.astype(np.float64)
        x /= np.linalg.norm(x, axis=-1, keepdims=True)
        blk[...] = _to_io(x.astype(np.float32), io)
    return _normal_f32(rng, shape, norm)


def _log_sigmoid_over_16(z64: np.ndarray) -> np.ndarray:
    # log(sigmoid(z)) = -softplus(-z) = -(max(-z,0) + log1p(exp(-|z|)))
    return (-(np.maximum(-z64, 0.0) + np.log1p(np.exp(-np.abs(z64)))) / 16.0)


def _log_alpha(rng, T, H, dk, decay):
    strong = {"split": (-1.0, -0.25), "extreme": (-4.0, -3.0)}
    if decay != "mild" and decay not in strong:
        raise ValueError(f"unknown decay recipe {decay!r}")
    la = np.empty((T, H, dk), dtype=np.float32)
    half = dk // 2
    nz = dk if decay == "mild" else half

    def fill(s, e, z):
        la[s:e, :, :nz] = _log_sigmoid_over_16(z).astype(np.float32)

    # the draws stay in order on this thread; each block's log-sigmoid runs
    # on the pool while the next block is drawn (a few blocks in flight)
    with ThreadPoolExecutor(max_workers=_workers()) as ex:
        pending = []
        for s in range(0, T, _BLOCK):
            e = min(s + _BLOCK, T)
            z = rng.standard_normal((e - s, H, nz))
            pending.append(ex.submit(fill, s, e, z))
            if decay in strong:
                lo, hi = strong[decay]
                la[s:e, :, half:] = rng.uniform(lo, hi, (e - s, H, dk - half)).astype(np.float32)
            if len(pending) > 2 * _workers():
                pending.pop(0).result()
        for f in pending:
            f.result()
    return la


@dataclass
class Prefill:
    """One packed prefill batch (numpy, host)."""
    q: np.ndarray            # [T, H, dk] float32 (bf16-exact when io == "bf16")
    k: np.ndarray            # [T, H, dk]
    v: np.ndarray            # [T, H, dv]
    log_alpha: np.ndarray    # [T, H, dk] float32
    beta: np.ndarray         # [T, H] float32
    h0: Optional[np.ndarray]  # [N, H, dk, dv] float32 or None
    cu_seqlens: np.ndarray   # [N+1] int32
    io: str                  # "bf16" or "f32"

    @property
    def T(self):
        return self.k.shape[0]

    @property
    def H(self):
        return self.k.shape[1]

    @property
    def N(self):
        return len(self.cu_seqlens) - 1


def _draw_lengths(rng, n, lo, hi):
    return tuple(int(x) for x in rng.integers(lo, hi, size=n, endpoint=True))


def make_prefill(lengths, H, seed, io="bf16", decay="mild", h0_std=None,
                 dk=D, dv=D, qk="unit", draw_lengths=None) -> Prefill:
    """Draws one packed batch with sequences of the given lengths. With
    draw_lengths = (n, lo, hi) the lengths are the stream's first draw
    (and must equal `lengths`, which varlen_lengths computes the same way)."""
    rng = np.random.default_rng(seed)
    if draw_lengths is not None:
        drawn = _draw_lengths(rng, *draw_lengths)
        if tuple(int(x) for x in lengths) != drawn:
            raise ValueError("lengths differ from the batch's seeded length draw")
    lengths = np.asarray(lengths, dtype=np.int64)
    T = int(lengths.sum())
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    unit = {"unit": True, "raw": False}[qk]
    q = _unit_rows(rng, (T, H, dk), io, unit)
    k = _unit_rows(rng, (T, H, dk), io, unit)
    v = _normal_f32(rng, (T, H, dv), _round_block(io))
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))).astype(np.float32)
    la = _log_alpha(rng, T, H, dk, decay)
    h0 = None
    if h0_std is not None:
        h0 = (_normal_f32(rng, (len(lengths), H, dk, dv)) * np.float32(h0_std)).astype(np.float32)
    return Prefill(q, k, v, la, beta, h0, cu, io)


@dataclass
class DecodeStep:
    """Inputs of one decode step: one token for each of N sequences."""
    q: np.ndarray          # [N, H, dk]
    k: np.ndarray          # [N, H, dk]
    v: np.ndarray          # [N, H, dv]
    log_alpha: np.ndarray  # [N, H, dk]
    beta: np.ndarray       # [N, H]
    io: str


def make_decode_state(N, H, seed, std=0.02, dk=D, dv=D) -> np.ndarray:
    """Initial decode states S0 [N, H, dk, dv] ~ N(0, std^2), float32."""
    rng = np.random.default_rng(seed)
    return (_normal_f32(rng, (N, H, dk, dv)) * np.float32(std)).astype(np.float32)


def make_decode_step(N, H, seed, step, io="bf16", dk=D, dv=D, qk="unit") -> DecodeStep:
    """Fresh token inputs for decode step ``step`` (rng seeded [seed, step])."""
    rng = np.random.default_rng([seed, step])
    unit = {"unit": True, "raw": False}[qk]
    q = _unit_rows(rng, (N, H, dk), io, unit)
    k = _unit_rows(rng, (N, H, dk), io, unit)
    v = _to_io(_normal_f32(rng, (N, H, dv)), io)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((N, H))))).astype(np.float32)
    la = _log_alpha(rng, N, H, dk, "mild")
    return DecodeStep(q, k, v, la, beta, io)


@dataclass
class Epilogue:
    """Inputs of the output epilogue for `rows` (token, head) rows."""
    o: np.ndarray        # [rows, dv] operator output stand-in, I/O dtype values
    gate: np.ndarray     # [rows, dv] sigmoid-gate pre-activation, I/O dtype values
    weight: np.ndarray   # [dv] float32 RMSNorm weight
    io: str


def make_epilogue(rows, seed, io="bf16", dv=D, o_std=0.3) -> Epilogue:
    """o ~ N(0, o_std^2) (the operator's outputs on the workloads above have
    this order of magnitude), gate ~ N(0, 1), weight = 1 + 0.1 N(0, 1):
    draws in that order, o and gate rounded to the I/O dtype."""
    rng = np.random.default_rng(seed)
    o = _to_io(_normal_f32(rng, (rows, dv)) * np.float32(o_std), io)
    gate = _to_io(_normal_f32(rng, (rows, dv)), io)
    weight = (1.0 + 0.1 * rng.standard_normal(dv)).astype(np.float32)
    return Epilogue(o, gate, weight, io)


@dataclass
class Config:
    """One of the five benchmark/parity configurations."""
    cid: int
    name: str
    kind: str                      # "prefill" or "decode"
    H: int
    io: str
    seed: int
    lengths: tuple = ()
    decay: str = "mild"
    h0_std: Optional[float] = None
    n_seqs: int = 1
    steps: int = 0
    extra: dict = field(default_factory=dict)

    def prefill(self) -> Prefill:
        assert self.kind == "prefill"
        return make_prefill(self.lengths, self.H, self.seed, self.io,
                            self.decay, self.h0_std,
                            draw_lengths=self.extra.get("draw_lengths"))


def varlen_lengths(seed, n, lo, hi):
    """The lengths a batch seeded `seed` draws first (make_prefill's
    draw_lengths)."""
    return _draw_lengths(np.random.default_rng(seed), n, lo, hi)


def config(cid: int) -> Config:
    """The five workloads: 0 tiny fp32, 1 8K prefill, 2 128K strong-decay
    prefill, 3 packed variable-length prefill, 4 decode 256 x 32 heads."""
    seed = 1000 + cid
    if cid == 0:
        return Config(0, "tiny_fp32_T512_H2", "prefill", H=2, io="f32",
                      seed=seed, lengths=(512,))
    if cid == 1:
        return Config(1, "prefill_T8192_H32_bf16", "prefill", H=32, io="bf16",
                      seed=seed, lengths=(8192,))
    if cid == 2:
        return Config(2, "prefill_T131072_H32_bf16_strong_decay", "prefill",
                      H=32, io="bf16", seed=seed, lengths=(131072,),
                      decay="split", h0_std=0.02)
    if cid == 3:
        # the lengths are the batch stream's first draw, then q, k, v, ...
        spec = (16, 512, 16384)
        return Config(3, "varlen_16seq_H32_bf16", "prefill", H=32, io="bf16",
                      seed=seed, lengths=varlen_lengths(seed, *spec), h0_std=0.02,
                      n_seqs=16, extra={"draw_lengths": spec})
    if cid == 4:
        return Config(4, "decode_N256_H32_bf16_64steps", "decode", H=32,
                      io="bf16", seed=seed, n_seqs=256, steps=64)
    raise ValueError(cid)
