"""Helpers shared by the GPU tests: host arrays to device tensors and the
error measures the tolerances are stated in."""
import numpy as np
import torch


def dev(x, dtype=torch.float32):
    """numpy -> contiguous device tensor (bf16-exact float32 values convert
    exactly to bf16)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dtype)


def io_dtype(io):
    return torch.bfloat16 if io == "bf16" else torch.float32


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_max_err(got, ref):
    """max |got - ref| / max |ref| (the operator's output tolerance measure)."""
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def rel_fro_err(got, ref):
    return float(np.linalg.norm((got - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-30))


def rel_fro_err_dev(got, ref):
    """rel_fro_err of a device tensor against a host fp64 array, evaluated
    in fp64 on the device (large states: the measure, not the operator)."""
    r = torch.from_numpy(np.ascontiguousarray(ref, dtype=np.float64)).to(got.device)
    num = torch.linalg.vector_norm(got.double() - r).item()
    den = torch.linalg.vector_norm(r).item()
    return float(num / max(den, 1e-30))


# Tolerances: output max-abs error relative to max|o|; state relative
# Frobenius error. fp32 I/O: 1e-4 on o and (unstated on the pages, chosen
# here) 1e-4 on the state; bf16 I/O: 2e-2 on o, 1e-2 on the state.
TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 1e-2)}


# --------------------------------------------------------------- workspace
# Decoder of the per-(chunk, head) blocks the prefill leaves in its workspace
# (layout documented in include/kda.h). Test-side only.
def _split_k(g, e):
    return 4 * g + e if e < 4 else 16 + 4 * g + (e - 4)


def _lane_maps():
    L = np.arange(64)
    r, g = L % 16, L // 16
    return r, g


def decode_block(ws_bytes, b, h, H, N, io):
    """Returns dict(W, Qt, Kp, U, Ut, gC) (float64) of chunk b, head h (the
    workspace of a call whose window held every chunk)."""
    esz = 2 if io == "bf16" else 4
    block = 40960 * esz + 128 * 4
    inter = 256 + (4 * (N + 1) + 255) // 256 * 256 + 2 * H * 128 * 128 * 4
    base = inter + (b * H + h) * block
    raw = np.frombuffer(ws_bytes, dtype=np.uint8, count=block, offset=base)
    if io == "bf16":
        el = (raw[:40960 * 2].view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    else:
        el = raw[:40960 * 4].view(np.float32)
    el = el.astype(np.float64)
    gC = raw[40960 * esz:].view(np.float32).astype(np.float64)
    r, g = _lane_maps()
    X = np.zeros((128, 128))
    for mt in range(8):
        for kb in range(4):
            frag = el[((mt * 4 + kb) * 64) * 8:((mt * 4 + kb) * 64 + 64) * 8].reshape(64, 8)
            for e in range(8):
                X[16 * mt + r, 32 * kb + np.array([_split_k(gg, e) for gg in g])] = frag[:, e]
    KT = np.zeros((128, 64))
    off = 16384
    for mt in range(8):
        for kb in range(2):
            frag = el[off + ((mt * 2 + kb) * 64) * 8:off + ((mt * 2 + kb) * 64 + 64) * 8].reshape(64, 8)
            for e in range(8):
                KT[16 * mt + r, 32 * kb + np.array([_split_k(gg, e) for gg in g])] = frag[:, e]
    U = np.zeros((64, 128))
    Ut = np.zeros((64, 128))
    off = 16384 + 8192
    for jt in range(8):
        for mt in range(8):
            frag = el[off + ((jt * 8 + mt) * 64) * 4:off + ((jt * 8 + mt) * 64 + 64) * 4].reshape(64, 4)
            for e in range(4):
                if mt < 4:
                    U[16 * mt + 4 * g + e, 16 * jt + r] = frag[:, e]
                else:
                    Ut[16 * (mt - 4) + r, 16 * jt + 4 * g + e] = frag[:, e]
    return dict(W=-X[:64], Qt=X[64:], Kp=KT.T, U=U, Ut=Ut, gC=gC)
