"""kda_chunk_fwd_noalloc (the prefill with its workspace in the library's
fixed per-GPU array) against kda_chunk_fwd with a caller workspace: the same
kernels, so the outputs and final states must be identical bit for bit, on
two calls in a row, the second smaller than the first (the array keeps the
first call's contents, which the second must not depend on)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gated_delta_rule_50_amd import kda, workloads  # noqa: E402
from tests.kda_testutil import dev  # noqa: E402

pytestmark = pytest.mark.gpu


def _inputs(lengths, H, seed, h0_std):
    p = workloads.make_prefill(lengths, H, seed=seed, io="bf16", h0_std=h0_std)
    bf = torch.bfloat16
    return p, (dev(p.q, bf), dev(p.k, bf), dev(p.v, bf), dev(p.log_alpha), dev(p.beta),
               None if p.h0 is None else dev(p.h0),
               dev(p.cu_seqlens, torch.int32) if len(lengths) > 1 else None)


def test_noalloc_matches_workspace_entry_point_twice():
    # first: a packed batch with initial states (chunk map path); second:
    # one shorter sequence with zero states (single-sequence path)
    cases = [([700, 1, 1300, 0, 129], 8, 501, 0.05), ([333], 4, 502, None)]
    assert kda.chunk_fwd_workspace_bytes(5, 2130, 8, torch.bfloat16) <= kda.NOALLOC_SCRATCH_BYTES
    for i, (lengths, H, seed, h0_std) in enumerate(cases):
        p, args = _inputs(lengths, H, seed, h0_std)
        print(f"noalloc call {i}: lengths {lengths}, H {H}", flush=True)
        o_ref, hf_ref = kda.chunk_fwd(*args)
        o = torch.empty_like(o_ref)
        hf = torch.empty_like(hf_ref)
        torch.cuda.synchronize()
        free_before = torch.cuda.mem_get_info()[0]
        kda.chunk_fwd_noalloc(*args, o=o, h_final=hf)
        torch.cuda.synchronize()
        if i > 0:
            # the array already exists: the second call changes no device memory use
            assert torch.cuda.mem_get_info()[0] == free_before
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), f"call {i}: o differs"
        assert torch.equal(hf.view(torch.int32), hf_ref.view(torch.int32)), f"call {i}: state"
        assert torch.isfinite(o.float()).all()


def test_noalloc_long_call_in_windows():
    """A call whose blocks exceed the array runs in windows sized to it: the
    8K x 32-head workload (330 MB of blocks in 128 MiB) equals the
    workspace entry point's one-window result bit for bit."""
    p, args = _inputs([8192], 32, 503, 0.02)
    assert kda.chunk_fwd_workspace_bytes(1, 8192, 32, torch.bfloat16) > kda.NOALLOC_SCRATCH_BYTES
    o_ref, hf_ref = kda.chunk_fwd(*args)
    o, hf = kda.chunk_fwd_noalloc(*args)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(hf.view(torch.int32), hf_ref.view(torch.int32))


def test_noalloc_rejects_a_call_beyond_the_array():
    """One chunk slot of 1024 heads needs more than the array: refused."""
    p, args = _inputs([64], 1024, 504, None)
    assert kda.chunk_fwd_workspace_min_bytes(1, 64, 1024, torch.bfloat16) > \
        kda.NOALLOC_SCRATCH_BYTES
    with pytest.raises(kda.KDAError) as e:
        kda.chunk_fwd_noalloc(*args)
    assert e.value.status == kda.KDA_ERR_SCRATCH
