"""MI355X-native Kimi Delta Attention forward operator.

``kda`` binds the C ABI of libkda.so (HIP kernels for gfx950);
``workloads`` draws the seeded synthetic inputs.
"""
from .kda import (KDAError, Prefill, Recurrent, alloc_workspace, check_inputs,  # noqa: F401
                  chunk_fwd, chunk_fwd_noalloc, chunk_fwd_workspace_bytes,
                  chunk_fwd_workspace_min_bytes, Decode, decode_step,
                  forward, lib, recurrent_fwd, rmsnorm_gate)
