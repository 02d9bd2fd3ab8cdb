"""sla_attention_fwd_noalloc: the forward with the library's static device
scratch as workspace, for callers that cannot allocate.  Its output must be
bit-identical to sla_attention_fwd's (the same kernels on the same inputs),
on two calls in a row, the second on a smaller input (the scratch keeps the
first call's contents)."""
import ctypes

import numpy as np
import pytest

from sparse_linear_attention_sagesla_amd.inputs import make_inputs, random_bf16

from gpu_util import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sla = pytest.importorskip("sparse_linear_attention_sagesla_amd")
from sparse_linear_attention_sagesla_amd import _lib  # noqa: E402


def _noalloc(q, k, v, keep, phi, out):
    B, H, N, d = q.shape
    rc = _lib.load().sla_attention_fwd_noalloc(
        _lib._ptr(q), _lib._ptr(k), _lib._ptr(v), B, H, N, d, 64, float(keep), _lib.PHI[phi],
        _lib._ptr(out), 1 if out.dtype == torch.float32 else 0,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return rc


def test_noalloc_matches_the_workspace_entry_point_twice():
    Q, K, V = make_inputs("tiny")
    cases = [((Q, K, V), 0.1, "elu1"),                                    # 6.3 MiB of scratch
             (tuple(random_bf16((1, 1, 1000, 128), 70 + t) for t in range(3)), 0.3, "relu")]
    for n, ((q_, k_, v_), keep, phi) in enumerate(cases):
        q, k, v = to_dev(q_), to_dev(k_), to_dev(v_)
        print(f"[noalloc] call {n} shape={tuple(q.shape)} keep={keep} {phi}", flush=True)
        for dtype in (torch.float32, torch.bfloat16):
            ref = sla.attention(q, k, v, keep, phi, dtype)
            out = torch.full_like(ref, 3.0)
            torch.cuda.synchronize()
            assert _noalloc(q, k, v, keep, phi, out) == _lib.SLA_OK
            torch.cuda.synchronize()
            assert torch.equal(out, ref), f"call {n} {dtype}"
            assert torch.isfinite(out.float()).all()


def test_noalloc_rejects_shapes_beyond_the_scratch():
    q = torch.empty(1, 40, 75600, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    assert sla.workspace_bytes(1, 40, 75600, 0.1, "elu1") > _lib.NOALLOC_SCRATCH_BYTES
    assert _noalloc(q, q, q, 0.1, "elu1", out) == _lib.SLA_ERR_SCRATCH
