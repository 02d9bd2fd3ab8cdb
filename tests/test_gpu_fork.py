"""sla_attention_fwd_fork: the forward with the selection on a second stream.

It runs the same kernels on the same data as sla_attention_fwd, only on two
streams with a fork after the statistics pass and a join before the attention
kernel, so its output must equal sla_attention_fwd's bit for bit, in both
output types and in every form of the linear branch (subtraction, direct,
pure linear, none)."""
import pytest

from sparse_linear_attention_sagesla_amd.inputs import random_bf16

from gpu_util import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sla = pytest.importorskip("sparse_linear_attention_sagesla_amd")


@pytest.mark.parametrize("keep,phi", [(0.1, "elu1"), (0.3, "relu"), (0.6, "elu1"), (0.0, "elu1"),
                                      (1.0, "elu1"), (0.3, "none")])
def test_fork_equals_single_stream(keep, phi):
    N = 64 * 21 - 13
    Q, K, V = (random_bf16((2, 3, N, 128), s) for s in (301, 302, 303))
    q, k, v = (to_dev(x) for x in (Q, K, V))
    print(f"[case] fork N={N} keep={keep} phi={phi}", flush=True)
    side = torch.cuda.Stream()
    for dtype in (torch.float32, torch.bfloat16):
        ref = sla.attention(q, k, v, keep, phi, dtype)
        got = sla.attention(q, k, v, keep, phi, dtype, side_stream=side)
        torch.cuda.synchronize()
        assert torch.equal(ref, got), f"{dtype}"


def test_fork_repeated_calls_keep_their_order():
    # back-to-back forked calls on changing inputs: each result equals the
    # single-stream one for its own inputs (the join orders every call's
    # selection before its attention kernel and after the previous call's)
    N = 64 * 12 - 5
    side = torch.cuda.Stream()
    outs, refs = [], []
    for s in range(3):
        q, k, v = (to_dev(random_bf16((1, 2, N, 128), 310 + 3 * s + t)) for t in range(3))
        outs.append(sla.attention(q, k, v, 0.25, "elu1", torch.float32, side_stream=side))
        refs.append(sla.attention(q, k, v, 0.25, "elu1", torch.float32))
    torch.cuda.synchronize()
    for a, b in zip(outs, refs):
        assert torch.equal(a, b)
