"""The attention call on two caller streams at once, and inside a captured graph.

A call forks its block scores and walk schedule to a side stream that the
library owns and joins them back with event edges before the attention
kernel.  Calls running on two streams at once, and a captured HIP graph
replayed several times with other work between the replays, must give the
same output bits as plain calls on one stream (every kernel is
deterministic).
"""
import numpy as np
import pytest

from sparse_linear_attention_sagesla_amd.inputs import random_bf16

from gpu_util import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sla = pytest.importorskip("sparse_linear_attention_sagesla_amd")

SHAPE = (1, 3, 64 * 40 - 23, 128)  # 40 blocks, ragged last block


def _inputs(seed):
    return tuple(to_dev(random_bf16(SHAPE, seed + t)) for t in range(3))


def test_two_streams_at_once():
    a, b = _inputs(11), _inputs(21)
    ref_a = sla.attention(*a, 0.1, "elu1", torch.float32)
    ref_b = sla.attention(*b, 0.15, "relu", torch.float32)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s1):
            out_a = sla.attention(*a, 0.1, "elu1", torch.float32)
        with torch.cuda.stream(s2):
            out_b = sla.attention(*b, 0.15, "relu", torch.float32)
        torch.cuda.synchronize()
        print(f"[streams] rep {rep}", flush=True)
        assert torch.equal(out_a, ref_a), f"stream 1, repetition {rep}"
        assert torch.equal(out_b, ref_b), f"stream 2, repetition {rep}"


@pytest.mark.parametrize("keep,phi", [(0.1, "elu1"), (0.6, "elu1"), (0.1, "none")])
def test_graph_capture_replays(keep, phi):
    q, k, v = _inputs(31)
    att = sla.SLAAttention(*SHAPE[:3], keep=keep, phi=phi, out_dtype=torch.float32)
    eager = att(q, k, v).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        att(q, k, v)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = att(q, k, v)
    for rep in range(3):
        att.out.fill_(7.0)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print(f"[graph] keep {keep} phi {phi} replay {rep}", flush=True)
        assert torch.equal(out, eager), f"replay {rep}"
