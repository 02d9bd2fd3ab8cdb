"""The attention call on two caller streams at once, and inside a captured graph.

A call enqueues all its work on the caller's stream and the library keeps no
state between calls.  Calls running on two streams at once, and a captured
HIP graph replayed several times with other work between the replays, must
give the same output bits as plain calls on one stream (every kernel is
deterministic); so must a graph captured around the very first call a fresh
process makes.
"""
import os
import subprocess
import sys
import textwrap

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


def test_fork_inside_graph_capture():
    """sla_attention_fwd_fork captured: the fork and join become graph
    dependencies between the selection and the staging branches."""
    q, k, v = _inputs(51)
    keep, phi = 0.1, "elu1"
    eager = sla.attention(q, k, v, keep, phi, torch.float32).clone()
    out = torch.empty(SHAPE, dtype=torch.float32, device=q.device)
    ws = torch.empty(sla.workspace_bytes(*SHAPE[:3], keep, phi), dtype=torch.uint8, device=q.device)
    side = torch.cuda.Stream()
    sla.attention(q, k, v, keep, phi, torch.float32, out=out, workspace=ws, side_stream=side)
    torch.cuda.synchronize()
    assert torch.equal(out, eager)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sla.attention(q, k, v, keep, phi, torch.float32, out=out, workspace=ws, side_stream=side)
    for rep in range(3):
        out.fill_(7.0)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print(f"[graph] fork replay {rep}", flush=True)
        assert torch.equal(out, eager), f"replay {rep}"


FIRST_CALL_IN_CAPTURE = textwrap.dedent("""
    import sys
    sys.path.insert(0, sys.argv[1])
    import torch
    import sparse_linear_attention_sagesla_amd as sla
    from sparse_linear_attention_sagesla_amd.inputs import random_bf16
    shape = (1, 3, 64 * 40 - 23, 128)
    q, k, v = (torch.from_numpy(random_bf16(shape, 41 + t).view("int16")).view(torch.bfloat16).cuda()
               for t in range(3))
    att = sla.SLAAttention(*shape[:3], keep=0.1, phi="elu1", out_dtype=torch.float32)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):      # the process's first library call
        out = att(q, k, v)
    outs = []
    for rep in range(3):
        att.out.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        outs.append(out.clone())
    eager = sla.attention(q, k, v, 0.1, "elu1", torch.float32)
    torch.cuda.synchronize()
    assert all(torch.equal(o, eager) for o in outs), "replay differs from the eager call"
    print("first call captured: ok", flush=True)
""")


def test_first_call_of_a_process_inside_graph_capture():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    print("[graph] fresh process, first call captured", flush=True)
    res = subprocess.run([sys.executable, "-c", FIRST_CALL_IN_CAPTURE, root], capture_output=True,
                         text=True, timeout=240)
    print(res.stdout[-2000:], res.stderr[-2000:], flush=True)
    assert res.returncode == 0 and "first call captured: ok" in res.stdout
