"""Oracle work units that the full-size GPU tests run in worker processes.

Test infrastructure: each job regenerates its head's inputs from the seeded
generator (bit-identical in any process) and runs the fp64 oracle on it, so
only small results cross the process boundary.
"""
import numpy as np

from oracle import sla_oracle as O
from sparse_linear_attention_sagesla_amd.inputs import WORKLOADS, make_dout, make_head


def sampled_blocks(job):
    """(h, oracle result on the listed query blocks of head h)."""
    name, h, keep, phi, blocks = job
    q, k, v = make_head(WORKLOADS[name], 0, h)
    r = O.sla_forward_head(q, k, v, 64, keep, phi, query_blocks=blocks)
    return h, {"out": r["out"], "out_linear": r["out_linear"], "rows": r["rows"]}


def selection_against(job):
    """The oracle's selection of head h against the GPU's: (h, rows that
    differ, differences within 1e-6 of the row's largest |score| of the k-th
    score, other differences, identical)."""
    name, h, keep, gpu_idx = job
    q, k, _ = make_head(WORKLOADS[name], 0, h)
    idx, sc = O.select_head(q, k, 64, keep)
    kk = idx.shape[1]
    rows = excused = bad = 0
    for i in range(idx.shape[0]):
        a, b = set(gpu_idx[i].tolist()), set(idx[i].tolist())
        if a == b:
            continue
        rows += 1
        kth = np.sort(sc[i])[::-1][kk - 1]
        tol = 1e-6 * np.abs(sc[i]).max()
        for j in a ^ b:
            if abs(sc[i, j] - kth) <= tol:
                excused += 1
            else:
                bad += 1
    return h, rows, excused, bad, bool(np.array_equal(gpu_idx, idx))


def codes(job):
    """(h, q8, k8, q_scale, k_scale, mu) of head h from the oracle's quantiser."""
    name, h = job
    q, k, _ = make_head(WORKLOADS[name], 0, h)
    return (h,) + tuple(O.quantize_qk(q, k, 64))


def backward_key_share(job):
    """The oracle backward of head h restricted to the listed query blocks:
    (dK rows, dV rows) of the listed key blocks, the share those query
    blocks contribute (with phi = none, the query blocks that keep a key block
    are the only ones that touch its rows)."""
    name, h, keep, phi, key_blocks, query_blocks = job
    wl = WORKLOADS[name]
    q, k, v = make_head(wl, 0, h)
    g = make_dout(wl, heads=[h])[0, 0]
    r = O.sla_backward_head(q, k, v, g, 64, keep, phi, query_blocks=query_blocks)
    rows = np.concatenate([np.arange(j * 64, min(wl.N, (j + 1) * 64)) for j in key_blocks])
    return r["dk"][rows], r["dv"][rows]
