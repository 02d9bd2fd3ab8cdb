"""Helpers shared by the GPU tests: device transfer, the parity criteria and
the pool of oracle worker processes."""
import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np

ATOL = 2e-3       # max-abs tolerance on the fp32 output
REL_L2 = 1e-3     # relative L2 tolerance on the fp32 output


def to_dev(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def bf16_bits_of(t) -> np.ndarray:
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def rne_bf16(x32: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def errors(got: np.ndarray, want: np.ndarray):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    diff = got - want
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    den = float(np.linalg.norm(want))
    rel = float(np.linalg.norm(diff) / den) if den > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_parity(got, want, atol=ATOL, rel_l2=REL_L2, what="out"):
    max_abs, rel = errors(got, want)
    print(f"[parity] {what}: max-abs {max_abs:.3e} rel-L2 {rel:.3e}", flush=True)
    assert max_abs <= atol, f"{what}: max-abs {max_abs:.3e} > {atol}"
    assert rel <= rel_l2, f"{what}: rel-L2 {rel:.3e} > {rel_l2}"


def selection_mismatches(gpu_idx: np.ndarray, ora_idx: np.ndarray, scores: np.ndarray, k: int,
                         tie_rel: float = 1e-6):
    """(#rows that differ, #differences excused as near-ties, #unexcused differences).

    A membership difference at (i, j) is excused when |s_ij - s_i,(k)| is at
    most tie_rel times the row's largest |score|, s_i,(k) being the k-th
    largest score of the row."""
    rows = excused = bad = 0
    for i in range(ora_idx.shape[0]):
        a, b = set(gpu_idx[i].tolist()), set(ora_idx[i].tolist())
        if a == b:
            continue
        rows += 1
        kth = np.sort(scores[i])[::-1][k - 1]
        tol = tie_rel * np.abs(scores[i]).max()
        for j in a ^ b:
            if abs(scores[i, j] - kth) <= tol:
                excused += 1
            else:
                bad += 1
    return rows, excused, bad


def oracle_pool():
    """Single-threaded oracle worker processes, at most 16 (the host share of
    one GPU), started with `spawn` (no GPU state crosses into them)."""
    saved = {v: os.environ.get(v) for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS")}
    for v in saved:
        os.environ[v] = "1"
    n = max(1, min(16, len(os.sched_getaffinity(0))))
    ex = cf.ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"))
    for v, old in saved.items():
        if old is None:
            os.environ.pop(v)
        else:
            os.environ[v] = old
    return ex, n
