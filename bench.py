"""Benchmark of the SageSLA attention forward on one MI355X.

One step = one sla_attention_fwd call (every stage: block statistics, K mean,
INT8 quantisation, top-k selection, linear-branch staging and state, the
block-sparse kernel with the fused linear branch and combine) over the whole
workload, inputs resident in HBM, bf16 output, workspace preallocated.

Prints one JSON line on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload wan14b720]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SLA attn fwd ms/call + effective TOPS (% MFMA peak), Wan-14B-720p shape"
PEAK_I8_OPS = 5.0e15        # MI355X dense INT8 MFMA
PEAK_F16_FLOPS = 2.5e15     # MI355X dense fp16/bf16 MFMA
PEAK_HBM = 8.0e12           # MI355X HBM3E bytes/s
PEAK_F64_FLOPS = 78.6e12    # MI355X fp64 vector
STAGES = ["stats", "kmean", "quantize", "topk", "linear_prep", "linear_final", "sparse", "schedule"]
BWD_STAGES = ["fwd_staging", "transpose", "columns", "query", "grad_h", "key"]
SPARSE_SRC = os.path.join(ROOT, "sparse_linear_attention_sagesla_amd", "csrc", "sla_sparse.hip")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "sparse_fwd_kernel_wan14b720_counters.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles (the library records them on the launch stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            ev = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(ev))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            out.append(ev.value)
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def measured_traffic(workload: str, keep: float, phi: str):
    """HBM bytes per sparse-kernel launch from the committed rocprofv3 counter
    summary (calibrated FETCH_SIZE + WRITE_SIZE), or None when that summary was
    taken on a different kernel source or workload."""
    import hashlib
    if (workload, keep, phi) != ("wan14b720", 0.1, "elu1") or not os.path.exists(TRAFFIC_PROFILE):
        return None
    fields = {}
    for line in open(TRAFFIC_PROFILE):
        if ":" in line and not line.startswith((" ", "#", "-", "|")):
            key, _, val = line.partition(":")
            fields[key.strip()] = val.strip()
    sha = hashlib.sha256(open(SPARSE_SRC, "rb").read()).hexdigest()
    if fields.get("kernel_source_sha256") != sha or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def work_counts(idx: np.ndarray, N: int, d: int, BH: int, keep_all: bool, linear: bool,
                direct: bool):
    """Algorithmic operation counts of one call from the selection idx [B,H,Nb,k].

    Valid-row products only (the ragged last block counts its real rows).
    Returns (int8 ops of Q.K^T, 16-bit flops of the sparse kernel)."""
    nb = idx.shape[2]
    rows = np.full(nb, 64, dtype=np.int64)
    rows[-1] = N - 64 * (nb - 1)
    kept_rows = rows[idx.reshape(-1, idx.shape[-1])].sum(axis=1)          # per (bh, i)
    ni = np.tile(rows, idx.shape[0] * idx.shape[1])
    kept_pairs_rows = float((ni * kept_rows).sum())                         # sum_i n_i sum_j n_j
    qk = 2.0 * d * kept_pairs_rows
    pv = 2.0 * d * kept_pairs_rows
    lin = 0.0
    if linear:
        if direct:
            lin = 2 * 2.0 * d * float((ni * (N - kept_rows)).sum())
        else:
            lin = 2 * 2.0 * d * kept_pairs_rows + 2.0 * d * d * N * BH     # kept share + phi(Q)H
    return qk, pv + lin


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_sample_job(job):
    """One worker of the CPU baseline: the fp64 oracle on one head, timed once
    for a single query block and once for the whole sample (the difference
    splits per-head setup from per-block time), after one untimed call so that
    first-use costs fall in neither.  Single-threaded BLAS."""
    from oracle import sla_oracle as O
    from sparse_linear_attention_sagesla_amd.inputs import WORKLOADS, make_head
    name, h, blocks, keep, phi = job
    q, k, v = make_head(WORKLOADS[name], 0, h)
    O.sla_forward_head(q, k, v, 64, keep, phi, query_blocks=blocks[:1])
    t0 = time.perf_counter()
    O.sla_forward_head(q, k, v, 64, keep, phi, query_blocks=blocks[:1])
    t1 = time.perf_counter()
    r = O.sla_forward_head(q, k, v, 64, keep, phi, query_blocks=blocks)
    t2 = time.perf_counter()
    return h, t1 - t0, t2 - t1, r["out"]


def _near_tie_job(job):
    """Oracle selection of one head against the GPU's: (rows that differ,
    differences within 1e-6 of the row's largest |score| of the k-th score,
    other differences)."""
    from oracle import sla_oracle as O
    from sparse_linear_attention_sagesla_amd.inputs import WORKLOADS, make_head
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
            excused, bad = (excused + 1, bad) if abs(sc[i, j] - kth) <= tol else (excused, bad + 1)
    return rows, excused, bad


def cpu_baseline(wl, keep, phi, gpu_out_rows=None, gpu_idx=None, blocks_per_head=160):
    """The fp64 oracle as it stands, on the host cores (one single-threaded
    process per core, at most 16, the host share of one GPU), on a bounded
    sample: one head per worker, the per-head setup (selection, K mean,
    quantisation) plus ``blocks_per_head`` query blocks spread over the head.
    The per-block and per-head times measured under that load give the time of
    the whole workload spread over the same cores.  With ``gpu_out_rows`` (the
    GPU's fp32 output on the sampled rows) the oracle's output on the sample
    is compared with it; with ``gpu_idx`` every head's selection is compared."""
    import concurrent.futures as cf
    import multiprocessing as mp
    from oracle import sla_oracle as O
    nb = O.n_blocks(wl.N, 64)
    cores = max(1, min(16, len(os.sched_getaffinity(0)), wl.B * wl.H))
    heads = list(range(cores))
    blocks = sorted(set(np.linspace(0, nb - 1, blocks_per_head).astype(int).tolist()))
    env = {v: os.environ.get(v) for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for v_ in env:
        os.environ[v_] = "1"
    try:
        ctx = mp.get_context("spawn")
        with cf.ProcessPoolExecutor(max_workers=cores, mp_context=ctx) as ex:
            t = time.perf_counter()
            res = list(ex.map(_oracle_sample_job, [(wl.name, h, blocks, keep, phi) for h in heads]))
            wall = time.perf_counter() - t
            ties = None
            if gpu_idx is not None:
                per = list(ex.map(_near_tie_job, [(wl.name, h, keep, gpu_idx[0, h])
                                                  for h in range(wl.H)]))
                ties = {"heads": wl.H, "rows_differing": int(sum(p[0] for p in per)),
                        "near_ties_excused": int(sum(p[1] for p in per)),
                        "unexcused": int(sum(p[2] for p in per))}
    finally:
        for v_, old in env.items():
            if old is None:
                os.environ.pop(v_, None)
            else:
                os.environ[v_] = old
    per_block = max(float(np.mean([(full - one) / max(len(blocks) - 1, 1) for _, one, full, _ in res])), 0.0)
    setup = float(np.mean([max(one - per_block, 0.0) for _, one, _, _ in res]))
    work_s = wl.B * wl.H * (setup + nb * per_block)
    out = {"value": 1e3 * work_s / cores, "unit": "ms/call", "cores": cores, "kind": "oracle",
           "sampled": True, "nproc": os.cpu_count(), "cpu_model": _cpu_model(),
           "sample": (f"{wl.name}: heads 0-{cores - 1}, one per single-threaded process; per "
                      f"head the setup (selection, K mean, quantisation, {setup:.2f} s) and "
                      f"{len(blocks)} query blocks spread over the head ({per_block * 1e3:.1f} ms "
                      f"each); value = {wl.B * wl.H} heads x (setup + {nb} blocks) over {cores} "
                      f"processes; {wall:.1f} s wall for the sample"),
           "sample_fraction": round(cores * len(blocks) / (wl.B * wl.H * nb), 5)}
    parity = None
    if gpu_out_rows is not None:
        got = np.concatenate([gpu_out_rows[h].astype(np.float64).ravel() for h, _, _, _ in res])
        want = np.concatenate([r.ravel() for _, _, _, r in res])
        diff = got - want
        parity = {"heads": cores, "query_blocks_per_head": len(blocks),
                  "max_abs": float(np.abs(diff).max()),
                  "rel_l2": float(np.linalg.norm(diff) / np.linalg.norm(want)),
                  "bar": {"max_abs": 2e-3, "rel_l2": 1e-3}}
    return out, parity, ties, blocks


def lowbit_leg(lib, _lib, op, q, k, v, wl, keep, phi, f16_equiv, exact_sparse_ms, steps, stream):
    """sla_attention_fwd_lowbit (phi(K) of the linear branch in FP8) on the same
    inputs: ms per call, and the attention kernel's time and roofline from
    calls with stage events (same algorithmic work as the exact forward)."""
    import torch
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    ph = _lib.PHI[phi]

    def call(events=None):
        ev = (ctypes.c_void_p * len(events))(*events) if events else None
        rc = lib.sla_attention_fwd_ex(
            _lib._ptr(q), _lib._ptr(k), _lib._ptr(v), B, H, N, d, 64, float(keep), ph,
            _lib._ptr(op.out), 0, None, _lib._ptr(op.workspace), op.workspace.numel(),
            ctypes.c_void_p(stream.cuda_stream), ev, _lib.OPT_PHI_K_FP8)
        if rc != 0:
            raise RuntimeError(lib.sla_status_string(rc).decode())

    call()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        call()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    hip = HipEvents()
    evs = [hip.create(2 * len(STAGES)) for _ in range(steps)]
    for e in evs:
        call(e)
    torch.cuda.synchronize()
    si = STAGES.index("sparse")
    sparse_ms = float(np.mean([hip.elapsed_ms(e[2 * si], e[2 * si + 1]) for e in evs]))
    for e in evs:
        hip.destroy(e)
    achieved = f16_equiv / (sparse_ms * 1e-3) / 1e12
    log(f"[bench] lowbit: {ms:.3f} ms/call, attention kernel {sparse_ms:.3f} ms")
    return {"ms_per_call": round(ms, 4), "steps": steps, "sparse_ms": round(sparse_ms, 4),
            "sparse_speedup_vs_exact": round(exact_sparse_ms / sparse_ms, 4),
            "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                         "peak": PEAK_F16_FLOPS / 1e12, "unit": "TFLOP/s",
                         "frac": round(achieved / (PEAK_F16_FLOPS / 1e12), 4),
                         "kernel": "sparse_fwd_kernel (FP8 phi(K))",
                         "note": "the products stay INT8 and fp16 (phi(K) is decoded to fp16 "
                                 "as it is read), so the peak is the fp16 one; 32 instead of "
                                 "40 KB staged per kept pair"},
            "note": "opt-in: linear branch's phi(K) as FP8 e4m3 with one power-of-two scale "
                    "per key block"}


def backward_leg(sla, lib, _lib, q, k, v, wl, keep, phi, fwd_ms, steps, stream, dev):
    """sla_attention_bwd on the same inputs and a seeded dO: ms per call (one
    warmup call, then `steps` timed calls back to back, bf16 gradients)."""
    import torch
    from sparse_linear_attention_sagesla_amd.inputs import make_dout
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    g = torch.from_numpy(make_dout(wl).view(np.int16)).view(torch.bfloat16).to(dev)
    ph = _lib.PHI[phi]
    nbytes = sla.workspace_size(sla.OP_ATTENTION_BWD, B, H, N, keep, ph)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    grads = [torch.empty(B, H, N, d, dtype=torch.bfloat16, device=dev) for _ in range(3)]

    def call(events=None):
        ev = (ctypes.c_void_p * len(events))(*events) if events else None
        rc = lib.sla_attention_bwd_timed(_lib._ptr(q), _lib._ptr(k), _lib._ptr(v), _lib._ptr(g), B,
                                         H, N, d, 64, float(keep), ph,
                                         *[_lib._ptr(x) for x in grads], 0, _lib._ptr(ws),
                                         ws.numel(), ctypes.c_void_p(stream.cuda_stream), ev)
        if rc != 0:
            raise RuntimeError(lib.sla_status_string(rc).decode())

    call()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        call()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    log(f"[bench] backward: {ms:.3f} ms/call over {steps} calls")
    # stage times from further calls with stage events
    hip = HipEvents()
    evs = [hip.create(2 * len(BWD_STAGES)) for _ in range(steps)]
    for e in evs:
        call(e)
    torch.cuda.synchronize()
    nb = sla.n_blocks(N)
    kk = sla.topk_count(nb, keep)
    linear = phi != "none" and kk < nb
    stage_ms = {}
    for si, name in enumerate(BWD_STAGES):
        if (name == "columns" and kk == 0) or (name == "grad_h" and not linear):
            continue
        stage_ms[name] = float(np.mean([hip.elapsed_ms(e[2 * si], e[2 * si + 1]) for e in evs]))
    for e in evs:
        hip.destroy(e)
    rec = {"ms_per_call": round(ms, 4), "steps": steps, "ratio_to_forward": round(ms / fwd_ms, 3),
           "grad_dtype": "bf16", "workspace_bytes": int(nbytes),
           "stages_ms": {n: round(v, 4) for n, v in stage_ms.items()},
           "note": "sla_attention_bwd: selection, codes and linear state recomputed, then "
                   "dQ (query side), G, dK/dV (key side)"}
    if kk > 0:
        # matrix-core work of the two attention kernels on valid rows, fp16-equivalent
        idx = sla.block_select(q, k, keep).cpu().numpy()
        nbk = idx.shape[2]
        rows = np.full(nbk, 64, dtype=np.int64)
        rows[-1] = N - 64 * (nbk - 1)
        kept_rows = rows[idx.reshape(-1, idx.shape[-1])].sum(axis=1)
        P = float((np.tile(rows, idx.shape[0] * idx.shape[1]) * kept_rows).sum())
        lin = 1.0 if linear else 0.0
        work = {  # (INT8 ops, fp16/bf16 flops)
            "query": (2 * 2 * d * P, 2 * d * P + lin * 4 * d * P + 4 * d * P
                      + lin * 3 * 2 * d * d * N * B * H),
            "key": (2 * d * P, 6 * d * P + lin * 4 * d * P + lin * 2 * 2 * d * d * N * B * H),
        }
        rl = {}
        for name, (i8, f16) in work.items():
            t_s = stage_ms[name] * 1e-3
            ach = (0.5 * i8 + f16) / t_s / 1e12
            rl[name] = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_F16_FLOPS / 1e12,
                        "unit": "TFLOP/s", "frac": round(ach / (PEAK_F16_FLOPS / 1e12), 4),
                        "kernel": "bwd_q_kernel" if name == "query" else "bwd_kv_kernel"}
        rec["roofline"] = rl
    rec["training"] = training_leg(sla, lib, _lib, q, k, v, g, wl, keep, phi, ph, ws, grads, ms, steps,
                                   stream, dev, P if kk > 0 else 0.0, linear)
    return rec


def training_leg(sla, lib, _lib, q, k, v, g, wl, keep, phi, ph, ws, grads, bwd_ms, steps, stream, dev,
                 pairs_rows, linear):
    """A training step's attention: sla_attention_fwd_train (the forward plus
    its residuals) and sla_attention_bwd_saved (the backward from them), each
    timed over `steps` calls after one warmup call; stage times of the saved
    backward; the query side's matrix-core roofline on its (one-sweep) work."""
    import torch
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    rbytes = sla.train_residual_bytes(B, H, N, keep, ph)
    res = torch.empty(rbytes, dtype=torch.uint8, device=dev)
    fws = torch.empty(sla.workspace_size(sla.OP_ATTENTION, B, H, N, keep, ph), dtype=torch.uint8,
                      device=dev)
    out = torch.empty(B, H, N, d, dtype=torch.bfloat16, device=dev)
    sp = ctypes.c_void_p(stream.cuda_stream)

    def fwd():
        rc = lib.sla_attention_fwd_train(_lib._ptr(q), _lib._ptr(k), _lib._ptr(v), B, H, N, d, 64,
                                         float(keep), ph, _lib._ptr(out), 0, _lib._ptr(res), rbytes,
                                         _lib._ptr(fws), fws.numel(), sp)
        if rc != 0:
            raise RuntimeError(lib.sla_status_string(rc).decode())

    def bwd(events=None):
        ev = (ctypes.c_void_p * len(events))(*events) if events else None
        rc = lib.sla_attention_bwd_saved(_lib._ptr(q), _lib._ptr(k), _lib._ptr(v), _lib._ptr(g),
                                         _lib._ptr(res), rbytes, B, H, N, d, 64, float(keep), ph,
                                         *[_lib._ptr(x) for x in grads], 0, _lib._ptr(ws), ws.numel(),
                                         sp, ev)
        if rc != 0:
            raise RuntimeError(lib.sla_status_string(rc).decode())

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(steps):
            fn()
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    f_ms = timed(fwd)
    b_ms = timed(bwd)
    log(f"[bench] training: forward with residuals {f_ms:.3f} ms, saved backward {b_ms:.3f} ms")
    hip = HipEvents()
    evs = [hip.create(2 * len(BWD_STAGES)) for _ in range(steps)]
    for e in evs:
        bwd(e)
    torch.cuda.synchronize()
    kk = sla.topk_count(sla.n_blocks(N), keep)
    stage_ms = {}
    for si, name in enumerate(BWD_STAGES):
        if (name == "columns" and kk == 0) or (name == "grad_h" and not linear):
            continue
        stage_ms[name] = float(np.mean([hip.elapsed_ms(e[2 * si], e[2 * si + 1]) for e in evs]))
    for e in evs:
        hip.destroy(e)
    rec = {"forward_ms": round(f_ms, 4), "backward_ms": round(b_ms, 4),
           "step_ms": round(f_ms + b_ms, 4), "residual_bytes": int(rbytes),
           "backward_stages_ms": {n: round(x, 4) for n, x in stage_ms.items()},
           "backward_speedup_vs_recompute": round(bwd_ms / b_ms, 3),
           "note": "sla_attention_fwd_train + sla_attention_bwd_saved: the query side reads the "
                   "forward's row statistics, outputs and kept share instead of re-walking the kept tiles"}
    if kk > 0:
        lin = 1.0 if linear else 0.0
        i8, f16 = 2 * d * pairs_rows, 4 * d * pairs_rows + lin * 3 * 2 * d * d * N * B * H
        ach = (0.5 * i8 + f16) / (stage_ms["query"] * 1e-3) / 1e12
        rec["query_roofline"] = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_F16_FLOPS / 1e12,
                                 "unit": "TFLOP/s", "frac": round(ach / (PEAK_F16_FLOPS / 1e12), 4),
                                 "kernel": "bwd_q_kernel (saved form)"}
    del res, fws, out
    return rec


def w8a8_leg(sla, wl, steps, stream, dev):
    """FusedNorm + W8A8 GEMM of the Wan-14B FFN up-projection at this
    workload's token count: x [N, 5120] bf16 N(0,1), W [13824, 5120] bf16
    N(0, 0.02^2) quantised per output channel once (untimed), then `steps`
    timed FusedNorm calls and `steps` timed GEMM calls (bf16 output)."""
    import torch
    M, K, Nf = wl.N, 5120, 13824
    g = torch.Generator(device=dev).manual_seed(11)
    x = torch.randn(M, K, device=dev, generator=g).to(torch.bfloat16)
    w = (0.02 * torch.randn(Nf, K, device=dev, generator=g)).to(torch.bfloat16)
    w8, sw = sla.rowquant_i8(w)
    x8, sx, _, _ = sla.fused_norm_i8(x)
    y = torch.empty(M, Nf, dtype=torch.bfloat16, device=dev)
    sla.w8a8_linear(x8, sx, w8, sw, out=y)
    torch.cuda.synchronize()

    def timed(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    norm_ms = timed(lambda: sla.fused_norm_i8(x))
    gemm_ms = timed(lambda: sla.w8a8_linear(x8, sx, w8, sw, out=y))
    del y
    # context: the vendor library's INT8 product of the same codes (int32
    # result, no scales) and its bf16 product of the unquantised operands
    acc = torch._int_mm(x8, w8.t())
    lib_i8_ms = timed(lambda: torch._int_mm(x8, w8.t()))
    del acc
    wt = w.t().contiguous()
    yb = torch.matmul(x, wt)
    lib_bf16_ms = timed(lambda: torch.matmul(x, wt))
    del yb, wt
    ops = 2.0 * M * Nf * K
    tops = ops / (gemm_ms * 1e-3) / 1e12
    norm_bytes = M * K * 2 + M * K + M * 12
    gbps = norm_bytes / (norm_ms * 1e-3) / 1e9
    log(f"[bench] w8a8: FusedNorm {norm_ms:.3f} ms, GEMM {gemm_ms:.3f} ms ({tops:.0f} TOPS); "
        f"library INT8 product {lib_i8_ms:.3f} ms, bf16 product {lib_bf16_ms:.3f} ms")
    return {"config": {"M": M, "K": K, "N": Nf, "layer": "Wan-14B FFN up-projection"},
            "fused_norm_ms": round(norm_ms, 4), "gemm_ms": round(gemm_ms, 4),
            "library_int8_mm_ms": round(lib_i8_ms, 4), "library_bf16_mm_ms": round(lib_bf16_ms, 4),
            "gemm_roofline": {"bound": "mfma", "achieved": round(tops, 1), "peak": PEAK_I8_OPS / 1e12,
                              "unit": "TOP/s", "frac": round(tops / (PEAK_I8_OPS / 1e12), 4),
                              "kernel": "w8a8_gemm_kernel"},
            "fused_norm_roofline": {"bound": "hbm", "achieved": round(gbps, 1),
                                    "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                                    "frac": round(gbps * 1e9 / PEAK_HBM, 4),
                                    "kernel": "rowquant_kernel<true>"}}


def dense_gemm_reference(dev, stream, n=16384, reps=3):
    """What the vendor library's dense fp16 product (torch.matmul, hipBLASLt)
    reaches on this GPU in this process: an n x n x n product, fp32
    accumulation, fp16 output, the best of `reps` runs after two untimed ones.
    It is the same matrix-core instruction family the attention kernel's P.V
    and linear-branch products use, on a plain dense GEMM: a practical
    ceiling beside the datasheet peak, for context."""
    import torch
    g = torch.Generator(device=dev).manual_seed(7)
    a = torch.randn(n, n, device=dev, generator=g, dtype=torch.float16)
    b = torch.randn(n, n, device=dev, generator=g, dtype=torch.float16)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    with torch.cuda.stream(stream):
        for it in range(reps + 2):
            start.record(stream)
            c = torch.matmul(a, b)
            end.record(stream)
            torch.cuda.synchronize()
            if it >= 2:
                times.append(start.elapsed_time(end) * 1e-3)
            del c
    del a, b
    t = min(times)
    tflops = 2.0 * n ** 3 / t / 1e12
    return {"kernel": "torch.matmul fp16 (hipBLASLt)", "shape": [n, n, n], "ms": round(t * 1e3, 4),
            "achieved": round(tflops, 1), "unit": "TFLOP/s",
            "frac_of_peak": round(tflops / (PEAK_F16_FLOPS / 1e12), 4),
            "note": f"best of {reps}; the attention kernel's roofline.frac_of_dense_gemm divides its "
                    "achieved rate by this one"}


def streaming_ceiling(dev, stream, mib=1024, reps=5):
    """What plain streaming reaches on this GPU in this process: a device copy of
    `mib` MiB (read + write bytes over time) and a read-only bf16 sum over
    the same buffer, each the best of `reps` runs on `stream`."""
    import torch
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    x = a.view(torch.bfloat16)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best(fn):
        fn()
        times = []
        for _ in range(reps):
            start.record(stream)
            fn()
            end.record(stream)
            torch.cuda.synchronize()
            times.append(start.elapsed_time(end) * 1e-3)
        return min(times)

    # three reads per write (about the statistics pass's mix, 4:1): d = a + b * c
    # over four bf16 tensors of a quarter of the buffer each
    m = n // 8
    ta, tb, tc, td = (torch.empty(m, dtype=torch.bfloat16, device=dev) for _ in range(4))
    for t_ in (ta, tb, tc):
        t_.fill_(1.0)
    with torch.cuda.stream(stream):
        t_copy = best(lambda: b.copy_(a))
        t_read = best(lambda: torch.sum(x, dtype=torch.float32))
        t_rw3 = best(lambda: torch.addcmul(ta, tb, tc, out=td))
    del a, b, x, ta, tb, tc, td
    return {"copy_gbps": round(2 * n / t_copy / 1e9, 1), "read_gbps": round(n / t_read / 1e9, 1),
            "read3_write1_gbps": round(4 * 2 * m / t_rw3 / 1e9, 1),
            "bytes": n, "note": "device copy (read + write bytes), bf16 sum (read bytes) and an "
                                "elementwise d = a + b*c (3 reads : 1 write), best of "
                                f"{reps}; stage_frac_of_copy divides each streaming stage's rate by the "
                                "copy rate, stage_frac_of_mix by the reference closest to its read/write mix"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan14b720")
    ap.add_argument("--keep", type=float, default=None)
    ap.add_argument("--phi", default="elu1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward-steps", type=int, default=3,
                    help="also time this many sla_attention_bwd calls (0: skip)")
    ap.add_argument("--lowbit-steps", type=int, default=5,
                    help="also time this many calls of the lower-bit forward (0: skip)")
    ap.add_argument("--w8a8-steps", type=int, default=5,
                    help="also time this many FusedNorm + W8A8 GEMM calls at the Wan-14B "
                         "FFN shape (0: skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 times), to scale "
                         "hardware byte counters against a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the SageSLA forward is sharded by heads with no "
              f"communication, so --gpus {args.gpus} is not run here", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.copy_calibration} MiB 5 times")
        return

    import sparse_linear_attention_sagesla_amd as sla
    from sparse_linear_attention_sagesla_amd import _lib
    from sparse_linear_attention_sagesla_amd.inputs import WORKLOADS, make_inputs

    wl = WORKLOADS[args.workload]
    keep = wl.keep[0] if args.keep is None else args.keep
    phi = args.phi
    if keep >= 1.0:
        phi = "none"
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    log(f"[bench] workload {wl.name} B={B} H={H} N={N} keep={keep} phi={phi}")
    t = time.perf_counter()
    Q, K, V = make_inputs(wl)
    log(f"[bench] inputs generated in {time.perf_counter() - t:.1f} s")
    dev = torch.device("cuda:0")

    def to_dev(x):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    op = sla.SLAAttention(B, H, N, keep=keep, phi=phi, out_dtype=torch.bfloat16, device=dev)
    lib = _lib.load()
    ph = _lib.PHI[phi]
    stream = torch.cuda.current_stream(dev)

    def call(events=None):
        # the plain entry point; with stage events, the same call recording them
        if events is None:
            rc = lib.sla_attention_fwd(
                _lib._ptr(q), _lib._ptr(k), _lib._ptr(v), B, H, N, d, 64, float(keep), ph,
                _lib._ptr(op.out), 0, _lib._ptr(op.workspace), op.workspace.numel(),
                ctypes.c_void_p(stream.cuda_stream))
        else:
            ev = (ctypes.c_void_p * len(events))(*events)
            rc = lib.sla_attention_fwd_ex(
                _lib._ptr(q), _lib._ptr(k), _lib._ptr(v), B, H, N, d, 64, float(keep), ph,
                _lib._ptr(op.out), 0, None, _lib._ptr(op.workspace), op.workspace.numel(),
                ctypes.c_void_p(stream.cuda_stream), ev, 0)
        if rc != 0:
            raise RuntimeError(lib.sla_status_string(rc).decode())

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    log(f"[bench] {args.warmup} warmup steps done")

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for s in range(args.steps):
        call()
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    log(f"[bench] {args.steps} timed steps: {ms_step:.3f} ms/step")

    # the same call with the selection on a second stream (sla_attention_fwd_fork)
    side = torch.cuda.Stream(device=dev)
    ref_out = op.out.clone()

    def call_fork():
        rc = lib.sla_attention_fwd_fork(
            _lib._ptr(q), _lib._ptr(k), _lib._ptr(v), B, H, N, d, 64, float(keep), ph,
            _lib._ptr(op.out), 0, _lib._ptr(op.workspace), op.workspace.numel(),
            ctypes.c_void_p(stream.cuda_stream), ctypes.c_void_p(side.cuda_stream))
        if rc != 0:
            raise RuntimeError(lib.sla_status_string(rc).decode())

    for _ in range(args.warmup):
        call_fork()
    torch.cuda.synchronize()
    fork_same = bool(torch.equal(op.out, ref_out))
    start.record(stream)
    for s in range(args.steps):
        call_fork()
    end.record(stream)
    torch.cuda.synchronize()
    ms_fork = start.elapsed_time(end) / args.steps
    del ref_out
    log(f"[bench] {args.steps} timed steps with the selection on a second stream: {ms_fork:.3f} ms/step "
        f"(output identical: {fork_same})")
    if not fork_same:
        raise RuntimeError("sla_attention_fwd_fork changed the output")
    # the headline call is the plain entry point (every stage on the caller's
    # stream); the forked one is reported beside it

    # stage breakdown: separate calls with stage events, in which the library
    # runs every stage on this stream one after another (timed alone)
    hip = HipEvents()
    evs = [hip.create(2 * len(STAGES)) for _ in range(min(args.steps, 5))]
    for e in evs:
        call(e)
    torch.cuda.synchronize()

    nb = sla.n_blocks(N)
    kk = sla.topk_count(nb, keep)
    linear = phi != "none" and kk < nb
    direct = linear and (nb - kk) <= kk
    skipped = {2}  # the INT8 coding runs inside the statistics and staging passes
    if kk == 0:
        skipped |= {0, 1, 3, 7}
    if direct:
        skipped.add(7)
    if not linear or direct:
        skipped.add(5)
    stage_ms = {}
    for si, name in enumerate(STAGES):
        if si in skipped:
            continue
        stage_ms[name] = float(np.mean([hip.elapsed_ms(e[2 * si], e[2 * si + 1]) for e in evs]))
    for e in evs:
        hip.destroy(e)

    if kk > 0:
        idx = sla.block_select(q, k, keep).cpu().numpy()
        ops_i8, ops_16 = work_counts(idx, N, d, B * H, kk == nb, linear, direct)
    else:
        ops_i8, ops_16 = 0.0, 2.0 * d * d * N * B * H * 2
    t_sparse = stage_ms["sparse"] * 1e-3
    f16_equiv = ops_i8 * (PEAK_F16_FLOPS / PEAK_I8_OPS) + ops_16
    achieved = f16_equiv / t_sparse / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_F16_FLOPS / 1e12,
                "unit": "TFLOP/s", "frac": round(achieved / (PEAK_F16_FLOPS / 1e12), 4),
                "traffic": measured_traffic(wl.name, keep, phi), "kernel": "sparse_fwd_kernel",
                "note": "fp16-equivalent: INT8 ops weighted 0.5 (INT8 peak is 2x the fp16 peak)"}
    codes = B * H * nb * 64 * d  # INT8 codes of one of Q, K
    bytes_io = {
        "stats": 2 * B * H * N * d * 2 + codes,
        "linear_prep": 2 * B * H * N * d * 2 + (2 if linear else 1) * B * H * nb * 64 * d * 2
        + (codes if kk > 0 else 0),
    }
    bw = {n: round(bytes_io[n] / (stage_ms[n] * 1e-3) / 1e9, 1) for n in bytes_io if n in stage_ms}
    hbm_frac = {n: round(g * 1e9 / PEAK_HBM, 3) for n, g in bw.items()}
    ceiling = streaming_ceiling(dev, stream)
    gemm_ref = dense_gemm_reference(dev, stream)
    roofline["frac_of_dense_gemm"] = round(achieved / gemm_ref["achieved"], 4)
    ceil_frac = {n: round(g / ceiling["copy_gbps"], 3) for n, g in bw.items()}
    # the statistics pass reads 4 bytes per byte written, the staging pass about 1:1.25
    mix_ref = {"stats": ceiling["read3_write1_gbps"], "linear_prep": ceiling["copy_gbps"]}
    mix_frac = {n: round(g / mix_ref[n], 3) for n, g in bw.items() if n in mix_ref}
    # whole call against its ideal: sparse work at the MFMA peaks, streaming
    # stages at the HBM peak, block scores at the fp64 vector peak
    ideal_s = ops_i8 / PEAK_I8_OPS + ops_16 / PEAK_F16_FLOPS
    ideal_s += sum(bytes_io[n] for n in bytes_io if n in stage_ms) / PEAK_HBM
    if kk > 0:
        ideal_s += 2.0 * B * H * nb * nb * d / PEAK_F64_FLOPS
    eff_tops = (ops_i8 + ops_16) / (ms_step * 1e-3) / 1e12
    dense_equiv = 4.0 * N * N * d * B * H / (ms_step * 1e-3) / 1e12
    rec = {
        "metric": METRIC, "value": round(ms_step, 4), "unit": "ms/call", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8+f16 (bf16 in/out)", "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "H": H, "N": N, "d": d, "block": 64,
                   "keep": keep, "k": kk, "phi": phi, "grid": wl.grid},
        "effective_tops": round(eff_tops, 2), "dense_equiv_tops": round(dense_equiv, 2),
        "stages_ms": {n: round(v, 4) for n, v in stage_ms.items()},
        "stage_hbm_gbps": bw,
        "stage_hbm_frac": hbm_frac,
        "streaming_ceiling": ceiling,
        "dense_gemm_reference": gemm_ref,
        "stage_frac_of_copy": ceil_frac,
        "stage_frac_of_mix": mix_frac,
        "call_roofline_frac": round(ideal_s / (ms_step * 1e-3), 4),
        "roofline": roofline,
        "call": {"entry": "sla_attention_fwd", "fork_ms": round(ms_fork, 4),
                 "fork_output_identical": fork_same,
                 "note": "value times sla_attention_fwd (every stage on the caller's stream); fork_ms "
                         "times sla_attention_fwd_fork (block scores, top-k and walk schedule on a "
                         "second caller stream, concurrent with the K mean and linear staging)"},
    }
    if args.lowbit_steps > 0 and linear:
        rec["lowbit"] = lowbit_leg(lib, _lib, op, q, k, v, wl, keep, phi, f16_equiv,
                                   stage_ms["sparse"], args.lowbit_steps, stream)
    if args.backward_steps > 0:
        rec["backward"] = backward_leg(sla, lib, _lib, q, k, v, wl, keep, phi, ms_step,
                                       args.backward_steps, stream, dev)
    if args.w8a8_steps > 0:
        rec["w8a8"] = w8a8_leg(sla, wl, args.w8a8_steps, stream, dev)
    if not args.no_cpu_baseline:
        from oracle import sla_oracle as O
        cores = max(1, min(16, len(os.sched_getaffinity(0)), B * H))
        blocks = sorted(set(np.linspace(0, nb - 1, 160).astype(int).tolist()))
        rows = np.concatenate([np.arange(i * 64, min(N, (i + 1) * 64)) for i in blocks])
        # the fp32 output on the sampled rows (one untimed call) and the selection
        out32 = sla.attention(q, k, v, keep, phi, torch.float32)
        gpu_rows = out32[0, :cores, torch.from_numpy(rows).to(dev)].cpu().numpy()
        del out32
        gpu_idx = idx if kk > 0 else None
        log(f"[bench] timing the CPU oracle on a bounded sample ({cores} processes) ...")
        base, parity, ties, _ = cpu_baseline(wl, keep, phi, gpu_rows, gpu_idx)
        rec["cpu_baseline"] = base
        rec["parity_sample"] = parity
        if ties is not None:
            rec["selection_vs_oracle"] = ties
        log(f"[bench] oracle: {base['value'] / 1e3:.1f} s/call on {cores} processes; parity "
            f"max-abs {parity['max_abs']:.2e} rel-L2 {parity['rel_l2']:.2e}; selection {ties}")
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
