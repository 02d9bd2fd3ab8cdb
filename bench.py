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


def cpu_baseline(Q, K, V, wl, keep, phi, n_blocks_sample=160):
    """The fp64 oracle on one head and a sample of its query blocks, scaled to ms/call."""
    from oracle import sla_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    nb = O.n_blocks(wl.N, 64)
    sample = sorted(set(np.linspace(0, nb - 1, n_blocks_sample + 1).astype(int).tolist()))
    t0 = time.perf_counter()
    O.sla_forward_head(Q[0, 0], K[0, 0], V[0, 0], 64, keep, phi, query_blocks=sample[:1])
    t1 = time.perf_counter()
    O.sla_forward_head(Q[0, 0], K[0, 0], V[0, 0], 64, keep, phi, query_blocks=sample)
    t2 = time.perf_counter()
    per_block = max((t2 - t1) - (t1 - t0), 0.0) / (len(sample) - 1)
    setup = max((t1 - t0) - per_block, 0.0)
    ms_call = 1e3 * wl.B * wl.H * (setup + nb * per_block)
    return {"value": ms_call, "unit": "ms/call", "cores": int(cores), "kind": "oracle",
            "sample": (f"head 0 of {wl.name}: per-head setup (selection, K mean, quantisation) "
                       f"{setup:.2f} s + {len(sample) - 1} sampled query blocks at "
                       f"{per_block * 1e3:.1f} ms each, scaled to {wl.B * wl.H} heads x {nb} "
                       f"query blocks; {t2 - t0:.1f} s of CPU work")}


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
        ev = (ctypes.c_void_p * len(events))(*events) if events else None
        rc = lib.sla_attention_fwd_timed(
            _lib._ptr(q), _lib._ptr(k), _lib._ptr(v), B, H, N, d, 64, float(keep), ph,
            _lib._ptr(op.out), 0, None, _lib._ptr(op.workspace), op.workspace.numel(),
            ctypes.c_void_p(stream.cuda_stream), ev)
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
        "call_roofline_frac": round(ideal_s / (ms_step * 1e-3), 4),
        "roofline": roofline,
    }
    if args.backward_steps > 0:
        rec["backward"] = backward_leg(sla, lib, _lib, q, k, v, wl, keep, phi, ms_step,
                                       args.backward_steps, stream, dev)
    if args.w8a8_steps > 0:
        rec["w8a8"] = w8a8_leg(sla, wl, args.w8a8_steps, stream, dev)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        rec["cpu_baseline"] = cpu_baseline(Q, K, V, wl, keep, phi)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
