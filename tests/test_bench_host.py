"""Host-side logic of bench.py (CPU only): the one-GPU refusal, the algorithmic
operation counts behind the roofline figure, and the source-hash gate on the
committed HBM traffic figure."""
import hashlib
import os
import subprocess
import sys

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert r.stdout == ""
    assert "one GPU" in r.stderr


def test_work_counts_match_a_pair_by_pair_count():
    rng = np.random.default_rng(7)
    B, H, N, d = 1, 3, 700, 128  # 11 blocks, the last of 60 rows
    nb = (N + 63) // 64
    k = 4
    idx = np.stack([np.stack([np.sort(rng.choice(nb, k, replace=False)) for _ in range(nb)])
                    for _ in range(B * H)]).reshape(B, H, nb, k)
    rows = [min(64, N - 64 * b) for b in range(nb)]
    qk = pv = kept_share = direct = 0.0
    for bh in range(B * H):
        for i in range(nb):
            for j in idx.reshape(B * H, nb, k)[bh, i]:
                qk += 2 * d * rows[i] * rows[j]          # Q.K^T, valid rows only
                pv += 2 * d * rows[i] * rows[j]          # P.V
                kept_share += 4 * d * rows[i] * rows[j]  # phi(Q)phi(K)^T then times V
            unkept = N - sum(rows[j] for j in idx.reshape(B * H, nb, k)[bh, i])
            direct += 4 * d * rows[i] * unkept
    got_qk, got_f16 = bench.work_counts(idx, N, d, B * H, False, True, False)
    assert got_qk == qk
    assert got_f16 == pv + kept_share + 2 * d * d * N * B * H  # + phi(Q)H per row
    _, got_soft = bench.work_counts(idx, N, d, B * H, False, False, False)
    assert got_soft == pv
    _, got_direct = bench.work_counts(idx, N, d, B * H, False, True, True)
    assert got_direct == pv + direct


def test_traffic_figure_follows_the_kernel_source(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel source\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    prof = tmp_path / "counters.md"
    prof.write_text(f"# counters\n\nkernel_source_sha256: {sha}\n"
                    "traffic_bytes_per_launch: 123456789\n")
    monkeypatch.setattr(bench, "SPARSE_SRC", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(prof))
    assert bench.measured_traffic("wan14b720", 0.1, "elu1") == 123456789
    # another workload, keep fraction or feature map was not measured
    assert bench.measured_traffic("wan14b480", 0.1, "elu1") is None
    assert bench.measured_traffic("wan14b720", 0.2, "elu1") is None
    assert bench.measured_traffic("wan14b720", 0.1, "relu") is None
    # a changed kernel invalidates the figure
    src.write_text("// kernel source, changed\n")
    assert bench.measured_traffic("wan14b720", 0.1, "elu1") is None


def test_committed_traffic_profile_names_its_source_hash():
    fields = {}
    for line in open(bench.TRAFFIC_PROFILE):
        key, sep, val = line.partition(":")
        if sep and not line.startswith((" ", "#", "-", "|")):
            fields[key.strip()] = val.strip()
    assert len(fields.get("kernel_source_sha256", "")) == 64
    assert int(fields["traffic_bytes_per_launch"]) > 0


def test_cpu_baseline_host_logic():
    """The CPU-baseline leg on the tiny workload: one process per head, its
    sample flagged and described, and the parity / selection summaries exact
    when they are handed the oracle's own output and selection."""
    import bench
    from oracle import sla_oracle as O
    from sparse_linear_attention_sagesla_amd.inputs import WORKLOADS, make_head
    wl = WORKLOADS["tiny"]
    blocks = sorted(set(np.linspace(0, 31, 6).astype(int).tolist()))
    rows, idx = [], []
    for h in range(wl.H):
        q, k, v = make_head(wl, 0, h)
        r = O.sla_forward_head(q, k, v, 64, 0.1, "elu1", query_blocks=blocks)
        rows.append(r["out"].astype(np.float32))
        idx.append(r["idx"])
    base, parity, ties, used = bench.cpu_baseline(wl, 0.1, "elu1", np.stack(rows),
                                                  np.stack(idx)[None], blocks_per_head=6)
    assert used == blocks
    assert base["sampled"] is True and base["kind"] == "oracle" and base["cores"] == 2
    assert base["nproc"] >= 1 and base["cpu_model"] and base["value"] > 0
    assert 0 < base["sample_fraction"] <= 1
    assert parity["max_abs"] < 1e-6 and parity["rel_l2"] < 1e-7   # fp32 rounding only
    assert ties == {"heads": 2, "rows_differing": 0, "near_ties_excused": 0, "unexcused": 0}
