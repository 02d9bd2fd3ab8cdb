"""The seeded generators: same bits in any process and thread layout, and
the smooth field is the trilinear interpolation it is described as."""
import hashlib
import os
import subprocess
import sys

import numpy as np

from sparse_linear_attention_sagesla_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _digest(arrs):
    h = hashlib.sha256()
    for a in arrs:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_generated_bits_do_not_depend_on_threads_or_process():
    wl = I.Workload("grid_small", 1, 4, 9 * 10 * 12, (9, 10, 12), 77)
    Q, K, V = I.make_inputs(wl, threads=4)
    here = _digest([Q, K, V])
    code = ("import sys; sys.path.insert(0, sys.argv[1]); import numpy as np, hashlib;"
            "from sparse_linear_attention_sagesla_amd import inputs as I;"
            "wl = I.Workload('grid_small', 1, 4, 9 * 10 * 12, (9, 10, 12), 77);"
            "h = hashlib.sha256();"
            "qs = [I.make_head(wl, 0, i) for i in range(4)];"
            "[h.update(np.ascontiguousarray(np.stack([q[t] for q in qs])).tobytes()) for t in range(3)];"
            "print(h.hexdigest())")
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1")
    other = subprocess.run([sys.executable, "-c", code, ROOT], env=env, capture_output=True,
                           text=True, check=True).stdout.strip()
    assert other == here
    tiny_a = I.make_inputs("tiny", threads=2)
    tiny_b = [np.stack([I.make_head(I.WORKLOADS["tiny"], 0, h)[t] for h in range(2)])[None]
              for t in range(3)]
    assert _digest(tiny_a) == _digest(tiny_b)


def test_smooth_field_is_trilinear_on_the_lattice():
    rng = np.random.Generator(np.random.PCG64(5))
    grid = (9, 10, 13)
    f = I._smooth_field(rng, grid, 3).reshape(*grid, 3)
    rng = np.random.Generator(np.random.PCG64(5))
    lat = rng.standard_normal((4, 4, 5, 3), dtype=np.float32).astype(np.float64)
    # the same field before the per-channel scaling, by direct trilinear weights
    ref = np.zeros(grid + (3,))
    for t in range(grid[0]):
        for h in range(grid[1]):
            for w in range(grid[2]):
                acc = 0.0
                for dt, wt in ((0, 1 - (t % 4) / 4), (1, (t % 4) / 4)):
                    for dh, wh in ((0, 1 - (h % 4) / 4), (1, (h % 4) / 4)):
                        for dw, ww in ((0, 1 - (w % 4) / 4), (1, (w % 4) / 4)):
                            acc = acc + wt * wh * ww * lat[t // 4 + dt, h // 4 + dh, w // 4 + dw]
                ref[t, h, w] = acc
    ref = ref / ref.reshape(-1, 3).std(axis=0)
    np.testing.assert_allclose(f, ref, rtol=0, atol=2e-6)
    # lattice points are the lattice values (scaled)
    np.testing.assert_allclose(f[::4, ::4, ::4], ref[::4, ::4, ::4], atol=2e-6)
