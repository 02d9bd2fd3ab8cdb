"""Aligned key-block walks of query-block groups, on constructed selections.

The attention kernel visits each query block's kept key blocks in an order
shared by the four query blocks of its group.  The order must not change the
result beyond rounding, and every kept block must be visited exactly once (a
missed or repeated tile would move the output far outside the tolerance).

The inputs are built so the selection is known in advance: key block j is a
constant row 4*e_c(j) (plus small noise) and query block i a sum of the e_c
of the blocks it should keep, so the scores are about 4 on the wanted blocks
and about 0 elsewhere.  The kept sets are chosen to need every path of the
walk scheduler: a group whose sets overlap like a triangle ({0,1}, {1,2},
{2,0}) cannot give every member one block per step without taking a shared
block for one owner at a time; a group with identical sets; a last group with
a single member; and a union of more than 512 blocks.
"""
import numpy as np
import pytest

from oracle import sla_oracle as O
from sparse_linear_attention_sagesla_amd.inputs import f32_to_bf16_bits, random_bf16

from gpu_util import assert_parity, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sla = pytest.importorskip("sparse_linear_attention_sagesla_amd")

D = 128


def _build(N, key_channel, query_sets, seed):
    """bf16 Q, K, V of one head: key block j = 4 e_{key_channel[j]}, query block
    i = sum of e_{key_channel[j]} over the blocks j in query_sets[i]; noise 0.05."""
    nb = -(-N // 64)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 31])))
    K = np.zeros((N, D), np.float32)
    Q = np.zeros((N, D), np.float32)
    for j in range(nb):
        K[64 * j:64 * (j + 1), key_channel[j]] = 4.0
    for i in range(nb):
        for ch in {key_channel[j] for j in query_sets[i]}:
            Q[64 * i:64 * (i + 1), ch] = 1.0
    K += 0.05 * rng.standard_normal(K.shape, dtype=np.float32)
    Q += 0.05 * rng.standard_normal(Q.shape, dtype=np.float32)
    V = random_bf16((N, D), seed + 1)
    return f32_to_bf16_bits(Q), f32_to_bf16_bits(K), V


def _check(Q, K, V, keep, phi, want_sets, blocks):
    N = Q.shape[0]
    q, k, v = (to_dev(x.reshape(1, 1, N, D)) for x in (Q, K, V))
    idx = sla.block_select(q, k, keep).cpu().numpy()[0, 0]
    for i in blocks:
        assert set(idx[i].tolist()) == set(want_sets[i]), f"selection of block {i}"
    out = sla.attention(q, k, v, keep, phi, torch.float32).cpu().numpy()[0, 0]
    r = O.sla_forward_head(Q, K, V, 64, keep, phi, query_blocks=blocks)
    assert_parity(out[r["rows"]], r["out"], what=f"constructed walk N={N} keep={keep:.4f} {phi}")


@pytest.mark.parametrize("phi", ["none", "elu1"])
def test_triangle_identical_and_single_member_groups(phi):
    # 9 key blocks, k = 2: group 0 needs a block split across steps, group 1
    # keeps the same blocks everywhere, group 2 has one member (ragged N)
    sets = [{0, 1}, {1, 2}, {2, 0}, {3, 4}, {5, 6}, {5, 6}, {5, 6}, {5, 6}, {7, 8}]
    N = 9 * 64 - 10
    Q, K, V = _build(N, list(range(9)), sets, seed=41)
    keep = 2 / 9
    assert O.topk_count(9, keep) == 2
    _check(Q, K, V, keep, phi, sets, list(range(9)))


@pytest.mark.parametrize("phi", ["none", "elu1"])
def test_large_union_with_triangle(phi):
    # 600 key blocks in five classes: T01 (0..109), T12 (110..219),
    # T20 (220..329), P (330..549), rest (550..599); k = 220.  Group 0 keeps
    # T01+T20, T01+T12, T12+T20 and P: a union of 550 blocks that also needs
    # splits; every other query block keeps P.
    nb = 600
    cls = [0] * 110 + [1] * 110 + [2] * 110 + [3] * 220 + [4] * 50
    T01, T12, T20 = set(range(0, 110)), set(range(110, 220)), set(range(220, 330))
    P = set(range(330, 550))
    sets = [T01 | T20, T01 | T12, T12 | T20, P] + [P] * (nb - 4)
    N = nb * 64 - 5
    Q, K, V = _build(N, cls, sets, seed=43)
    keep = 220 / 600
    assert O.topk_count(nb, keep) == 220
    _check(Q, K, V, keep, phi, sets, [0, 1, 2, 3, 4, 301, 599])


# The backward's key side walks the columns of the selection (for each key
# block, the query blocks that keep it), ordered by how many of the key
# block's group of four share each query block, so that columns of different
# lengths and owner sets that overlap like a triangle are both walked.  A
# column walk that missed or repeated a query block would move dK and dV far
# outside the backward's tolerance.

def _check_backward(Q, K, V, keep, phi, seed, tag):
    from test_gpu_backward import _check
    N = Q.shape[0]
    G = random_bf16((N, D), seed)
    q, k, v, g = (to_dev(x.reshape(1, 1, N, D)) for x in (Q, K, V, G))
    print(f"[case] column walks {tag} N={N} keep={keep:.4f} {phi}", flush=True)
    got = [x.float().cpu().numpy()[0, 0]
           for x in sla.attention_bwd(q, k, v, g, keep=keep, phi=phi, grad_dtype=torch.float32)]
    r = O.sla_backward_head(Q, K, V, G, block=64, keep=keep, phi_kind=phi)
    for x, name in zip(got, ("dq", "dk", "dv")):
        _check(f"column walks {tag} {name}", x, r[name])


@pytest.mark.parametrize("phi", ["none", "elu1"])
def test_backward_column_walks_triangle(phi):
    # columns 0, 1, 2 hold query blocks {0, 2}, {0, 1}, {1, 2}: the owner sets
    # form a triangle; columns 3..8 have lengths 0 to 4
    sets = [{0, 1}, {1, 2}, {2, 0}, {3, 4}, {5, 6}, {5, 6}, {5, 6}, {5, 6}, {7, 8}]
    N = 9 * 64 - 10
    Q, K, V = _build(N, list(range(9)), sets, seed=41)
    _check_backward(Q, K, V, 2 / 9, phi, 45, "triangle")


def test_backward_column_walks_large_union():
    # 600 query blocks keeping two of key blocks 0, 1, 2 in turn: the first
    # group's three columns of 400 query blocks each form a triangle over a
    # union of 600 (columns longer than a wave's 64 lanes take several rounds
    # of the list builder); the other columns are empty
    nb = 600
    pairs = [{0, 1}, {1, 2}, {2, 0}]
    sets = [pairs[i % 3] for i in range(nb)]
    N = nb * 64 - 7
    Q, K, V = _build(N, [0, 1, 2] + [3] * (nb - 3), sets, seed=47)
    keep = 2 / nb
    assert O.topk_count(nb, keep) == 2
    _check_backward(Q, K, V, keep, "none", 48, "large union")


def test_one_group_kernel_for_large_unions():
    # 1700 key blocks at keep 0.3 (k = 510): four groups' queues would not fit
    # the four-group kernel's LDS, so the walks come from the one-group kernel;
    # sampled query blocks cover a whole group and the ragged last one
    nb = 1700
    N = nb * 64 - 13
    Q, K, V = (random_bf16((N, D), s) for s in (61, 62, 63))
    keep = 0.3
    assert O.topk_count(nb, keep) == 510
    q, k, v = (to_dev(x.reshape(1, 1, N, D)) for x in (Q, K, V))
    print(f"[case] one-group schedule kernel N={N} keep={keep}", flush=True)
    out = sla.attention(q, k, v, keep, "elu1", torch.float32).cpu().numpy()[0, 0]
    blocks = [0, 1, 2, 3, 850, nb - 1]
    r = O.sla_forward_head(Q, K, V, 64, keep, "elu1", query_blocks=blocks)
    assert_parity(out[r["rows"]], r["out"], what=f"one-group schedule N={N}")
