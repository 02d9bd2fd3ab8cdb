"""Pins of the fp64 CPU oracle against facts that do not come from the oracle.

Each test checks the oracle against a hand-worked example, a closed form, an
invariant, a brute-force construction or a library routine, chosen so that a
plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed operand, a wrong rounding) fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import sla_oracle as O
from sparse_linear_attention_sagesla_amd.inputs import (
    WORKLOADS, f32_to_bf16_bits, make_head, random_bf16)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


# ---------------------------------------------------------------- top-k count
@pytest.mark.parametrize("nb,keep,k", [
    (32, 0.10, 4), (512, 0.10, 52), (1182, 0.10, 119), (1182, 0.05, 60),
    (1182, 0.20, 237), (1182, 1.0, 1182), (1182, 0.0, 0), (30, 0.10, 3),
    (10, 0.01, 1), (7, 0.5, 4), (1, 0.1, 1), (1182, 0.15, 178)])
def test_topk_count_values(nb, keep, k):
    assert O.topk_count(nb, keep) == k


def test_topk_count_is_smallest_count_reaching_keep():
    for nb in (1, 2, 3, 7, 30, 32, 512, 1182):
        for keep in np.linspace(0.001, 0.999, 97):
            k = O.topk_count(nb, float(keep))
            assert 1 <= k <= nb
            assert k / nb >= keep - 1e-9
            assert k == 1 or (k - 1) / nb < keep - 1e-12


# ------------------------------------------------------- hand-worked example
def test_golden_two_block_example():
    g = json.load(open(os.path.join(GOLDEN, "two_block_example.json")))
    q, k, v = bf(g["Q"]), bf(g["K"]), bf(g["V"])
    r = O.sla_forward_head(q, k, v, block=g["block"], keep=g["keep"], phi_kind=g["phi"])
    assert r["idx"].tolist() == g["idx"]
    assert r["mu"].tolist() == g["mu"]
    assert r["q8"].tolist() == g["q8"]
    assert r["k8"].tolist() == g["k8"]
    den = np.float32(g["scale_den"])
    assert r["q_scale"].tolist() == [np.float32(a) / den for a in g["q_scale_num"]]
    assert r["k_scale"].tolist() == [np.float32(a) / den for a in g["k_scale_num"]]
    want = np.array([[float(Fraction(x)) for x in row] for row in g["out"]])
    want_s = np.array([[float(Fraction(x)) for x in row] for row in g["out_softmax"]])
    np.testing.assert_allclose(r["out"], want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["out_softmax"], want_s, rtol=0, atol=1e-12)


def test_zero_queries_tie_to_lowest_blocks_and_uniform_softmax():
    """Q = 0: every score ties at 0, so blocks 0..k-1 are kept; the INT8 logits
    are all 0, so the softmax branch is the plain mean of the kept values; phi(0)=1
    makes the linear weights the channel sums of phi(k)."""
    N, d, blk = 256, 128, 64
    q = bf(np.zeros((N, d)))
    k = random_bf16((N, d), 11)
    v = random_bf16((N, d), 12)
    r = O.sla_forward_head(q, k, v, block=blk, keep=0.5, phi_kind="elu1")
    assert (r["idx"] == np.array([[0, 1]] * 4)).all()
    v64 = O.bf16_to_f64(v)
    k64 = O.bf16_to_f64(k)
    np.testing.assert_allclose(r["out_softmax"], np.tile(v64[:128].mean(0), (N, 1)), atol=1e-13)
    w = np.where(k64[128:] > 0, k64[128:] + 1, np.exp(np.minimum(k64[128:], 0))).sum(1)
    lin = (w[:, None] * v64[128:]).sum(0) / w.sum()
    np.testing.assert_allclose(r["out_linear"], np.tile(lin, (N, 1)), atol=1e-12)


# ----------------------------------------------------------------- quantiser
def test_quantizer_round_half_even_and_extremes():
    x = np.zeros((64, 128), np.float32)
    x[0, :8] = [127, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, -127]
    x[1, 0] = 126.5
    codes, sc = O.quantize_blocks(x, 64)
    assert sc[0] == np.float32(1.0)
    assert codes[0, :8].tolist() == [127, 2, 4, -2, 0, 2, 0, -127]
    assert codes[1, 0] == 126


def test_quantizer_bounds_zero_block_and_pad_rows():
    x = O.bf16_to_f32(random_bf16((150, 128), 3, scale=3.0))
    x[64:128] = 0.0
    codes, sc = O.quantize_blocks(x, 64)
    assert codes.shape == (192, 128)
    assert sc[1] == 0 and not codes[64:128].any()
    assert not codes[150:].any()
    for i in (0, 2):
        blk = x[i * 64:min(150, (i + 1) * 64)]
        c = codes[i * 64:i * 64 + blk.shape[0]].astype(np.float64)
        a = np.abs(blk).max()
        assert sc[i] == np.float32(a) / np.float32(127)
        assert np.abs(c).max() == 127
        at = np.unravel_index(np.abs(blk).argmax(), blk.shape)
        assert abs(c[at]) == 127
        err = np.abs(c * float(sc[i]) - blk.astype(np.float64))
        assert err.max() <= 0.5 * float(sc[i]) * (1 + 1e-5)


def test_key_mean_is_correctly_rounded_sum():
    wl = WORKLOADS["wan13b480"]
    _, k, _ = make_head(wl, 0, 0)
    mu = O.key_channel_mean(k, 64)
    k64 = O.bf16_to_f64(k)
    for c in range(0, 128, 9):
        exact = Fraction(math.fsum(k64[:, c].tolist())) / k64.shape[0]
        assert mu[c] == np.float32(float(exact))


def test_pooled_means_are_correctly_rounded_block_sums():
    _, k, _ = make_head(WORKLOADS["tiny"], 0, 1)
    kb = O.pooled_means(k[:2000], 64)           # ragged last block of 16 rows
    k64 = O.bf16_to_f64(k[:2000])
    assert kb.shape == (32, 128)
    for i in (0, 5, 31):
        rows = k64[i * 64:min(2000, (i + 1) * 64)]
        for c in (0, 63, 127):
            exact = Fraction(math.fsum(rows[:, c].tolist())) / rows.shape[0]
            assert kb[i, c] == np.float32(float(exact))


def test_int8_accumulator_matches_integer_loop():
    q, k, _ = make_head(WORKLOADS["tiny"], 0, 0)
    q8, k8, *_ = O.quantize_qk(q[:256], k[:256], 64)
    acc = O.qk_accumulator(q8, k8, 1, 3, 64)
    a = q8[64:128].astype(np.int64)
    b = k8[192:256].astype(np.int64)
    for r in (0, 17, 63):
        for c in (0, 40, 63):
            assert acc[r, c] == sum(int(a[r, t]) * int(b[c, t]) for t in range(128))
    assert np.abs(acc).max() <= 128 * 127 * 127


# ------------------------------------------------------------ scores, top-k
def test_block_scores_within_rounding_of_exact_dot():
    rng = np.random.default_rng(5)
    qb = rng.standard_normal((6, 128)).astype(np.float32)
    kb = rng.standard_normal((9, 128)).astype(np.float32)
    s = O.block_scores(qb, kb)
    for i in range(6):
        for j in range(9):
            prods = [float(qb[i, c]) * float(kb[j, c]) for c in range(128)]
            exact = math.fsum(prods)
            bound = 128 * 2.0 ** -53 * sum(abs(p) for p in prods)
            assert abs(s[i, j] - exact) <= bound
    # sign / transpose check against an independent fp64 product
    np.testing.assert_allclose(s, qb.astype(np.float64) @ kb.astype(np.float64).T, rtol=1e-12)


def test_selection_brute_force_rank_and_ties():
    rng = np.random.default_rng(7)
    s = rng.integers(-3, 4, size=(20, 30)).astype(np.float64)   # many exact ties
    for k in (1, 3, 10, 30):
        idx = O.select_blocks(s, k)
        assert idx.shape == (20, k)
        for i in range(20):
            want = [j for j in range(30)
                    if sum(1 for jj in range(30)
                           if s[i, jj] > s[i, j] or (s[i, jj] == s[i, j] and jj < j)) < k]
            assert idx[i].tolist() == want


def test_duplicated_key_blocks_keep_lower_index():
    N, blk = 512, 64
    q = random_bf16((N, 128), 21, offset=0.5)
    k = random_bf16((N, 128), 22)
    k[64:128] = bf(4.0 * O.bf16_to_f32(q[0:64]))   # key block 1 aligned with query block 0
    k[256:320] = k[64:128]                         # key block 4 duplicates key block 1 exactly
    idx, s = O.select_head(q, k, blk, keep=1 / 8)  # k = 1
    assert (s[:, 1] == s[:, 4]).all()
    assert s[0, 1] == s[0].max()
    assert idx[0].tolist() == [1]
    idx2, _ = O.select_head(q, k, blk, keep=2 / 8)
    assert 1 in idx2[0] and 4 in idx2[0]


# ------------------------------------------------- special cases of the method
def _dense_softmax(q64, k64, v64):
    d = q64.shape[1]
    out = np.empty_like(q64)
    for t in range(q64.shape[0]):
        lg = np.array([sum(q64[t, c] * k64[u, c] for c in range(d)) for u in range(k64.shape[0])]) / math.sqrt(d)
        w = np.exp(lg - lg.max())
        out[t] = (w[:, None] * v64).sum(0) / w.sum()
    return out


def test_keep_all_without_quantisation_is_dense_attention():
    N = 96
    q, k, v = (random_bf16((N, 128), s) for s in (31, 32, 33))
    r = O.sla_forward_head(q, k, v, block=64, keep=1.0, phi_kind="none", quantize=False)
    q64, k64, v64 = (O.bf16_to_f64(x) for x in (q, k, v))
    np.testing.assert_allclose(r["out"], _dense_softmax(q64, k64, v64), atol=1e-12)
    torch = pytest.importorskip("torch")
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q64)[None], torch.from_numpy(k64)[None], torch.from_numpy(v64)[None])[0]
    np.testing.assert_allclose(r["out"], ref.numpy(), atol=1e-12)


def test_keep_all_quantised_is_dense_attention_on_dequantised_inputs():
    N = 200
    q, k, v = (random_bf16((N, 128), s, scale=2.0) for s in (41, 42, 43))
    r = O.sla_forward_head(q, k, v, block=64, keep=1.0, phi_kind="none")
    blocks = np.arange(N) // 64
    qh = r["q8"][:N].astype(np.float64) * r["q_scale"][blocks][:, None]
    kh = r["k8"][:N].astype(np.float64) * r["k_scale"][blocks][:, None]
    want = _dense_softmax(qh, kh, O.bf16_to_f64(v))
    np.testing.assert_allclose(r["out"], want, atol=1e-12)


def _brute_linear(q64, k64, v64, phi_kind, mask=None):
    fq, fk = O.phi(q64, phi_kind), O.phi(k64, phi_kind)
    W = fq @ fk.T
    if mask is not None:
        W = W * mask
    den = W.sum(1, keepdims=True)
    out = np.zeros_like(q64)
    ok = den[:, 0] != 0
    out[ok] = (W @ v64)[ok] / den[ok]
    return out


@pytest.mark.parametrize("phi_kind", ["elu1", "relu"])
def test_keep_zero_is_pure_linear_attention(phi_kind):
    N = 130
    q, k, v = (random_bf16((N, 128), s) for s in (51, 52, 53))
    r = O.sla_forward_head(q, k, v, block=64, keep=0.0, phi_kind=phi_kind)
    want = _brute_linear(*(O.bf16_to_f64(x) for x in (q, k, v)), phi_kind)
    np.testing.assert_allclose(r["out"], want, atol=1e-12)
    assert not r["out_softmax"].any()


def test_branch_decomposition_matches_token_level_construction():
    """Random block mask on a tiny head: the oracle's blockwise sum equals an
    explicit N x N construction (masked softmax on dequantised logits plus the
    complement-masked, row-normalised kernel attention)."""
    N, blk = 300, 64
    nb = O.n_blocks(N, blk)
    q, k, v = (random_bf16((N, 128), s) for s in (61, 62, 63))
    rng = np.random.default_rng(64)
    idx = np.sort(np.stack([rng.choice(nb, 2, replace=False) for _ in range(nb)]), axis=1)
    r = O.sla_forward_head(q, k, v, block=blk, keep=2 / nb, phi_kind="elu1", idx=idx)
    qb = np.arange(N) // blk
    M = np.zeros((N, N), bool)
    for i in range(nb):
        for j in idx[i]:
            M[np.ix_(qb == i, qb == j)] = True
    qh = r["q8"][:N].astype(np.float64) * r["q_scale"][qb][:, None]
    kh = r["k8"][:N].astype(np.float64) * r["k_scale"][qb][:, None]
    lg = np.where(M, qh @ kh.T / math.sqrt(128), -np.inf)
    p = np.exp(lg - lg.max(1, keepdims=True))
    v64 = O.bf16_to_f64(v)
    soft = (p @ v64) / p.sum(1, keepdims=True)
    lin = _brute_linear(O.bf16_to_f64(q), O.bf16_to_f64(k), v64, "elu1", mask=~M)
    np.testing.assert_allclose(r["out_softmax"], soft, atol=1e-12)
    np.testing.assert_allclose(r["out_linear"], lin, atol=1e-12)
    np.testing.assert_allclose(r["out"], soft + lin, atol=1e-12)


def _complement_average(q64, k64, v64, phi_kind, unsel_rows, t):
    """Token-level normalised linear attention of query t over the rows
    ``unsel_rows``: a loop over the keys, each weight phi(q_t) . phi(k_u)."""
    fq = O.phi(q64[t], phi_kind)
    num = np.zeros(v64.shape[1])
    den = 0.0
    for u in unsel_rows:
        w = float(np.dot(fq, O.phi(k64[u], phi_kind)))
        num += w * v64[u]
        den += w
    return num, den


def test_linear_rule_zero_denominator_relu():
    """Reading R12 (normalised linear attention [TUT §2.1], zero when the
    denominator vanishes).  A ReLU row whose every weight phi(q).phi(k_u)
    over the unselected keys is zero, while those keys exist, gets O_l = 0
    exactly, and its output is the softmax branch alone; other rows get the
    token-level weighted average.  Built by sign structure, not by the
    oracle's own denominator: rows 0-31 have phi(q) = 0 (every entry < 0),
    rows 32-63 have features only on channels 0-7, where every unselected
    key has phi(k) = 0."""
    N, blk = 256, 64
    rng = np.random.default_rng(7)
    pos = lambda shape: rng.uniform(0.25, 2.0, shape)
    q = pos((N, 128))
    q[0:32] *= -1.0
    q[32:64, 8:] *= -1.0
    k = pos((N, 128))
    for j in (0, 2):                                   # unselected blocks
        k[j * blk:(j + 1) * blk, :8] *= -1.0
    v = rng.standard_normal((N, 128)) + 1.0
    qb, kb, vb = bf(q), bf(k), bf(v)
    idx = np.array([[1, 3]] * 4, dtype=np.int32)       # every query block keeps 1 and 3
    r = O.sla_forward_head(qb, kb, vb, block=blk, keep=0.5, phi_kind="relu", idx=idx)
    q64, k64, v64 = (O.bf16_to_f64(x) for x in (qb, kb, vb))
    unsel = np.r_[0:64, 128:192]
    assert (r["out_linear"][:64] == 0.0).all()
    np.testing.assert_array_equal(r["out"][:64], r["out_softmax"][:64])
    for t in list(range(0, 64, 9)):
        num, den = _complement_average(q64, k64, v64, "relu", unsel, t)
        assert den == 0.0 and not num.any()
    for t in list(range(64, N, 17)):
        num, den = _complement_average(q64, k64, v64, "relu", unsel, t)
        assert den > 0.0
        np.testing.assert_allclose(r["out_linear"][t], num / den, rtol=1e-12, atol=1e-12)


def test_linear_rule_elu1_never_zero_and_empty_complement():
    """elu+1 features are positive, so no row of a non-empty complement has a
    zero denominator, even with large negative entries (weights near e^-60);
    with every block kept the complement is empty, the linear branch is 0 and
    the output is dense softmax attention on the INT8 logits."""
    N, blk = 192, 64
    rng = np.random.default_rng(8)
    q = rng.uniform(-30.0, -20.0, (N, 128))
    k = rng.uniform(-30.0, -20.0, (N, 128))
    v = rng.standard_normal((N, 128))
    qb, kb, vb = bf(q), bf(k), bf(v)
    idx = np.array([[0]] * 3, dtype=np.int32)
    r = O.sla_forward_head(qb, kb, vb, block=blk, keep=1 / 3, phi_kind="elu1", idx=idx)
    q64, k64, v64 = (O.bf16_to_f64(x) for x in (qb, kb, vb))
    for t in (0, 70, 191):
        num, den = _complement_average(q64, k64, v64, "elu1", np.arange(64, N), t)
        assert den > 0.0
        np.testing.assert_allclose(r["out_linear"][t], num / den, rtol=1e-9, atol=1e-12)
    full = O.sla_forward_head(qb, kb, vb, block=blk, keep=1.0, phi_kind="elu1")
    assert not full["out_linear"].any()
    bq = np.arange(N) // blk
    qh = full["q8"][:N].astype(np.float64) * full["q_scale"][bq][:, None]
    kh = full["k8"][:N].astype(np.float64) * full["k_scale"][bq][:, None]
    lg = qh @ kh.T / math.sqrt(128)
    p = np.exp(lg - lg.max(1, keepdims=True))
    np.testing.assert_allclose(full["out"], (p @ v64) / p.sum(1, keepdims=True), atol=1e-12)


def test_single_token_returns_its_value():
    q, k, v = (random_bf16((1, 128), s) for s in (71, 72, 73))
    for keep, ph in ((1.0, "none"), (1.0, "elu1"), (0.5, "elu1")):
        r = O.sla_forward_head(q, k, v, block=64, keep=keep, phi_kind=ph)
        np.testing.assert_allclose(r["out"][0], O.bf16_to_f64(v)[0], atol=1e-14)


def test_value_scaling_and_shift_invariants():
    N = 320
    q, k, v = (random_bf16((N, 128), s) for s in (81, 82, 83))
    v = bf(np.clip(np.round(O.bf16_to_f32(v) * 4) / 4, -3, 3))   # quarter grid: shifts stay exact
    base = O.sla_forward_head(q, k, v, block=64, keep=0.4, phi_kind="elu1")
    v2 = bf(2.0 * O.bf16_to_f32(v))                       # exact in bf16
    r2 = O.sla_forward_head(q, k, v2, block=64, keep=0.4, phi_kind="elu1")
    np.testing.assert_allclose(r2["out"], 2.0 * base["out"], atol=1e-12)
    c = np.zeros(128, np.float32)
    c[:4] = [1.0, -2.0, 0.5, 4.0]
    v3 = bf(O.bf16_to_f32(v) + c)
    assert (O.bf16_to_f32(v3) == O.bf16_to_f32(v) + c).all()
    r3 = O.sla_forward_head(q, k, v3, block=64, keep=0.4, phi_kind="elu1")
    # each branch is a weighted average of values, so a constant shift adds once per branch
    np.testing.assert_allclose(r3["out"], base["out"] + 2.0 * c, atol=1e-12)
    r4 = O.sla_forward_head(q, k, v3, block=64, keep=1.0, phi_kind="none")
    r5 = O.sla_forward_head(q, k, v, block=64, keep=1.0, phi_kind="none")
    np.testing.assert_allclose(r4["out"], r5["out"] + c, atol=1e-12)


def test_smoothing_changes_only_codes_not_the_selection():
    wl = WORKLOADS["sweep"]
    q, k, v = make_head(wl, 0, 0)
    N = 64 * 24
    q, k, v = q[:N], k[:N], v[:N]
    a = O.sla_forward_head(q, k, v, keep=1.0, phi_kind="none")
    b = O.sla_forward_head(q, k, v, keep=1.0, phi_kind="none", smooth=False)
    exact = O.sla_forward_head(q, k, v, keep=1.0, phi_kind="none", quantize=False)["out"]
    ea = np.linalg.norm(a["out"] - exact) / np.linalg.norm(exact)
    eb = np.linalg.norm(b["out"] - exact) / np.linalg.norm(exact)
    # K smoothing removes the +8 outlier offset before quantising, which must
    # make the INT8 attention closer to exact attention
    assert ea < eb
    print(f"rel-L2 vs exact dense: smoothed {ea:.3e}  unsmoothed {eb:.3e}")


def test_generators_are_seeded_and_shaped():
    a = make_head(WORKLOADS["tiny"], 0, 1)
    b = make_head(WORKLOADS["tiny"], 0, 1)
    c = make_head(WORKLOADS["tiny"], 0, 0)
    assert all((x == y).all() for x, y in zip(a, b))
    assert not (a[0] == c[0]).all()
    assert a[0].shape == (2048, 128) and a[0].dtype == np.uint16


# ----------------------------------------------------- lower-bit option (FP8)
def test_e4m3_rounding_against_the_format():
    """e4m3 (OCP FP8: bias 7, 3 mantissa bits, subnormals (m/8) 2^-6, largest
    448): representable values map to themselves; midpoints go to the even
    mantissa; subnormal spacing is 2^-9."""
    vals = sorted({(m / 8) * 2.0 ** -6 for m in range(8)} |
                  {(1 + m / 8) * 2.0 ** (e - 7) for e in range(1, 16) for m in range(8)
                   if not (e == 15 and m == 7)})
    assert vals[-1] == 448.0 and len(vals) == 8 + 15 * 8 - 1
    np.testing.assert_array_equal(O.round_e4m3(np.array(vals)), vals)
    cases = {1.0625: 1.0, 1.1875: 1.25, 3.0 * 2.0 ** -10: 2.0 ** -8, 2.0 ** -10: 0.0,
             2.0 ** -9: 2.0 ** -9, 100.0: 96.0, 104.0: 104.0, 108.0: 112.0, 250.0: 256.0,
             0.3: 0.3125, 0.0: 0.0}
    for x, want in cases.items():
        assert O.round_e4m3(np.array([x]))[0] == want, x
    rng = np.random.default_rng(3)
    x = rng.uniform(2.0 ** -6, 448.0, 20000)
    r = O.round_e4m3(x)
    assert (np.abs(r - x) <= 2.0 ** -4 * x + 1e-300).all()       # half of 2^-3 relative
    assert (np.diff(O.round_e4m3(np.sort(x))) >= 0).all()         # monotone


def test_phi_k_fp8_block_scale():
    """Per-block power-of-two scale: the block's largest feature lands in
    [128, 256) before rounding, so features within a factor 2^-4 of it keep
    three mantissa bits; features already on the scaled e4m3 grid are kept."""
    fk = np.zeros((130, 4))
    fk[0:64] = np.array([[300.0, 0.5, 1.0, 37.0]])        # block max 300 -> scale 2^-1
    fk[64:128] = np.array([[1e-3, 2e-3, 3e-3, 5e-3]])     # block max 5e-3 -> scale 2^15
    fk[128:] = 0.0                                         # all-zero block stays zero
    r = O.phi_k_e4m3_blocks(fk, 64)
    np.testing.assert_array_equal(r[0], [288.0, 0.5, 1.0, 36.0])   # 150 -> 144 (spacing 16)
    s = 2.0 ** 15
    np.testing.assert_array_equal(r[64], O.round_e4m3(fk[64] * s) / s)
    assert 128 <= fk[64].max() * s < 256
    assert not r[128:].any()


def test_phi_k_fp8_equals_exact_mode_on_grid_inputs():
    """With ReLU features already on each block's scaled e4m3 grid, the
    lower-bit option is the exact forward, and in general its linear branch is
    still a weighted average of the values (inside their range per channel)."""
    N = 192
    rng = np.random.default_rng(4)
    q = rng.integers(-3, 6, (N, 128)).astype(np.float64) / 4
    k = rng.integers(-3, 8, (N, 128)).astype(np.float64) / 8   # max 7/8 -> 3 bits suffice
    v = rng.standard_normal((N, 128))
    qb, kb, vb = bf(q), bf(k), bf(v)
    a = O.sla_forward_head(qb, kb, vb, 64, 1 / 3, "relu")
    b = O.sla_forward_head(qb, kb, vb, 64, 1 / 3, "relu", phi_k_fp8=True)
    np.testing.assert_allclose(b["out"], a["out"], rtol=0, atol=1e-12)
    kg = bf(rng.standard_normal((N, 128)) * 2)
    c = O.sla_forward_head(qb, kg, vb, 64, 1 / 3, "elu1", phi_k_fp8=True)
    e = O.sla_forward_head(qb, kg, vb, 64, 1 / 3, "elu1")
    v64 = O.bf16_to_f64(vb)
    assert (c["out_linear"] <= v64.max(0) + 1e-12).all() and (c["out_linear"] >= v64.min(0) - 1e-12).all()
    assert 0 < np.abs(c["out_linear"] - e["out_linear"]).max() < 0.1
