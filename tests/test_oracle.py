"""Pins for the CPU oracle: each check comes from outside the oracle itself.

Pins used: hand-worked examples (tests/golden), closed forms (the per-bit
logistic factorisation of the bucket softmax), limits (tau -> 0 gives the
hard bucket, tau -> infinity the uniform table, large tau the linear
small-signal regime), invariants (sums, bounds, symmetries), the SimHash
collision law for random hyperplanes, a library routine (torch's
scaled_dot_product_attention in float64 for k = N) and an independent
pure-Python brute force with exact rational arithmetic on tiny inputs.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _bf16_values(x):
    """Round float64 samples to bfloat16 values (returned as float64)."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(
        torch.bfloat16).to(torch.float64).numpy()


# --------------------------------------------------------------------- hash

def test_hash_golden(golden_dir):
    g = _load(golden_dir, "hash_hand.json")
    for case in g["cases"]:
        ids = O.hash_keys(np.array(case["K"], float), np.array(case["R"], float),
                          case["L"], case["P"])
        assert ids.tolist() == case["ids"]


def _exact_sign_bits(K, R):
    K = np.asarray(K)
    R = np.asarray(R)
    out = np.zeros((K.shape[0], R.shape[1]), dtype=bool)
    for n in range(K.shape[0]):
        for c in range(R.shape[1]):
            s = sum((Fraction(float(K[n, i])) * Fraction(float(R[i, c]))
                     for i in range(K.shape[1])), Fraction(0))
            out[n, c] = s > 0
    return out


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_hash_bits_match_exact_rationals(kind):
    r = _rng(1)
    K = r.standard_normal((40, 16)).astype(np.float32).astype(np.float64)
    R = r.standard_normal((16, 12)).astype(np.float32).astype(np.float64)
    if kind == "bf16":
        K, R = _bf16_values(K), _bf16_values(R)
    # a few rows built to project to exactly zero or almost zero
    K[0] = 0.0
    K[1, :] = 0.0
    K[1, 0], K[1, 1] = R[1, 0], -R[0, 0]   # exact cancellation on column 0
    assert np.array_equal(O.hash_bits(K, R), _exact_sign_bits(K, R))


def test_hash_certified_sign_beats_naive_float64():
    # Exact projection is 2^-10 > 0, but a left-to-right float64 sum gives 0.
    K = np.array([[2.0 ** 60, 2.0 ** -10, -(2.0 ** 60), 0.0]])
    R = np.ones((4, 1))
    naive = ((K[0, 0] + K[0, 1]) + K[0, 2]) + K[0, 3]
    assert naive == 0.0
    assert O.hash_bits(K, R)[0, 0]
    assert not O.hash_bits(-K, R)[0, 0]
    assert not O.hash_bits(np.zeros((1, 4)), R)[0, 0]


def test_hash_symmetries():
    r = _rng(2)
    K = r.standard_normal((64, 32))
    R = r.standard_normal((32, 24))
    L, P = 4, 6
    ids = O.hash_keys(K, R, L, P)
    # positive power-of-two scaling is exact and keeps every sign
    assert np.array_equal(O.hash_keys(K * 2.0 ** 7, R, L, P), ids)
    assert np.array_equal(O.hash_keys(K, R * 2.0 ** -5, L, P), ids)
    # negating a key flips every (non-zero) projection: complement bucket
    assert np.array_equal(O.hash_keys(-K, R, L, P), (2 ** P - 1) - ids)


def test_simhash_collision_law():
    """One random hyperplane separates two vectors at angle theta with
    probability theta/pi (Goemans-Williamson / Charikar SimHash), so the bits
    agree with probability 1 - theta/pi and a P-bit bucket id matches with
    probability (1 - theta/pi)^P."""
    r = _rng(3)
    d = 32
    x = r.standard_normal(d)
    x /= np.linalg.norm(x)
    w = r.standard_normal(d)
    w -= (w @ x) * x
    w /= np.linalg.norm(w)
    for theta in (0.3, 1.0, 2.0):
        y = math.cos(theta) * x + math.sin(theta) * w
        for P in (1, 3):
            L = 6000
            R = r.standard_normal((d, L * P))
            ids = O.hash_keys(np.stack([x, y]), R, L, P)
            frac = float(np.mean(ids[0] == ids[1]))
            expect = (1 - theta / math.pi) ** P
            sigma = math.sqrt(expect * (1 - expect) / L)
            assert abs(frac - expect) < 5 * sigma + 1e-3, (theta, P, frac, expect)


def test_value_norms():
    V = np.array([[3.0, 4.0, 0.0], [0.0, 0.0, 0.0], [1.0, 1.0, 1.0]])
    assert np.allclose(O.value_norms(V), [5.0, 0.0, math.sqrt(3.0)], rtol=0, atol=1e-15)
    r = _rng(4)
    V = r.standard_normal((3, 50, 16))
    assert np.allclose(O.value_norms(V), np.linalg.norm(V, axis=-1), rtol=1e-14)


# ----------------------------------------------------------- soft assignment

def test_soft_assignment_golden(golden_dir):
    g = _load(golden_dir, "soft_assignment_hand.json")
    tol = g["tolerance"]
    for c in g["cases"]:
        Q = np.array(c["Q"], float)[None, None, :]
        R = np.array(c["R"], float)
        p = O.soft_bucket_probs(Q, R, c["L"], c["P"], c["tau"])
        assert np.allclose(p[0, 0, 0], c["probs"], atol=tol, rtol=0)
        key = np.array(c["key"], float)[None, None, None, :]
        ids = O.hash_keys(key, R, c["L"], c["P"])
        assert int(ids[0, 0, 0, 0]) == c["key_bucket"]
        vn = O.value_norms(np.array(c["value"], float)[None, None, None, :])
        s = O.soft_scores(p, ids, vn, 1)
        assert abs(s[0, 0, 0] - c["score"]) < tol


@pytest.mark.parametrize("P,tau", [(1, 0.7), (4, 0.5), (6, 0.2), (8, 0.3), (8, 3.0)])
def test_soft_probs_sum_and_logistic_factorisation(P, tau):
    r = _rng(10 + P)
    L, d = 5, 24
    Q = r.standard_normal((2, 3, d)) * 0.3
    R = r.standard_normal((d, L * P))
    p = O.soft_bucket_probs(Q, R, L, P, tau)
    assert np.allclose(p.sum(-1), 1.0, rtol=0, atol=1e-12)
    # closed form: p(u) = prod_j sigmoid(2 s_j(u) z_j / tau)
    z = (Q @ R).reshape(2, 3, L, P)
    u = np.arange(2 ** P)
    closed = np.ones((2, 3, L, 2 ** P))
    for j in range(P):
        s = np.where((u >> j) & 1, 1.0, -1.0)
        closed *= 1.0 / (1.0 + np.exp(-2.0 * s[None, None, None, :] * z[..., j:j + 1] / tau))
    assert np.allclose(p, closed, rtol=1e-12, atol=1e-300)


def test_soft_probs_tau_limits_and_linear_regime():
    r = _rng(20)
    L, P, d = 7, 5, 16
    Q = r.standard_normal((1, 2, d))
    R = r.standard_normal((d, L * P))
    z = (Q @ R).reshape(1, 2, L, P)
    assert np.abs(z).min() > 1e-4
    # tau -> 0: one-hot on the hard bucket of the query (Theorem 3 limit)
    p0 = O.soft_bucket_probs(Q, R, L, P, 1e-6)
    hard = O.hard_query_buckets(Q, R, L, P)
    onehot = np.zeros_like(p0)
    np.put_along_axis(onehot, hard[..., None], 1.0, axis=-1)
    assert np.allclose(p0, onehot, atol=1e-12, rtol=0)
    # tau -> infinity: uniform table
    pinf = O.soft_bucket_probs(Q, R, L, P, 1e30)
    assert np.array_equal(pinf, np.full_like(pinf, 2.0 ** -P))
    # large tau: (2^P p(u) - 1) tau -> sum_j s_j(u) z_j (small-signal regime)
    S = O.bucket_signs(P)
    lin = z @ S.T
    for tau in (1e3, 1e4):
        p = O.soft_bucket_probs(Q, R, L, P, tau)
        approx = (2 ** P * p - 1.0) * tau
        assert np.max(np.abs(approx - lin)) < 50.0 * np.abs(z).sum(-1).max() ** 2 / tau


def test_soft_probs_query_negation_maps_to_complement_bucket():
    r = _rng(21)
    L, P, d = 3, 4, 8
    Q = r.standard_normal((1, 1, d))
    R = r.standard_normal((d, L * P))
    p = O.soft_bucket_probs(Q, R, L, P, 0.4)
    pn = O.soft_bucket_probs(-Q, R, L, P, 0.4)
    comp = (2 ** P - 1) - np.arange(2 ** P)
    assert np.allclose(pn, p[..., comp], rtol=1e-13, atol=1e-300)


def test_hard_table_golden(golden_dir):
    """Hand-worked tau -> 0 tables, including projections of exactly 0."""
    g = _load(golden_dir, "hard_table_hand.json")
    for case in g["cases"]:
        Q = np.array(case["Q"], float)[None, None, :]
        R = np.eye(Q.shape[-1])
        t = O.hard_bucket_table(Q, R, case["L"], case["P"])[0, 0]
        assert t.tolist() == case["table"]
        if "key" in case:
            K = np.array(case["key"], float)[None, None, None, :]
            V = np.array(case["value"], float)[None, None, None, :]
            ids = O.hash_keys(K, R, case["L"], case["P"])
            s = O.soft_scores(t[None, None], ids, O.value_norms(V), 1)
            assert s[0, 0, 0] == case["score"]


def _with_zero_projections(seed, d=16, L=6, P=4):
    """Queries with some projections exactly 0 (pairs of coordinates that
    cancel exactly: q_2m = r_2m+1, q_2m+1 = -r_2m for the chosen column),
    the other projections at least 1e-3 away from 0."""
    r = _rng(seed)
    R = np.round(r.standard_normal((d, L * P)) * 64) / 64      # exact products
    while True:
        Q = np.round(r.standard_normal((2, 3, d)) * 64) / 64
        for (b, h, c) in [(0, 0, 1), (0, 2, 5), (1, 1, 9), (1, 2, 9 + P)]:
            Q[b, h, 0::2] = R[1::2, c]
            Q[b, h, 1::2] = -R[0::2, c]
        z = Q @ R
        nz = np.abs(z[z != 0])
        if nz.min() > 1e-3:
            return Q, R, L, P, z


def test_hard_table_is_the_tau0_limit_of_the_soft_table():
    """A different route: the literal softmax of soft_bucket_probs at a tiny
    tau, with exact-zero projections present (their bit splits 1/2 : 1/2)."""
    Q, R, L, P, z = _with_zero_projections(50)
    assert (z == 0).sum() == 4
    hard = O.hard_bucket_table(Q, R, L, P)
    soft = O.soft_bucket_probs(Q, R, L, P, 1e-9)
    assert np.allclose(hard, soft, atol=1e-12, rtol=0)
    assert np.array_equal(hard.sum(-1), np.ones(hard.shape[:-1]))
    # the tables holding a zero projection split their mass over 2 buckets
    zt = (z.reshape(2, 3, L, P) == 0).any(-1)
    assert np.array_equal((hard > 0).sum(-1), np.where(zt, 2, 1))


def test_hard_table_without_zeros_is_one_hot_at_the_hard_bucket():
    r = _rng(51)
    L, P, d = 9, 6, 32
    Q = r.standard_normal((2, 4, d))
    R = r.standard_normal((d, L * P))
    hard = O.hard_bucket_table(Q, R, L, P)
    onehot = np.zeros_like(hard)
    np.put_along_axis(onehot, O.hard_query_buckets(Q, R, L, P)[..., None], 1.0, axis=-1)
    assert np.array_equal(hard, onehot)


# -------------------------------------------------------------------- scores

def _small_problem(seed, B=2, Hq=4, Hkv=2, d=16, N=50, L=6, P=3, tau=0.5):
    r = _rng(seed)
    Q = r.standard_normal((B, Hq, d))
    K = r.standard_normal((B, Hkv, N, d))
    V = r.standard_normal((B, Hkv, N, d))
    R = r.standard_normal((d, L * P))
    return Q, K, V, R, L, P, tau


def test_scores_bounds_and_tau0_hard_collisions():
    Q, K, V, R, L, P, tau = _small_problem(30)
    G = Q.shape[1] // K.shape[1]
    ids = O.hash_keys(K, R, L, P)
    vn = O.value_norms(V)
    s = O.soft_scores(O.soft_bucket_probs(Q, R, L, P, tau), ids, vn, G)
    for h in range(Q.shape[1]):
        assert np.all(s[:, h] >= 0)
        assert np.all(s[:, h] <= L * vn[:, h // G] * (1 + 1e-12))
    # tau -> 0: value norm times the number of tables whose hard bucket
    # equals the query's own hard bucket (computed here from sign vectors)
    z = (Q @ R).reshape(*Q.shape[:2], L, P)
    assert np.abs(z).min() > 1e-4
    s0 = O.soft_scores(O.soft_bucket_probs(Q, R, L, P, 1e-6), ids, vn, G)
    kbits = (K @ R > 0).reshape(*K.shape[:3], L, P)
    for b in range(Q.shape[0]):
        for h in range(Q.shape[1]):
            g = h // G
            same = np.all(kbits[b, g] == (z[b, h] > 0)[None, :, :], axis=-1)
            count = same.sum(-1)
            assert np.allclose(s0[b, h], vn[b, g] * count, atol=1e-12, rtol=0)


def test_scores_uniform_table_ranks_by_value_norm():
    Q, K, V, R, L, P, _ = _small_problem(31)
    ids = O.hash_keys(K, R, L, P)
    vn = O.value_norms(V)
    s = O.soft_scores(O.soft_bucket_probs(Q, R, L, P, 1e30), ids, vn, 2)
    for h in range(4):
        assert np.allclose(s[:, h], L * 2.0 ** -P * vn[:, h // 2], rtol=1e-15, atol=0)


def test_scores_gqa_uses_floor_h_over_g():
    Q, K, V, R, L, P, tau = _small_problem(32, B=1, Hq=6, Hkv=3)
    ids = O.hash_keys(K, R, L, P)
    vn = O.value_norms(V)
    vn[0, 1] *= 1000.0   # KV head 1 serves query heads 2 and 3 only
    s = O.soft_scores(O.soft_bucket_probs(Q, R, L, P, tau), ids, vn, 2)
    big = s.max(-1)[0]
    assert big[2] > 50 * max(big[0], big[1], big[4], big[5])
    assert big[3] > 50 * max(big[0], big[1], big[4], big[5])


def test_group_scores_reduce_to_soft_scores_and_sum_the_group():
    # G = 1: the group score is the head's own soft score
    Q, K, V, R, L, P, tau = _small_problem(33, B=1, Hq=3, Hkv=3)
    ids = O.hash_keys(K, R, L, P)
    vn = O.value_norms(V)
    p = O.soft_bucket_probs(Q, R, L, P, tau)
    assert np.array_equal(O.group_scores(p, ids, vn, 1), O.soft_scores(p, ids, vn, 1))
    # every head of a group asks the same query: G times one head's score,
    # and the shared top-k is that head's top-k
    Q, K, V, R, L, P, tau = _small_problem(34, B=1, Hq=4, Hkv=2)
    Q[:, 1] = Q[:, 0]
    Q[:, 3] = Q[:, 2]
    ids = O.hash_keys(K, R, L, P)
    vn = O.value_norms(V)
    p = O.soft_bucket_probs(Q, R, L, P, tau)
    gs = O.group_scores(p, ids, vn, 2)
    one = O.soft_scores(p, ids, vn, 2)
    assert np.allclose(gs[:, 0], 2 * one[:, 0], rtol=1e-14, atol=0)
    assert np.allclose(gs[:, 1], 2 * one[:, 2], rtol=1e-14, atol=0)
    k = 5
    assert np.array_equal(O.topk_indices(gs[0, 0], k), O.topk_indices(one[0, 0], k))


def test_group_scores_brute_force():
    Q, K, V, R, L, P, tau = _small_problem(35, B=1, Hq=4, Hkv=2)
    ids = O.hash_keys(K, R, L, P)
    vn = O.value_norms(V)
    p = O.soft_bucket_probs(Q, R, L, P, tau)
    gs = O.group_scores(p, ids, vn, 2)
    N = ids.shape[2]
    for g in range(2):
        for n in range(N):
            tot = 0.0
            for j in range(2):
                for l in range(L):
                    tot += float(p[0, 2 * g + j, l, int(ids[0, g, n, l])])
            assert abs(gs[0, g, n] - float(vn[0, g, n]) * tot) <= 1e-12 * max(1.0, abs(gs[0, g, n]))


# --------------------------------------------------------------------- top-k

def test_topk_golden(golden_dir):
    g = _load(golden_dir, "topk_attention_hand.json")["topk"]
    s = np.array(g["scores"])
    for c in g["cases"]:
        assert O.topk_indices(s, c["k"]).tolist() == c["idx"]


def test_topk_matches_python_sort_with_ties():
    r = _rng(40)
    for trial in range(20):
        N = int(r.integers(1, 300))
        s = r.integers(0, 7, size=N).astype(np.float64) * 0.25  # many ties
        k = int(r.integers(1, N + 5))
        ref = sorted(sorted(range(N), key=lambda i: (-s[i], i))[:k])
        assert O.topk_indices(s, k).tolist() == ref


def test_topk_all_equal_takes_lowest_indices():
    s = np.full((2, 100), 3.5)
    assert np.array_equal(O.topk_indices(s, 7), np.tile(np.arange(7), (2, 1)))


# ----------------------------------------------------------------- attention

def test_attention_golden(golden_dir):
    g = _load(golden_dir, "topk_attention_hand.json")["attention"]
    q = np.array(g["q"], float)[None, None]
    K = np.array(g["K"], float)[None, None]
    V = np.array(g["V"], float)[None, None]
    out = O.subset_attention(q, K, V, np.array(g["idx"])[None, None], 1)
    assert np.allclose(out[0, 0], g["out"], atol=g["tolerance"], rtol=0)


def test_attention_full_subset_is_dense_sdpa():
    Q, K, V, _, _, _, _ = _small_problem(50, B=2, Hq=4, Hkv=2, d=16, N=37)
    idx = np.tile(np.arange(37), (2, 4, 1))
    out = O.subset_attention(Q, K, V, idx, 2)
    q = torch.from_numpy(Q)[:, :, None, :]
    k = torch.from_numpy(K).repeat_interleave(2, dim=1)
    v = torch.from_numpy(V).repeat_interleave(2, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)[:, :, 0]
    assert np.allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_attention_single_key_returns_its_value():
    Q, K, V, _, _, _, _ = _small_problem(51, N=9)
    idx = np.full((2, 4, 1), 5)
    out = O.subset_attention(Q, K, V, idx, 2)
    for h in range(4):
        assert np.array_equal(out[:, h], V[:, h // 2, 5])


# --------------------------------------------- whole path, pure-Python brute force

def _brute_decode(Q, K, V, R, L, P, tau, k):
    """Independent pure-Python decode on tiny inputs: exact rational hash,
    explicit enumeration of buckets, full stable sort, dense softmax."""
    B, Hq, d = len(Q), len(Q[0]), len(Q[0][0])
    Hkv, N = len(K[0]), len(K[0][0])
    G = Hq // Hkv
    C = L * P

    def dot_exact(a, b):
        return sum((Fraction(x) * Fraction(y) for x, y in zip(a, b)), Fraction(0))

    col = [[R[i][c] for i in range(d)] for c in range(C)]
    outs, idxs = [], []
    for b in range(B):
        ob, ib = [], []
        for h in range(Hq):
            g = h // G
            q = Q[b][h]
            z = [sum(q[i] * col[c][i] for i in range(d)) for c in range(C)]
            probs = []
            for l in range(L):
                logits = []
                for u in range(2 ** P):
                    t = 0.0
                    for j in range(P):
                        t += z[l * P + j] if (u >> j) & 1 else -z[l * P + j]
                    logits.append(t / tau)
                m = max(logits)
                e = [math.exp(x - m) for x in logits]
                tot = sum(e)
                probs.append([x / tot for x in e])
            scores = []
            for n in range(N):
                key = K[b][g][n]
                total = 0.0
                for l in range(L):
                    u = 0
                    for j in range(P):
                        if dot_exact(key, col[l * P + j]) > 0:
                            u |= 1 << j
                    total += probs[l][u]
                vn = math.sqrt(sum(x * x for x in V[b][g][n]))
                scores.append(vn * total)
            order = sorted(range(N), key=lambda i: (-scores[i], i))
            sel = sorted(order[: min(k, N)])
            logits = [sum(q[i] * K[b][g][n][i] for i in range(d)) / math.sqrt(d) for n in sel]
            m = max(logits)
            w = [math.exp(x - m) for x in logits]
            tot = sum(w)
            out = [sum(w[t] * V[b][g][n][i] for t, n in enumerate(sel)) / tot for i in range(d)]
            ob.append(out)
            ib.append(sel)
        outs.append(ob)
        idxs.append(ib)
    return np.array(outs), np.array(idxs)


@pytest.mark.parametrize("seed,k", [(60, 5), (61, 17), (62, 64)])
def test_whole_path_matches_pure_python_brute_force(seed, k):
    r = _rng(seed)
    B, Hq, Hkv, d, N, L, P, tau = 1, 4, 2, 8, 40, 2, 3, 0.35
    Q = _bf16_values(r.standard_normal((B, Hq, d)))
    K = _bf16_values(r.standard_normal((B, Hkv, N, d)))
    V = _bf16_values(r.standard_normal((B, Hkv, N, d)))
    R = _bf16_values(r.standard_normal((d, L * P)))
    ids = O.hash_keys(K, R, L, P)
    vn = O.value_norms(V)
    out, idx, s, p = O.decode(Q, K, V, R, ids, vn, L, P, tau, k)
    bout, bidx = _brute_decode(Q.tolist(), K.tolist(), V.tolist(), R.tolist(), L, P, tau, k)
    assert np.array_equal(idx, bidx)
    assert np.allclose(out, bout, rtol=1e-12, atol=1e-12)
