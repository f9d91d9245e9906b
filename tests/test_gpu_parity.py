"""GPU parity: every HIP stage and the whole decode path against the CPU oracle.

Gates (tolerances follow from the arithmetic of each step):
  * bucket ids and selected index sets: bit-exact;
  * value norms: 1e-5 relative;
  * soft probabilities: 1e-6 relative (float32 rounding of float64 values)
    plus an absolute floor of 1e-37 for float32 underflow;
  * scores: 1e-5 relative plus an absolute floor of 1e-30 (float32 scores of
    keys whose probabilities underflow where float64 keeps tiny values);
  * top-k: bit-exact against the oracle's selection on the GPU's own scores;
    against the oracle's float64 scores, differences are allowed only for
    keys whose score lies within the score tolerance of the k-th score;
  * attention output: 2e-2 absolute for bf16 (output rounding), 1e-4 for
    float32, with the oracle attending over the GPU's selection.
"""

import sys

import numpy as np
import pytest
import torch

import oracle as O
import soft_lsh_sparse_amd as S
import synthetic as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def tau32(tau):
    return float(np.float32(tau))


def assert_close_rel(got, ref, rel, floor, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    lim = rel * np.abs(ref) + floor
    bad = err > lim
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first at "
            f"{tuple(i)}: got {got[tuple(i)]!r} ref {ref[tuple(i)]!r}")


def table_to_oracle_layout(table, G):
    """[B, Hkv, 2^P, L, G] -> [B, Hq, L, 2^P]."""
    B, Hkv, nb, L, _ = table.shape
    t = table.permute(0, 1, 4, 3, 2).reshape(B, Hkv * G, L, nb)
    return f64(t)


# --------------------------------------------------------------------- hash

HASH_CASES = [
    # (n_heads, N, stride, d, L, P, dtype)
    (1, 1024, 1024, 64, 8, 4, "f32"),
    (2, 1000, 1000, 128, 32, 8, "bf16"),
    (3, 77, 80, 64, 16, 4, "bf16"),
    (1, 33, 33, 128, 64, 6, "bf16"),
    (2, 513, 513, 128, 7, 3, "bf16"),
    (1, 1, 1, 128, 64, 8, "bf16"),
    (2, 300, 310, 128, 11, 8, "f32"),
    (1, 500, 500, 128, 8, 1, "bf16"),
    (1, 257, 257, 64, 40, 5, "bf16"),
]


@pytest.mark.parametrize("case", HASH_CASES)
def test_hash_keys_bit_exact(case):
    n_heads, N, stride, d, L, P, dt = case
    log(f"hash case {case}")
    w = W.custom_workload(B=1, Hq=n_heads, Hkv=n_heads, d=d, N=stride, dtype=dt, L=L, P=P)
    K, V = W.make_keys_values(w, DEV, seed=11)
    R = W.make_hyperplanes(w, DEV, seed=11)
    K, V = K[0], V[0]
    ids, vn = S.hash_keys(K, V, R, L, P, n_keys=N)
    torch.cuda.synchronize()
    ref_ids = O.hash_keys(f64(K[:, :N]), f64(R), L, P)
    ref_vn = O.value_norms(f64(V[:, :N]))
    got = ids[:, :N].cpu().numpy()
    assert np.array_equal(got, ref_ids), f"{int((got != ref_ids).sum())} ids differ"
    assert_close_rel(vn[:, :N].cpu().numpy(), ref_vn, 1e-5, 0.0, "vnorm")


@pytest.mark.parametrize("L,P", [(16, 8), (6, 8), (21, 6)])
def test_hash_near_zero_projections_are_exact(L, P):
    """Keys built so that some projections are exactly 0 or cancel far below
    float32 resolution: the certified-sign fix-up must get every bit right
    (deferred list with whole id words, deferred list with other P, and the
    in-kernel path when id rows are not whole words)."""
    log(f"hash near-zero L={L} P={P}")
    d = 128
    g = torch.Generator().manual_seed(5)
    R = torch.randn(d, L * P, generator=g).to(torch.bfloat16)
    R[0:3, :] = 1.0
    Rf = R.float()
    rows = []
    for c in range(L * P):
        # exact zero: k_i = r_jc, k_j = -r_ic on two rows with nonzero r
        k = torch.zeros(d)
        i, j = 5 + (c % 50), 60 + (c % 60)
        k[i], k[j] = Rf[j, c], -Rf[i, c]
        rows.append(k)
    for s in (1.0, -1.0):
        # big + small - big along rows 0..2 (R = 1 there): exact sign of small
        k = torch.randn(d, generator=g) * 1e-3
        k[0], k[1], k[2] = 2.0 ** 20, s * 2.0 ** -10, -(2.0 ** 20)
        k[3:] = 0.0
        rows.append(k)
    rows.append(torch.zeros(d))
    K = torch.stack(rows)[None].to(torch.bfloat16)
    n = K.shape[1]
    K = K.to(DEV).contiguous()
    V = torch.randn(1, n, d, generator=g).to(torch.bfloat16).to(DEV)
    R = R.to(DEV).contiguous()
    ids, _ = S.hash_keys(K, V, R, L, P)
    torch.cuda.synchronize()
    ref = O.hash_keys(f64(K), f64(R), L, P)
    assert np.array_equal(ids.cpu().numpy(), ref)
    bits = O.hash_bits(f64(K), f64(R))
    assert bits[0, L * P].all() and not bits[0, L * P + 1].any()


def test_hash_fixup_list_overflow_settles_in_kernel():
    """More uncertain projections than the fix-up list holds (all-zero and
    tiny keys): the overflow is settled inside the main kernel."""
    log("hash fix-up overflow")
    w = W.custom_workload(B=1, Hq=2, Hkv=2, d=128, N=4096, dtype="bf16", L=64, P=8)
    K, V = W.make_keys_values(w, DEV, seed=21)
    R = W.make_hyperplanes(w, DEV, seed=21)
    K, V = K[0].clone(), V[0]
    K[:, ::2] = 0                               # 4096 zero keys x 512 projections
    K[:, 1::4] = K[:, 1::4] * 2.0 ** -120       # tiny keys near the absolute floor
    ids, _ = S.hash_keys(K, V, R, w.L, w.P)
    torch.cuda.synchronize()
    ref = O.hash_keys(f64(K), f64(R), w.L, w.P)
    got = ids.cpu().numpy()
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} ids differ"


def test_hash_every_id_of_a_64_table_prefill():
    """Every id of 2 x 16384 Llama-shaped keys (outlier channels, planted
    keys), 64 tables of 8 bits: about 2.5k projections go through the
    deferred fix-up list."""
    w = W.custom_workload("llama3_8b_32k", B=1, Hq=8, Hkv=2, N=16384, L=64, P=8)
    log(f"hash all ids {w.name}")
    K, V = W.make_keys_values(w, DEV, seed=4)
    R = W.make_hyperplanes(w, DEV, seed=4)
    ids, vn = S.hash_keys(K[0], V[0], R, w.L, w.P)
    torch.cuda.synchronize()
    ref = O.hash_keys(f64(K[0]), f64(R), w.L, w.P)
    got = ids.cpu().numpy()
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} ids differ"
    assert_close_rel(vn.cpu().numpy(), O.value_norms(f64(V[0])), 1e-5, 0.0, "vnorm")


def test_hash_append_with_row_offset():
    log("hash append")
    w = W.custom_workload(B=1, Hq=2, Hkv=2, d=128, N=700, dtype="bf16", L=32, P=8)
    K, V = W.make_keys_values(w, DEV, seed=3)
    R = W.make_hyperplanes(w, DEV, seed=3)
    K, V = K[0], V[0]
    full_ids, full_vn = S.hash_keys(K, V, R, 32, 8)
    ids = torch.zeros_like(full_ids)
    vn = torch.zeros_like(full_vn)
    S.hash_keys(K, V, R, 32, 8, n_keys=500, ids=ids, vnorm=vn)
    S.hash_keys(K, V, R, 32, 8, n_keys=1, ids=ids, vnorm=vn, row_offset=500)
    S.hash_keys(K, V, R, 32, 8, ids=ids, vnorm=vn, row_offset=501)
    torch.cuda.synchronize()
    assert torch.equal(ids, full_ids)
    assert torch.equal(vn, full_vn)


# ----------------------------------------------------------- bucket probs

@pytest.mark.parametrize("B,Hq,Hkv,d,L,P,tau,dt", [
    (1, 1, 1, 64, 8, 4, 0.5, "f32"),
    (2, 8, 2, 128, 32, 8, 0.3, "bf16"),
    (1, 32, 8, 128, 64, 6, 0.2, "bf16"),
    (1, 4, 4, 64, 5, 1, 0.05, "bf16"),
    (3, 16, 2, 128, 9, 7, 2.0, "f32"),
])
def test_bucket_probs(B, Hq, Hkv, d, L, P, tau, dt):
    log(f"bucket_probs {(B, Hq, Hkv, d, L, P, tau, dt)}")
    w = W.custom_workload(B=B, Hq=Hq, Hkv=Hkv, d=d, N=8, dtype=dt, L=L, P=P, tau=tau)
    Q = W.make_query(w, DEV, seed=2)
    R = W.make_hyperplanes(w, DEV, seed=2)
    table = S.bucket_probs(Q, R, Hkv, L, P, tau)
    torch.cuda.synchronize()
    got = table_to_oracle_layout(table, Hq // Hkv)
    ref = O.soft_bucket_probs(f64(Q), f64(R), L, P, tau32(tau))
    assert_close_rel(got, ref, 1e-6, 1e-37, "probs")
    assert np.allclose(got.sum(-1), 1.0, atol=1e-5, rtol=0)


# ------------------------------------------------------------------ score

@pytest.mark.parametrize("B,Hq,Hkv,N,L,P", [
    (1, 1, 1, 1024, 8, 4),
    (2, 8, 2, 5000, 32, 8),
    (1, 8, 2, 3001, 64, 6),
    (1, 4, 1, 777, 16, 5),
    (1, 16, 2, 1500, 13, 3),
    (2, 4, 2, 100, 1, 8),
    (1, 2, 1, 65, 24, 2),
])
def test_score_stage(B, Hq, Hkv, N, L, P):
    """Score kernel against the oracle fed the same table, ids and norms."""
    log(f"score {(B, Hq, Hkv, N, L, P)}")
    w = W.custom_workload(B=B, Hq=Hq, Hkv=Hkv, d=128, N=N, dtype="bf16", L=L, P=P,
                          tau=0.3, lognormal_v=True)
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=4)
    ids, vn = S.hash_keys(K, V, R, L, P)
    table = S.bucket_probs(Q, R, Hkv, L, P, 0.3)
    sc = S.score(table, ids, vn, Hq)
    torch.cuda.synchronize()
    ref = O.soft_scores(table_to_oracle_layout(table, Hq // Hkv), ids.cpu().numpy(),
                        f64(vn), Hq // Hkv)
    assert_close_rel(sc.cpu().numpy(), ref, 1e-5, 1e-30, "scores")


# ------------------------------------------------------------------ top-k

@pytest.mark.parametrize("rows,n,k,kind", [
    (1, 1024, 64, "rand"),
    (7, 5000, 300, "ties"),
    (3, 70000, 1, "rand"),
    (2, 70000, 4096, "ties"),
    (4, 129, 128, "rand"),
    (4, 129, 129, "rand"),
    (4, 129, 1000, "rand"),
    (2, 1, 1, "rand"),
    (3, 4096, 100, "const"),
    (2, 20000, 1000, "zeros"),
    (32, 32768, 1024, "lognormal"),
    (5, 300001, 7777, "ties"),
])
def test_topk_stage(rows, n, k, kind):
    log(f"topk {(rows, n, k, kind)}")
    g = torch.Generator().manual_seed(rows * 1000003 + n + k)
    if kind == "rand":
        s = torch.rand(rows, n, generator=g)
    elif kind == "ties":
        s = torch.randint(0, 50, (rows, n), generator=g).float() * 0.125
    elif kind == "const":
        s = torch.full((rows, n), 2.5)
    elif kind == "zeros":
        s = torch.zeros(rows, n)
        s[:, ::7] = torch.rand(rows, (n + 6) // 7, generator=g)
    else:
        s = torch.exp(torch.randn(rows, n, generator=g) * 3.0)
    idx = S.topk(s.to(DEV), k)
    torch.cuda.synchronize()
    ref = O.topk_indices(s.numpy(), k)
    assert np.array_equal(idx.cpu().numpy(), ref)


# --------------------------------------------------------------- attention

@pytest.mark.parametrize("B,Hq,Hkv,d,N,kk,dt", [
    (1, 1, 1, 64, 1024, 64, "f32"),
    (2, 8, 2, 128, 3000, 1000, "bf16"),
    (1, 32, 8, 128, 20000, 4096, "bf16"),
    (1, 4, 4, 64, 50, 50, "bf16"),
    (1, 2, 1, 128, 10, 1, "f32"),
    (2, 8, 1, 128, 700, 333, "f32"),
    # the plan's routes: rows of one chunk write the output directly (the
    # f32 and 50-key cases above); short rows in one-wave blocks of 64 keys
    # (1000 and 333 keys above); 4-wave chunks merged from registers (8 and
    # 10 chunks, ragged) or through LDS (more than 16 chunks)
    (1, 4, 2, 64, 3000, 2048, "bf16"),
    (1, 4, 1, 128, 8000, 2500, "bf16"),
    (1, 4, 2, 64, 3000, 2049, "f32"),
    (1, 2, 1, 128, 9000, 5000, "bf16"),
    (1, 32, 8, 128, 40000, 6000, "bf16"),
])
def test_sparse_attn_stage(B, Hq, Hkv, d, N, kk, dt):
    log(f"attn {(B, Hq, Hkv, d, N, kk, dt)}")
    w = W.custom_workload(B=B, Hq=Hq, Hkv=Hkv, d=d, N=N, dtype=dt, lognormal_v=True)
    Q, K, V, _ = W.make_decode_inputs(w, DEV, seed=6)
    g = torch.Generator().manual_seed(9)
    idx = torch.stack([torch.stack([torch.sort(torch.randperm(N, generator=g)[:kk]).values
                                    for _ in range(Hq)]) for _ in range(B)])
    idx = idx.to(torch.int32).to(DEV)
    out = S.sparse_attn(Q, K, V, idx)
    torch.cuda.synchronize()
    ref = O.subset_attention(f64(Q), f64(K), f64(V), idx.cpu().numpy(), Hq // Hkv)
    tol = 2e-2 if dt == "bf16" else 1e-4
    assert np.max(np.abs(f64(out) - ref)) <= tol


# ------------------------------------------------ GQA group-shared variant

@pytest.mark.parametrize("B,Hq,Hkv,N,k", [
    (1, 8, 2, 3000, 256),       # selection from candidates, ragged tail
    (2, 4, 1, 1500, 2000),      # k >= N: every key, one set per KV head
    (1, 8, 8, 2048, 64),        # G = 1: the per-head decode
    (1, 8, 2, 30000, 6000),     # large k: candidates gathered before the select
])
def test_decode_group_shared_matches_the_oracle(B, Hq, Hkv, N, k):
    w = W.custom_workload(B=B, Hq=Hq, Hkv=Hkv, d=128, N=N, dtype="bf16", L=32, P=8,
                          tau=0.3, k=k, lognormal_v=True)
    log(f"group-shared {(B, Hq, Hkv, N, k)}")
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=17)
    ids, vn = S.hash_keys(K, V, R, w.L, w.P)
    kk = min(k, N)
    idx = torch.empty((B, Hkv, kk), dtype=torch.int32, device=DEV)
    sc = torch.empty((B, Hkv, N), dtype=torch.float32, device=DEV)
    out, _, _ = S.decode_group_shared(Q, K, V, R, ids, vn, w.L, w.P, w.tau, k, idx_out=idx,
                                      scores_out=sc)
    torch.cuda.synchronize()
    G = Hq // Hkv
    p = O.soft_bucket_probs(f64(Q), f64(R), w.L, w.P, tau32(w.tau))
    ref_sc = O.group_scores(p, ids.cpu().numpy(), f64(vn), G)
    sc_np, idx_np = sc.cpu().numpy(), idx.cpu().numpy()
    assert_close_rel(sc_np, ref_sc, 1e-5, 1e-30, "group scores")
    for b in range(B):
        for g in range(Hkv):
            assert np.array_equal(idx_np[b, g], O.topk_indices(sc_np[b, g], kk)), (b, g)
    # every head of a group attends over its group's set
    idx_h = np.repeat(idx_np, G, axis=1)
    ref = O.subset_attention(f64(Q), f64(K), f64(V), idx_h, G)
    assert np.max(np.abs(f64(out) - ref)) <= 2e-2
    if G == 1:  # one head per group: the per-head decode, bit for bit
        out1, idx1, _ = S.decode(Q, K, V, R, ids, vn, w.L, w.P, w.tau, k,
                                 idx_out=torch.empty_like(idx))
        torch.cuda.synchronize()
        assert torch.equal(idx1, idx)


# ------------------------------------------------ hard-LSH comparison

@pytest.mark.parametrize("dt,L,P", [("bf16", 32, 8), ("f32", 8, 4), ("bf16", 11, 6)])
def test_hard_bucket_table_is_one_hot_at_the_query_buckets(dt, L, P):
    w = W.custom_workload(B=2, Hq=8, Hkv=2, d=128, N=64, dtype=dt, L=L, P=P)
    Q, _, _, R = W.make_decode_inputs(w, DEV, seed=15)
    table = S.hard_bucket_table(Q, R, w.Hkv, L, P)
    torch.cuda.synchronize()
    t = table.cpu().numpy()                       # [B, Hkv, 2^P, L, G]
    hb = O.hard_query_buckets(f64(Q), f64(R), L, P)  # [B, Hq, L]
    onehot = np.zeros_like(t)
    G = w.Hq // w.Hkv
    for b in range(w.B):
        for h in range(w.Hq):
            for l in range(L):
                onehot[b, h // G, hb[b, h, l], l, h % G] = 1.0
    assert np.array_equal(t, onehot)
    assert np.array_equal(table_to_oracle_layout(table, G),
                          O.hard_bucket_table(f64(Q), f64(R), L, P))


@pytest.mark.parametrize("dt,L,P", [("bf16", 16, 8), ("f32", 8, 4), ("bf16", 21, 6)])
def test_hard_bucket_table_splits_exactly_zero_query_projections(dt, L, P):
    """Query rows built so that chosen projections are exactly 0 (coordinate
    pairs that cancel: q_2m = r_2m+1,c and q_2m+1 = -r_2m,c, exact products):
    the tau -> 0 table gives such a bit 1/2 : 1/2, as the oracle's limit does."""
    w = W.custom_workload(B=2, Hq=4, Hkv=2, d=128, N=64, dtype=dt, L=L, P=P)
    Q, _, _, R = W.make_decode_inputs(w, DEV, seed=17)
    C = L * P
    picks = [(0, 0, 3), (0, 1, C // 2), (1, 3, C - 1)]
    for (b, h, c) in picks:
        Q[b, h, 0::2] = R[1::2, c]
        Q[b, h, 1::2] = -R[0::2, c]
    z = f64(Q) @ f64(R)                                 # exact: products fit float64
    for (b, h, c) in picks:
        assert z[b, h, c] == 0.0
    log(f"hard table {dt} L={L} P={P}: {(z == 0).sum()} exactly-zero projections")
    table = S.hard_bucket_table(Q, R, w.Hkv, L, P)
    torch.cuda.synchronize()
    got = table_to_oracle_layout(table, w.G)
    ref = O.hard_bucket_table(f64(Q), f64(R), L, P)
    assert np.array_equal(got, ref)
    for (b, h, c) in picks:
        assert np.count_nonzero(got[b, h, c // P]) == 2
        assert np.max(got[b, h, c // P]) == 0.5


def test_hard_scores_are_value_norm_weighted_collision_counts():
    w = W.custom_workload(B=1, Hq=8, Hkv=2, d=128, N=5000, dtype="bf16", L=32, P=8,
                          lognormal_v=True)
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=16)
    ids, vn = S.hash_keys(K, V, R, w.L, w.P)
    sc = S.score(S.hard_bucket_table(Q, R, w.Hkv, w.L, w.P), ids, vn, w.Hq)
    torch.cuda.synchronize()
    hb = O.hard_query_buckets(f64(Q), f64(R), w.L, w.P)       # [B, Hq, L]
    ids_np = ids.cpu().numpy().astype(np.int64)              # [B, Hkv, N, L]
    G = w.Hq // w.Hkv
    counts = np.stack([(ids_np[0, h // G] == hb[0, h][None, :]).sum(-1)
                       for h in range(w.Hq)])[None]          # [B, Hq, N]
    ref = counts * f64(vn)[:, np.arange(w.Hq) // G]
    assert_close_rel(sc.cpu().numpy(), ref, 1e-6, 0.0, "hard scores")
    ref2 = O.soft_scores(O.hard_bucket_table(f64(Q), f64(R), w.L, w.P), ids_np, f64(vn), G)
    assert_close_rel(sc.cpu().numpy(), ref2, 1e-6, 0.0, "hard scores (oracle table)")


# ------------------------------------------------ dense attention baseline

@pytest.mark.parametrize("B,Hq,Hkv,d,N,dt", [
    (1, 4, 1, 128, 1, "bf16"),          # one key
    (1, 4, 1, 128, 37, "bf16"),         # part of one batch
    (2, 8, 2, 128, 2500, "bf16"),       # several chunks and a ragged tail
    (1, 8, 1, 64, 1500, "bf16"),        # 8 heads per KV head
    (1, 2, 1, 128, 3333, "bf16"),       # 2 heads per KV head, four chunks, ragged
    (1, 4, 4, 64, 2049, "bf16"),        # one head per KV head, one key past two chunks
    (1, 2, 1, 64, 777, "f32"),
    (1, 3, 3, 128, 4096, "f32"),        # one head per KV head, whole chunks
])
def test_dense_attn_matches_the_oracle(B, Hq, Hkv, d, N, dt):
    log(f"dense {(B, Hq, Hkv, d, N, dt)}")
    w = W.custom_workload(B=B, Hq=Hq, Hkv=Hkv, d=d, N=N, dtype=dt, lognormal_v=True)
    Q, K, V, _ = W.make_decode_inputs(w, DEV, seed=12)
    out = S.dense_attn(Q, K, V)
    torch.cuda.synchronize()
    idx = np.broadcast_to(np.arange(N), (B, Hq, N))
    ref = O.subset_attention(f64(Q), f64(K), f64(V), idx, Hq // Hkv)
    tol = 2e-2 if dt == "bf16" else 1e-4
    assert np.max(np.abs(f64(out) - ref)) <= tol


def test_dense_attn_reads_only_the_first_n_rows():
    w = W.custom_workload(B=1, Hq=4, Hkv=1, d=128, N=3000, dtype="bf16", lognormal_v=True)
    Q, K, V, _ = W.make_decode_inputs(w, DEV, seed=13)
    out = S.dense_attn(Q, K, V, n=2049)
    torch.cuda.synchronize()
    idx = np.broadcast_to(np.arange(2049), (1, 4, 2049))
    ref = O.subset_attention(f64(Q), f64(K), f64(V), idx, 4)
    assert np.max(np.abs(f64(out) - ref)) <= 2e-2


def test_dense_attn_at_128k_sampled_rows():
    """The bench's dense baseline: B=4, 32/8 heads, d=128, 131072 keys;
    four query rows checked against the oracle over every key."""
    w = W.WORKLOADS["llama3_8b_128k_b4"]
    log(f"dense 128k {w}")
    Q, K, V, _ = W.make_decode_inputs(w, DEV, seed=0)
    out = S.dense_attn(Q, K, V)
    torch.cuda.synchronize()
    G = w.Hq // w.Hkv
    for b, h in [(0, 0), (1, 13), (2, 22), (3, 31)]:
        g = h // G
        ref = O.subset_attention(f64(Q[b:b + 1, h:h + 1]), f64(K[b:b + 1, g:g + 1]),
                                 f64(V[b:b + 1, g:g + 1]),
                                 np.arange(w.N).reshape(1, 1, -1), 1)
        assert np.max(np.abs(f64(out[b, h]) - ref[0, 0])) <= 2e-2, (b, h)


def test_dense_attn_equals_sparse_attn_over_every_key():
    """k = N: the sparse path over all indices and the dense baseline agree
    (both float32 accumulation; different orders, so within rounding)."""
    w = W.custom_workload(B=1, Hq=8, Hkv=2, d=128, N=3000, dtype="bf16", lognormal_v=True)
    Q, K, V, _ = W.make_decode_inputs(w, DEV, seed=14)
    idx = torch.arange(w.N, dtype=torch.int32, device=DEV).expand(1, 8, w.N).contiguous()
    a = S.sparse_attn(Q, K, V, idx)
    d = S.dense_attn(Q, K, V)
    torch.cuda.synchronize()
    assert np.max(np.abs(f64(a) - f64(d))) <= 1e-2


# ----------------------------------------------------------- decode end to end

def _check_decode(w, seed=0, step=0):
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=seed, step=step)
    ids, vn = S.hash_keys(K, V, R, w.L, w.P)
    kk = w.kk
    idx = torch.empty((w.B, w.Hq, kk), dtype=torch.int32, device=DEV)
    sc = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=DEV)
    out, _, _ = S.decode(Q, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, idx_out=idx,
                         scores_out=sc)
    torch.cuda.synchronize()
    G = w.G
    rows = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    p_ref = O.soft_bucket_probs(f64(Q), f64(R), w.L, w.P, tau32(w.tau))
    ids_np = ids.cpu().numpy()
    vn64 = f64(vn)
    sc_np = sc.cpu().numpy()
    idx_np = idx.cpu().numpy()
    out64 = f64(out)
    Q64 = f64(Q)
    swaps = 0
    for (b, h) in rows:
        g = h // G
        s_ref = O.soft_scores(p_ref[b:b + 1, h:h + 1], ids_np[b:b + 1, g:g + 1],
                              vn64[b:b + 1, g:g + 1], 1)[0, 0]
        assert_close_rel(sc_np[b, h], s_ref, 1e-5, 1e-30, f"scores row {(b, h)}")
        # (i) selection is exact on the GPU's own scores
        sel = O.topk_indices(sc_np[b, h], w.k)
        assert np.array_equal(idx_np[b, h], sel), f"top-k row {(b, h)}"
        # (ii) against float64 scores: differences only inside the band
        sel_ref = O.topk_indices(s_ref, w.k)
        diff = np.setxor1d(sel, sel_ref)
        if diff.size:
            kth = np.sort(s_ref)[::-1][kk - 1]
            band = np.abs(s_ref[diff] - kth) <= 1e-5 * kth + 1e-30
            assert band.all(), f"selection differs outside the band in row {(b, h)}"
            swaps += diff.size // 2
        # the oracle attends over the GPU's selection (the gathered rows only)
        sel_t = torch.from_numpy(idx_np[b, h]).long().to(DEV)
        Kg = f64(K[b, g][sel_t])[None, None]
        Vg = f64(V[b, g][sel_t])[None, None]
        ref_out = O.subset_attention(Q64[b:b + 1, h:h + 1], Kg, Vg,
                                     np.arange(kk)[None, None], 1)[0, 0]
        tol = 2e-2 if w.dtype == "bf16" else 1e-4
        assert np.max(np.abs(out64[b, h] - ref_out)) <= tol, f"out row {(b, h)}"
    log(f"{w.name}: {len(rows)} rows checked, {swaps} tolerance-band swaps")
    return ids, vn, out, idx, sc


def test_decode_tiny_fp32_full_oracle():
    w = W.WORKLOADS["tiny_fp32_1k"]
    log(f"decode {w.name}")
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=0)
    ids, vn = S.hash_keys(K, V, R, w.L, w.P)
    idx = torch.empty((1, 1, w.kk), dtype=torch.int32, device=DEV)
    sc = torch.empty((1, 1, w.N), dtype=torch.float32, device=DEV)
    out, _, _ = S.decode(Q, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, idx_out=idx,
                         scores_out=sc)
    torch.cuda.synchronize()
    ref_ids = O.hash_keys(f64(K), f64(R), w.L, w.P)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    r_out, r_idx, r_s, _ = O.decode(f64(Q), f64(K), f64(V), f64(R), ref_ids,
                                    O.value_norms(f64(V)), w.L, w.P, tau32(w.tau), w.k)
    assert_close_rel(sc.cpu().numpy(), r_s, 1e-5, 1e-30, "scores")
    assert np.array_equal(idx.cpu().numpy(), O.topk_indices(sc.cpu().numpy(), w.k))
    assert np.array_equal(idx.cpu().numpy(), r_idx)
    assert np.max(np.abs(f64(out) - r_out)) <= 1e-4


def test_decode_small_gqa_full():
    w = W.custom_workload(B=2, Hq=8, Hkv=2, d=128, N=5000, dtype="bf16", L=32, P=8,
                          tau=0.3, k=300, outlier_channels=4, outlier_scale=8.0,
                          lognormal_v=True, planted=16, name="small_gqa")
    log("decode small_gqa")
    _check_decode(w)


@pytest.mark.parametrize("Hq,Hkv,L,P,d", [
    (8, 2, 16, 8, 128),   # 16-table region layout, table built in the block
    (8, 2, 16, 6, 128),   # rotated 16 tables, two blocks per CU
    (8, 2, 32, 6, 128),   # rotated 32 tables, table from the table kernel
    (8, 2, 64, 6, 128),   # 64-table region layout (6 bits)
    (4, 2, 32, 8, 128),   # two query heads per block, table built in the block
    (4, 4, 32, 8, 128),   # one query head per block
    (8, 2, 32, 8, 64),    # head dimension 64: the build's four-part projections
])
def test_decode_scorer_layouts(Hq, Hkv, L, P, d):
    """The decode through each score kernel layout (region or rotated
    order, table built in the block or copied from the table kernel, one,
    two or four query heads per block, head dimension 128 or 64): every
    row's scores, selection and output against the oracle, over 20011 keys
    (several blocks, a ragged last one)."""
    w = W.custom_workload(B=2, Hq=Hq, Hkv=Hkv, d=d, N=20011, dtype="bf16", L=L, P=P,
                          tau=0.3, k=700, outlier_channels=4, outlier_scale=8.0,
                          lognormal_v=True, planted=16, name=f"layout_{Hq}_{Hkv}_{L}_{P}_{d}")
    log(f"decode {w.name}")
    _check_decode(w, seed=29)


@pytest.mark.parametrize("Hq,Hkv,L,P,dt", [(8, 2, 64, 8, "bf16"), (16, 2, 64, 8, "bf16"),
                                           (8, 2, 64, 8, "f32"), (8, 1, 128, 8, "f32")])
def test_decode_packs_query_heads_when_the_group_table_overflows_lds(Hq, Hkv, L, P, dt):
    """The group's tables (2^P * L * G floats) exceed the LDS: the score
    blocks take Gp < G query heads each and stream the KV head's ids once per
    pack; every row still matches the oracle."""
    w = W.custom_workload(B=2, Hq=Hq, Hkv=Hkv, d=128, N=5000, dtype=dt, L=L, P=P, tau=0.3,
                          k=300, outlier_channels=4, outlier_scale=8.0, lognormal_v=True,
                          planted=16, name=f"gpack_{Hq}_{Hkv}_{L}_{dt}")
    log(f"decode {w.name}")
    _check_decode(w, seed=23)


def test_score_stage_packs_query_heads():
    """socket_score on a group table too large for one block (L=64, P=8,
    G=4): each block copies its pack's heads out of the full table."""
    w = W.custom_workload(B=1, Hq=8, Hkv=2, d=128, N=3000, dtype="bf16", L=64, P=8, tau=0.3,
                          lognormal_v=True)
    log("score stage with packs")
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=24)
    ids, vn = S.hash_keys(K, V, R, w.L, w.P)
    table = S.bucket_probs(Q, R, w.Hkv, w.L, w.P, w.tau)
    sc = S.score(table, ids, vn, w.Hq)
    torch.cuda.synchronize()
    p = table_to_oracle_layout(table, w.G)
    ref = O.soft_scores(p, ids.cpu().numpy(), f64(vn), w.G)
    assert_close_rel(sc.cpu().numpy(), ref, 1e-5, 1e-30, "packed stage scores")


def test_decode_is_deterministic():
    w = W.WORKLOADS["llama3_8b_32k"]
    log("decode determinism")
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=1)
    ids, vn = S.hash_keys(K, V, R, w.L, w.P)
    ids2, vn2 = S.hash_keys(K, V, R, w.L, w.P)
    assert torch.equal(ids, ids2) and torch.equal(vn, vn2)
    res = []
    for _ in range(2):
        idx = torch.empty((w.B, w.Hq, w.kk), dtype=torch.int32, device=DEV)
        sc = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=DEV)
        out, _, _ = S.decode(Q, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, idx_out=idx,
                             scores_out=sc)
        res.append((out, idx, sc))
    torch.cuda.synchronize()
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a, b)


def test_decode_replays_from_a_hip_graph():
    """A decode step enqueues kernels only (no memset, no host synchronisation),
    so it can be captured in a HIP graph. Four replays over two queries, with
    eager work and a synchronisation between them, reproduce the eager results
    bit for bit."""
    w = W.WORKLOADS["llama3_8b_32k"]
    log("decode graph replay")
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=3)
    Q2 = W.make_query(w, DEV, seed=3, step=1)
    ids, vn = S.hash_keys(K, V, R, w.L, w.P)
    need = S.decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.N, w.L, w.P, w.k)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    ref = []
    for q in (Q, Q2):
        idx = torch.empty((w.B, w.Hq, w.kk), dtype=torch.int32, device=DEV)
        o, i, _ = S.decode(q, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, idx_out=idx,
                           workspace=ws)
        ref.append((o.clone(), i.clone()))
    torch.cuda.synchronize()
    qbuf = Q.clone()
    out = torch.empty_like(Q)
    idx = torch.empty((w.B, w.Hq, w.kk), dtype=torch.int32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        S.decode(qbuf, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, out=out, idx_out=idx,
                 workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        S.decode(qbuf, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, out=out, idx_out=idx,
                 workspace=ws)
    for rep in range(4):
        qbuf.copy_((Q, Q2)[rep % 2])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[rep % 2][0]), f"replay {rep}"
        assert torch.equal(idx, ref[rep % 2][1]), f"replay {rep}"
        busy = (K[0, 0, :4096].float() * 2.0).sum()  # eager work between replays
        assert torch.isfinite(busy)
    del g


def _append_and_decode(Q, K, V, R, ids, vn, w, n, ws, out, idx, sc=None):
    """One decode-loop step: hash the key appended at row n - 1 of every head
    (n = 1 at that offset), then decode over the first n keys."""
    S.hash_keys(K, V, R, w.L, w.P, n_keys=1, ids=ids, vnorm=vn, row_offset=n - 1)
    S.decode(Q, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, n_keys=n, out=out, idx_out=idx,
             scores_out=sc, workspace=ws)


def test_decode_loop_appends_one_key_per_step():
    """Decode loop: every step appends one key per KV head (hashed alone,
    through the one-launch path) and decodes over the grown cache. After each
    step the ids and norms equal a prefill of the same rows bit for bit, and
    the step matches the oracle (scores, exact selection on those scores,
    output over the selection)."""
    w = W.custom_workload(B=1, Hq=8, Hkv=2, d=128, N=1030, dtype="bf16", L=32, P=8,
                          tau=0.3, k=64, lognormal_v=True)
    log("decode loop with appends")
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=8)
    n0 = 1024
    ids = torch.zeros((w.B, w.Hkv, w.N, w.L), dtype=torch.uint8, device=DEV)
    vn = torch.zeros((w.B, w.Hkv, w.N), dtype=torch.float32, device=DEV)
    S.hash_keys(K, V, R, w.L, w.P, n_keys=n0, ids=ids, vnorm=vn)
    full_ids, full_vn = S.hash_keys(K, V, R, w.L, w.P)
    ws = torch.empty(S.decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.N, w.L, w.P, w.k),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty_like(Q)
    kk = min(w.k, n0)
    for t in range(w.N - n0):
        n = n0 + t + 1
        Qt = W.make_query(w, DEV, seed=8, step=t)
        idx = torch.empty((w.B, w.Hq, kk), dtype=torch.int32, device=DEV)
        sc = torch.empty((w.B, w.Hq, n), dtype=torch.float32, device=DEV)
        _append_and_decode(Qt, K, V, R, ids, vn, w, n, ws, out, idx, sc)
        torch.cuda.synchronize()
        assert torch.equal(ids[:, :, :n], full_ids[:, :, :n]), f"ids after step {t}"
        assert torch.equal(vn[:, :, :n], full_vn[:, :, :n]), f"norms after step {t}"
        p_ref = O.soft_bucket_probs(f64(Qt), f64(R), w.L, w.P, tau32(w.tau))
        sc_np, idx_np = sc.cpu().numpy(), idx.cpu().numpy()
        ref_sc = O.soft_scores(p_ref, ids[:, :, :n].cpu().numpy(), f64(vn[:, :, :n]), w.G)
        assert_close_rel(sc_np, ref_sc, 1e-5, 1e-30, f"scores step {t}")
        for h in range(w.Hq):
            assert np.array_equal(idx_np[0, h], O.topk_indices(sc_np[0, h], w.k)), (t, h)
        ref_out = O.subset_attention(f64(Qt), f64(K[:, :, :n]), f64(V[:, :, :n]), idx_np, w.G)
        assert np.max(np.abs(f64(out) - ref_out)) <= 2e-2, f"output step {t}"


def test_decode_loop_replays_from_one_hip_graph():
    """Four steps of the decode loop (append, then decode over the grown
    cache) captured in one HIP graph: two replays, with eager work between
    them, reproduce the eager loop's outputs and selections bit for bit."""
    w = W.custom_workload(B=2, Hq=8, Hkv=2, d=128, N=4100, dtype="bf16", L=32, P=8,
                          tau=0.3, k=256, lognormal_v=True)
    log("decode loop graph")
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=9)
    n0, steps = 4096, 4
    qs = [W.make_query(w, DEV, seed=9, step=t) for t in range(steps)]
    ws = torch.empty(S.decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.N, w.L, w.P, w.k),
                     dtype=torch.uint8, device=DEV)
    outs = [torch.empty_like(Q) for _ in range(steps)]
    idxs = [torch.empty((w.B, w.Hq, w.kk), dtype=torch.int32, device=DEV) for _ in range(steps)]

    def fresh_cache():
        ids = torch.zeros((w.B, w.Hkv, w.N, w.L), dtype=torch.uint8, device=DEV)
        vn = torch.zeros((w.B, w.Hkv, w.N), dtype=torch.float32, device=DEV)
        S.hash_keys(K, V, R, w.L, w.P, n_keys=n0, ids=ids, vnorm=vn)
        return ids, vn

    ids, vn = fresh_cache()
    for t in range(steps):
        _append_and_decode(qs[t], K, V, R, ids, vn, w, n0 + t + 1, ws, outs[t], idxs[t])
    torch.cuda.synchronize()
    ref = [(o.clone(), i.clone()) for o, i in zip(outs, idxs)]
    ids, vn = fresh_cache()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream before capture
        _append_and_decode(qs[0], K, V, R, ids, vn, w, n0 + 1, ws, outs[0], idxs[0])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(steps):
            _append_and_decode(qs[t], K, V, R, ids, vn, w, n0 + t + 1, ws, outs[t], idxs[t])
    for rep in range(2):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for t in range(steps):
            assert torch.equal(outs[t], ref[t][0]), (rep, t)
            assert torch.equal(idxs[t], ref[t][1]), (rep, t)
        busy = (K[0, 0, :4096].float() * 2.0).sum()  # eager work between replays
        assert torch.isfinite(busy)
    del g


def test_decode_identical_group_queries_give_identical_outputs():
    w = W.custom_workload(B=1, Hq=8, Hkv=2, d=128, N=4000, dtype="bf16", L=32, P=8,
                          tau=0.3, k=256, lognormal_v=True)
    log("decode GQA identical")
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=8)
    Q = Q[:, ::4].repeat_interleave(4, dim=1).contiguous()
    ids, vn = S.hash_keys(K, V, R, w.L, w.P)
    idx = torch.empty((1, 8, 256), dtype=torch.int32, device=DEV)
    out, _, _ = S.decode(Q, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, idx_out=idx)
    torch.cuda.synchronize()
    for h in range(8):
        assert torch.equal(out[0, h], out[0, (h // 4) * 4])
        assert torch.equal(idx[0, h], idx[0, (h // 4) * 4])


@pytest.mark.parametrize("N,k", [(1, 1), (5, 3), (5, 5), (64, 1000), (1000, 1)])
def test_decode_edge_sizes(N, k):
    w = W.custom_workload(B=1, Hq=4, Hkv=2, d=128, N=N, dtype="bf16", L=32, P=8,
                          tau=0.3, k=k, lognormal_v=True, name=f"edge_{N}_{k}")
    log(f"decode edge N={N} k={k}")
    _, _, out, idx, _ = _check_decode(w)
    if N == 1:
        _, _, V, _ = W.make_decode_inputs(w, DEV)
        for h in range(4):
            assert torch.equal(out[0, h], V[0, h // 2, 0])
    if k >= N:
        assert torch.equal(idx.cpu(), torch.arange(N, dtype=torch.int32).expand(1, 4, N))


@pytest.mark.parametrize("name", ["llama3_8b_32k", "tiny_fp32_1k"])
def test_decode_scores_equal_stage_pipeline_bit_for_bit(name):
    """The decode path builds each head's probability table inside the score
    kernel; it must equal the standalone table + score stages exactly."""
    w = W.WORKLOADS[name]
    log(f"decode vs stages {w.name}")
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=5)
    ids, vn = S.hash_keys(K, V, R, w.L, w.P)
    sc = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=DEV)
    idx = torch.empty((w.B, w.Hq, w.kk), dtype=torch.int32, device=DEV)
    S.decode(Q, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, idx_out=idx, scores_out=sc)
    table = S.bucket_probs(Q, R, w.Hkv, w.L, w.P, w.tau)
    sc2 = S.score(table, ids, vn, w.Hq)
    idx2 = S.topk(sc2, w.k)
    torch.cuda.synchronize()
    assert torch.equal(sc, sc2)
    assert torch.equal(idx, idx2)


def _sample_positions(n):
    """Keys the decode's threshold estimate scores: key_i = floor(i * n / n_s),
    n_s = min(n, 2048)."""
    n_s = min(n, 2048)
    return (np.arange(n_s, dtype=np.int64) * n) // n_s


@pytest.mark.parametrize("name", ["llama3_8b_128k_b4", "llama3_8b_1m"])
def test_decode_without_score_rows_selects_the_same(name):
    """Without score rows the decode keeps only the candidates above the
    estimated threshold; selection and output must not change."""
    w = W.WORKLOADS[name]
    log(f"decode with / without score rows {w.name}")
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=3)
    ids, vn = S.hash_keys(K, V, R, w.L, w.P)
    idx = torch.empty((w.B, w.Hq, w.kk), dtype=torch.int32, device=DEV)
    sc = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=DEV)
    out, _, _ = S.decode(Q, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, idx_out=idx,
                         scores_out=sc)
    idx2 = torch.empty_like(idx)
    out2, _, _ = S.decode(Q, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, idx_out=idx2)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert torch.equal(out, out2)
    sc_np = sc.cpu().numpy()
    idx_np = idx.cpu().numpy()
    for (b, h) in [(0, 0), (w.B - 1, w.Hq - 1)]:
        assert np.array_equal(idx_np[b, h], O.topk_indices(sc_np[b, h], w.k))


@pytest.mark.parametrize("with_rows,Hq,k", [(True, 4, 1024), (False, 4, 1024), (False, 8, 1024),
                                             (False, 4, 6000), (True, 4, 6000)])
def test_decode_threshold_fallback_selects_from_full_rows(with_rows, Hq, k):
    """Value norms vanish except on the sampled keys of KV head 0, so that head's
    rows see fewer than k keys reach the estimated threshold and are selected
    from fully scored rows; KV head 1 takes the candidate path. Ties among the
    zero scores go to the lower indices. k = 6000: the candidates are gathered
    first (and head 0's rows have fewer of them than k)."""
    w = W.custom_workload(B=1, Hq=Hq, Hkv=2, d=128, N=65536, dtype="bf16", L=32, P=8,
                          tau=0.3, k=k, lognormal_v=True, name="fallback")
    log(f"decode threshold fallback with_rows={with_rows} Hq={Hq} k={k}")
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=11)
    ids, vn = S.hash_keys(K, V, R, w.L, w.P)
    pos = torch.from_numpy(_sample_positions(w.N)).to(DEV)
    vn_mod = vn.clone()
    keep = vn[0, 0, pos].clone()
    vn_mod[0, 0].zero_()
    vn_mod[0, 0, pos] = keep
    idx = torch.empty((1, Hq, w.kk), dtype=torch.int32, device=DEV)
    sc = torch.empty((1, Hq, w.N), dtype=torch.float32, device=DEV) if with_rows else None
    out, _, _ = S.decode(Q, K, V, R, ids, vn_mod, w.L, w.P, w.tau, w.k, idx_out=idx,
                         scores_out=sc)
    table = S.bucket_probs(Q, R, w.Hkv, w.L, w.P, w.tau)
    sc_ref = S.score(table, ids, vn_mod, w.Hq)
    torch.cuda.synchronize()
    if with_rows:
        assert torch.equal(sc, sc_ref)
    s_np = sc_ref.cpu().numpy()
    idx_np = idx.cpu().numpy()
    for h in range(Hq):
        assert np.array_equal(idx_np[0, h], O.topk_indices(s_np[0, h], w.k)), f"head {h}"
    # head 0's selection: only sampled keys score above zero
    samples = _sample_positions(w.N)
    if w.kk <= samples.size:
        assert np.isin(idx_np[0, 0], samples).all()
    else:  # every sampled key that scores above zero, the rest zeros
        assert np.isin(samples[s_np[0, 0, samples] > 0], idx_np[0, 0]).all()
    Q64 = f64(Q)
    for h in (0, Hq - 1):
        g = h // w.G
        sel_t = idx[0, h].long()
        ref = O.subset_attention(Q64[:, h:h + 1], f64(K[0, g][sel_t])[None, None],
                                 f64(V[0, g][sel_t])[None, None],
                                 np.arange(w.kk)[None, None], 1)[0, 0]
        assert np.max(np.abs(f64(out[0, h]) - ref)) <= 2e-2


@pytest.mark.parametrize("N", [9000, 9001, 40000])
def test_decode_all_scores_tied(N):
    """Every key in the same buckets with the same value norm: all scores of a
    row are equal, every key reaches the threshold (beyond the LDS copy of
    the candidates at N = 40000), and the k lowest indices are selected."""
    w = W.custom_workload(B=1, Hq=4, Hkv=1, d=128, N=N, dtype="bf16", L=32, P=8,
                          tau=0.3, k=700, lognormal_v=False, name="tied")
    log(f"decode all tied N={N}")
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=12)
    ids = torch.full((1, 1, N, w.L), 5, dtype=torch.uint8, device=DEV)
    vn = torch.ones((1, 1, N), dtype=torch.float32, device=DEV)
    idx = torch.empty((1, 4, w.kk), dtype=torch.int32, device=DEV)
    out, _, _ = S.decode(Q, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, idx_out=idx)
    torch.cuda.synchronize()
    want = torch.arange(w.kk, dtype=torch.int32).expand(1, 4, w.kk)
    assert torch.equal(idx.cpu(), want)


@pytest.mark.parametrize("N,k", [(30000, 6000), (100000, 8000)])
def test_decode_gathered_candidates(N, k):
    """With k large enough the selection first gathers each row's candidates
    into one contiguous run (16K of them in LDS, the rest read from the run):
    full oracle check of every row, and the call without score rows (whose
    row buffers hold the gathered runs) selects the same."""
    w = W.custom_workload(B=1, Hq=4, Hkv=2, d=128, N=N, dtype="bf16", L=32, P=8,
                          tau=0.3, k=k, outlier_channels=4, outlier_scale=8.0,
                          lognormal_v=True, planted=16, name="gathered")
    log(f"decode gathered candidates N={N} k={k}")
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=5)
    ids, vn, out, idx, sc = _check_decode(w, seed=5)
    idx2 = torch.empty_like(idx)
    out2, _, _ = S.decode(Q, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, idx_out=idx2)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert torch.equal(out, out2)


@pytest.mark.parametrize("N,top", [(40000, 19000), (40000, 19001), (40000, 40000),
                                   (24000, 9000), (24000, 9001)])
def test_decode_gathered_ties(N, top):
    """All keys below `top` share one score, the others score 0: k = 6000 of
    the tied keys are taken, the lowest indices first. top = 19000 or 19001:
    the candidates are gathered (past the LDS copy); top = 40000: they
    overflow the row's gather region and are read from the sub-lists;
    N = 24000: gathered, all in LDS. Odd counts end in half a pair."""
    w = W.custom_workload(B=1, Hq=4, Hkv=1, d=128, N=N, dtype="bf16", L=32, P=8,
                          tau=0.3, k=6000, lognormal_v=False, name="tied_gathered")
    log(f"decode gathered ties N={N} top={top}")
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=13)
    ids = torch.full((1, 1, N, w.L), 5, dtype=torch.uint8, device=DEV)
    vn = torch.zeros((1, 1, N), dtype=torch.float32, device=DEV)
    vn[..., :top] = 1.0
    for with_rows in (False, True):
        idx = torch.empty((1, 4, w.kk), dtype=torch.int32, device=DEV)
        sc = torch.empty((1, 4, N), dtype=torch.float32, device=DEV) if with_rows else None
        S.decode(Q, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, idx_out=idx, scores_out=sc)
        torch.cuda.synchronize()
        want = torch.arange(w.kk, dtype=torch.int32).expand(1, 4, w.kk)
        assert torch.equal(idx.cpu(), want), f"with_rows={with_rows}"


def test_decode_gathered_ties_in_the_threshold_bin():
    """64 value-norm levels of 625 keys each, spread over the index range by
    a permutation (i * 7919 mod N), all keys in the same buckets: scores tie
    exactly within a level. k = 20300 takes the 32 top levels whole and 300
    of the next level's 625 tied keys, the lowest indices first. The
    candidates (more than the 16K the select copies into LDS) are gathered,
    and the threshold bin's 625 keys are collected into LDS after the first
    radix pass, each tagged with the chunk it came from."""
    N, levels, per, k = 40000, 64, 625, 20300
    w = W.custom_workload(B=1, Hq=4, Hkv=1, d=128, N=N, dtype="bf16", L=32, P=8,
                          tau=0.3, k=k, lognormal_v=False, name="tied_levels")
    log(f"decode gathered ties in the threshold bin N={N} k={k}")
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=14)
    level = (np.arange(N, dtype=np.int64) * 7919 % N) // per
    ids = torch.full((1, 1, N, w.L), 5, dtype=torch.uint8, device=DEV)
    vn = torch.from_numpy((1.0 + level / levels).astype(np.float32)).view(1, 1, N).to(DEV)
    top = np.nonzero(level >= levels // 2)[0]
    tied = np.nonzero(level == levels // 2 - 1)[0][:k - len(top)]
    want = np.sort(np.concatenate([top, tied])).astype(np.int32)
    assert len(want) == k
    for with_rows in (False, True):
        idx = torch.empty((1, 4, k), dtype=torch.int32, device=DEV)
        sc = torch.empty((1, 4, N), dtype=torch.float32, device=DEV) if with_rows else None
        S.decode(Q, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, idx_out=idx, scores_out=sc)
        torch.cuda.synchronize()
        for h in range(4):
            assert np.array_equal(idx[0, h].cpu().numpy(), want), f"with_rows={with_rows} h={h}"


@pytest.mark.parametrize("with_rows", [False, True])
def test_decode_clustered_candidates(with_rows):
    """The first 4096 keys sit, in every table, in query head 0's most likely
    bucket, with a value norm of 1; the others keep their own buckets with a
    norm of 1e-3. L = 24 (tables summed in the same order for every key), so
    head 0's candidates are exactly those 4096 tied keys (every other score
    is below 24e-3, theirs at least 24/256), in full sub-lists too long for
    the select's per-thread copy (its direct-to-LDS path runs), and its k
    lowest indices are selected. Every head's selection equals the oracle's
    top-k of the GPU's own scores."""
    w = W.custom_workload(B=1, Hq=4, Hkv=1, d=128, N=65536, dtype="bf16", L=24, P=8,
                          tau=0.3, k=2000, lognormal_v=False, name="clustered")
    log(f"decode clustered candidates with_rows={with_rows}")
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=14)
    ids, vn = S.hash_keys(K, V, R, w.L, w.P)
    table = S.bucket_probs(Q, R, w.Hkv, w.L, w.P, w.tau)  # [B, Hkv, 2^P, L, G]
    best = table[0, 0, :, :, 0].argmax(dim=0).to(torch.uint8)  # per table
    ids[..., :4096, :] = best
    vn = torch.full_like(vn, 1e-3)
    vn[..., :4096] = 1.0
    idx = torch.empty((1, 4, w.kk), dtype=torch.int32, device=DEV)
    sc = torch.empty((1, 4, w.N), dtype=torch.float32, device=DEV) if with_rows else None
    S.decode(Q, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, idx_out=idx, scores_out=sc)
    sc_ref = S.score(table, ids, vn, w.Hq)
    torch.cuda.synchronize()
    if with_rows:
        assert torch.equal(sc, sc_ref)
    s_np, idx_np = sc_ref.cpu().numpy(), idx.cpu().numpy()
    for h in range(4):
        assert np.array_equal(idx_np[0, h], O.topk_indices(s_np[0, h], w.k)), f"head {h}"
    assert s_np[0, 0, 4096:].max() < s_np[0, 0, 0]
    assert np.array_equal(idx_np[0, 0], np.arange(w.kk))


@pytest.mark.parametrize("with_rows", [False, True])
def test_decode_many_sub_lists(with_rows):
    """One KV head of 600000 keys: 147 score blocks of 16 waves give 2352
    candidate sub-lists per row, more than the select's 1024 threads, each
    of which then copies several short sub-lists.
    Selection equals the oracle's top-k of the GPU's own scores."""
    w = W.custom_workload(B=1, Hq=4, Hkv=1, d=128, N=600000, dtype="bf16", L=32, P=8,
                          tau=0.3, k=500, lognormal_v=True, name="many_sub_lists")
    log(f"decode many sub-lists with_rows={with_rows}")
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=15)
    ids, vn = S.hash_keys(K, V, R, w.L, w.P)
    idx = torch.empty((1, 4, w.kk), dtype=torch.int32, device=DEV)
    sc = torch.empty((1, 4, w.N), dtype=torch.float32, device=DEV) if with_rows else None
    S.decode(Q, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, idx_out=idx, scores_out=sc)
    table = S.bucket_probs(Q, R, w.Hkv, w.L, w.P, w.tau)
    sc_ref = S.score(table, ids, vn, w.Hq)
    torch.cuda.synchronize()
    if with_rows:
        assert torch.equal(sc, sc_ref)
    s_np, idx_np = sc_ref.cpu().numpy(), idx.cpu().numpy()
    for h in range(4):
        assert np.array_equal(idx_np[0, h], O.topk_indices(s_np[0, h], w.k)), f"head {h}"


@pytest.mark.parametrize("N,k", [(2097152, 4096), (2092000, 500), (2092000, 16384)])
def test_decode_unequal_wave_shares(N, k):
    """64 tables, one KV head of about 2M keys: 256 score blocks of 8192
    keys, whose 16 waves take unequal shares of 640, 512, 512 and 384 keys
    (waves 0-3, 4-7, 8-11, 12-15). With N = 2092000 the last block holds
    3040 keys, cut inside wave 4's share. Every score is written once (the
    score rows equal socket_score's) and the selection, from short
    sub-lists (k = 500) or gathered candidates (k = 16384), equals the
    oracle's top-k of the GPU's own scores."""
    w = W.custom_workload(B=1, Hq=4, Hkv=1, d=128, N=N, dtype="bf16", L=64, P=6,
                          tau=0.2, k=k, lognormal_v=True, name="unequal_shares")
    log(f"decode unequal wave shares N={N} k={k}")
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=17)
    ids, vn = S.hash_keys(K, V, R, w.L, w.P)
    idx = torch.empty((1, 4, w.kk), dtype=torch.int32, device=DEV)
    sc = torch.empty((1, 4, w.N), dtype=torch.float32, device=DEV)
    S.decode(Q, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, idx_out=idx, scores_out=sc)
    idx2 = torch.empty_like(idx)
    S.decode(Q, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, idx_out=idx2)
    table = S.bucket_probs(Q, R, w.Hkv, w.L, w.P, w.tau)
    sc_ref = S.score(table, ids, vn, w.Hq)
    torch.cuda.synchronize()
    assert torch.equal(sc, sc_ref)
    assert torch.equal(idx, idx2)
    s_np, idx_np = sc_ref.cpu().numpy(), idx.cpu().numpy()
    for h in range(4):
        assert np.array_equal(idx_np[0, h], O.topk_indices(s_np[0, h], w.k)), f"head {h}"


def test_decode_group_shared_unequal_wave_shares():
    """The group-shared decode with 64 tables of 6 bits over 2092000 keys of
    one KV head: its score kernel (one summed row per KV head) takes the
    same unequal wave shares, the last block cut inside wave 4's share. The
    summed scores match the oracle's, the selection is the oracle's top-k of
    the GPU's own scores (equal with and without score rows) and every head
    attends over it."""
    w = W.custom_workload(B=1, Hq=4, Hkv=1, d=128, N=2092000, dtype="bf16", L=64, P=6,
                          tau=0.2, k=4096, lognormal_v=True, name="group_unequal_shares")
    log("group-shared decode, unequal wave shares")
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=18)
    ids, vn = S.hash_keys(K, V, R, w.L, w.P)
    kk = w.kk
    idx = torch.empty((1, 1, kk), dtype=torch.int32, device=DEV)
    sc = torch.empty((1, 1, w.N), dtype=torch.float32, device=DEV)
    out, _, _ = S.decode_group_shared(Q, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, idx_out=idx,
                                      scores_out=sc)
    idx2 = torch.empty_like(idx)
    S.decode_group_shared(Q, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, idx_out=idx2)
    torch.cuda.synchronize()
    p = O.soft_bucket_probs(f64(Q), f64(R), w.L, w.P, tau32(w.tau))
    ref_sc = O.group_scores(p, ids.cpu().numpy(), f64(vn), 4)
    sc_np, idx_np = sc.cpu().numpy(), idx.cpu().numpy()
    assert_close_rel(sc_np, ref_sc, 1e-5, 1e-30, "group scores")
    assert np.array_equal(idx_np[0, 0], O.topk_indices(sc_np[0, 0], kk))
    assert torch.equal(idx, idx2)
    sel = idx[0, 0].long()
    Kg = f64(K[0, 0][sel])[None, None]
    Vg = f64(V[0, 0][sel])[None, None]
    ref = O.subset_attention(f64(Q), Kg, Vg, np.tile(np.arange(kk), (1, 4, 1)), 4)
    assert np.max(np.abs(f64(out) - ref)) <= 2e-2


@pytest.mark.parametrize("N", [6145, 8191])
def test_decode_gathered_ragged_last_segment(N):
    """One query head, k = 6000 (the candidates are gathered): the last score
    block holds a few keys only, so most of its waves' sub-lists are empty
    and start past the row's end; nothing may be read there. Selection
    equals the oracle's top-k of the GPU's own scores, with and without
    score rows."""
    w = W.custom_workload(B=1, Hq=1, Hkv=1, d=128, N=N, dtype="bf16", L=32, P=8,
                          tau=0.3, k=6000, lognormal_v=True, name="gathered_tail")
    log(f"decode gathered ragged last segment N={N}")
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=16)
    ids, vn = S.hash_keys(K, V, R, w.L, w.P)
    idx = torch.empty((1, 1, w.kk), dtype=torch.int32, device=DEV)
    sc = torch.empty((1, 1, N), dtype=torch.float32, device=DEV)
    S.decode(Q, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, idx_out=idx, scores_out=sc)
    idx2 = torch.empty_like(idx)
    S.decode(Q, K, V, R, ids, vn, w.L, w.P, w.tau, w.k, idx_out=idx2)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert np.array_equal(idx.cpu().numpy()[0, 0], O.topk_indices(sc.cpu().numpy()[0, 0], w.k))
