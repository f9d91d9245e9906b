"""Plain fp64 CPU oracle for SOCKET's soft-collision sparse-attention decode.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this module. It shares no code with the HIP library and
never calls it; the product path never calls this.

Sources (cited by page title and section; the pages give no code and no
formulas beyond the symbols L, k, tau):
  [SOCKET-es] "Resumen Técnico: SOCKET - Estimador de Núcleo de Colisión Suave
              para Atención Escasa" (gist.science/es/paper/2602.06283)
  [SOCKET-de] "SOCKET: SOft Collision Kernel EsTimator for Sparse Attention"
              (gist.science/de/paper/2602.06283), Technische Zusammenfassung

The method is an approximation, so this module follows its steps in the
pages' order: (1) prefill hashing into L tables with random projections and
caching the value norms; (2) soft assignment of the query to every bucket of
every table through a temperature softmax; (3) the soft collision score of
each key, weighted by its value norm; (4) deterministic top-k; (5) exact
attention over the selected keys. Every step is written in float64 from its
plain definition; numpy's matmul, sort and exp are the only library steps.

Readings where the pages are silent (each one is also used by the GPU path):
  * Logit form of the soft hash. Table l uses projections z_{lP..lP+P-1} of
    the query onto hyperplanes lP..lP+P-1. Bucket u in [0, 2^P) gets the
    logit (1/tau) * sum_j s_j(u) z_{lP+j}, with s_j(u) = +1 when bit j of u is
    set and -1 otherwise; the probabilities are the softmax of these 2^P
    logits. The top bucket's logit is |z_l|_1 / tau (the l1 magnitude the
    pages attribute to hard LSH), the distribution factorises into per-bit
    logistic terms that are linear in z for large tau (the small-signal
    regime of Lemma 4) and it tends to the hard bucket as tau -> 0
    (Theorem 3).
  * Projections are raw dot products: neither the query nor the hyperplanes
    are normalised.
  * Hash bit j of table l is 1 when the exact projection onto column lP+j is
    > 0 (a projection of exactly 0 gives 0); bit j carries weight 2^j. One R
    is shared by every batch entry and head.
  * The value-norm weight is the Euclidean norm of the value row, applied
    once after the L probabilities are summed.
  * GQA: query head h reads KV head floor(h / G), G = Hq / Hkv; tables,
    scores and the top-k are per query head.
  * Top-k ties go to the lower key index; exactly min(k, N) indices are
    returned, in ascending index order.
  * Attention over the subset uses the scale 1/sqrt(d), is renormalised over
    the subset only, and has no sink, window or causal mask.
  * Hard LSH (the tau -> 0 limit of the soft table): the limit puts equal
    mass on every bucket that maximises the logit, so a projection of exactly
    0 leaves its bit free and splits the mass 1/2 : 1/2 (sigma(0) = 1/2 at any
    tau); the hash itself still sends such a key projection to bit 0.
Parity status: every function below is pinned by the CPU tests in
tests/test_oracle.py (closed forms, limits, hand-worked examples, brute force
with exact rationals); none is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "hash_bits",
    "pack_bucket_ids",
    "hash_keys",
    "value_norms",
    "bucket_signs",
    "query_projections",
    "soft_bucket_probs",
    "soft_scores",
    "group_scores",
    "topk_indices",
    "subset_attention",
    "decode",
    "hard_query_buckets",
    "hard_bucket_table",
]

_U64 = 2.0 ** -53  # unit roundoff of float64


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Step 1: prefill hashing  [SOCKET-es, Mecanismo Central: LSH Suave, item 1]
#                          [SOCKET-de, Kernmechanismus, Vorverarbeitung]
# ---------------------------------------------------------------------------

def hash_bits(K, R, chunk: int = 1 << 16) -> np.ndarray:
    """Sign bit of every exact projection: True where K[n] . R[:, c] > 0.

    The float64 matmul is trusted only where its result is farther from zero
    than the worst-case summation error (d * u * sum_i |K_i R_ic|, doubled).
    Elsewhere the exact sum of the (exactly representable) products is taken
    with math.fsum, whose result is the correctly rounded exact sum, so its
    sign is the sign of the exact projection. Rows are processed in chunks
    only to bound memory.
    """
    K = np.asarray(K)
    R = _f64(R)
    d = K.shape[-1]
    rows = K.reshape(-1, d)
    bits = np.empty((rows.shape[0], R.shape[1]), dtype=bool)
    absR = np.abs(R)
    for start in range(0, rows.shape[0], chunk):
        Kc = _f64(rows[start:start + chunk])
        y = Kc @ R
        bound = 2.0 * d * _U64 * (np.abs(Kc) @ absR)
        b = y > 0
        for n, c in np.argwhere(np.abs(y) <= bound):
            exact = math.fsum((Kc[n, :] * R[:, c]).tolist())
            b[n, c] = exact > 0
        bits[start:start + chunk] = b
    return bits.reshape(*K.shape[:-1], R.shape[1])


def pack_bucket_ids(bits, L: int, P: int) -> np.ndarray:
    """Bucket id of table l = sum_j bits[..., l*P + j] * 2^j, as uint8."""
    bits = np.asarray(bits, dtype=bool)
    shape = bits.shape[:-1]
    b = bits.reshape(*shape, L, P).astype(np.int64)
    weights = np.left_shift(1, np.arange(P, dtype=np.int64))
    return (b * weights).sum(-1).astype(np.uint8)


def hash_keys(K, R, L: int, P: int) -> np.ndarray:
    """ids[..., n, l]: bucket of key n in table l (K [..., N, d], R [d, L*P])."""
    assert _f64(R).shape[-1] == L * P
    return pack_bucket_ids(hash_bits(K, R), L, P)


def value_norms(V) -> np.ndarray:
    """Euclidean norm of every value row, cached at prefill.

    [SOCKET-es, Mecanismo Central: LSH Suave, item 1]
    """
    V = _f64(V)
    return np.sqrt((V * V).sum(-1))


# ---------------------------------------------------------------------------
# Step 2: soft assignment  [SOCKET-es, Mecanismo Central: LSH Suave, item 2]
#                          [SOCKET-de, Kernmechanismus, Weiche Zuweisung]
# ---------------------------------------------------------------------------

def bucket_signs(P: int) -> np.ndarray:
    """S[u, j] = +1 if bit j of bucket u is set, else -1 (shape [2^P, P])."""
    u = np.arange(2 ** P)[:, None]
    j = np.arange(P)[None, :]
    return np.where((u >> j) & 1, 1.0, -1.0)


def query_projections(Q, R, L: int, P: int) -> np.ndarray:
    """z[..., l, j] = Q[...] . R[:, l*P + j] (raw, unnormalised)."""
    z = _f64(Q) @ _f64(R)
    return z.reshape(*z.shape[:-1], L, P)


def soft_bucket_probs(Q, R, L: int, P: int, tau: float) -> np.ndarray:
    """p[..., l, u]: softmax over the 2^P buckets of table l.

    logit(l, u) = (1/tau) * sum_j s_j(u) * z[l, j]; the maximum logit is
    subtracted before exponentiating.
    """
    z = query_projections(Q, R, L, P)
    logits = (z @ bucket_signs(P).T) / float(tau)
    logits = logits - logits.max(axis=-1, keepdims=True)
    e = np.exp(logits)
    return e / e.sum(axis=-1, keepdims=True)


def hard_query_buckets(Q, R, L: int, P: int) -> np.ndarray:
    """The query's own hard bucket per table, with the hash's convention:
    bit j is 1 when z[l, j] > 0 (a projection of exactly 0 gives bit 0)."""
    z = query_projections(Q, R, L, P)
    weights = np.left_shift(1, np.arange(P, dtype=np.int64))
    return ((z > 0).astype(np.int64) * weights).sum(-1)


def hard_bucket_table(Q, R, L: int, P: int) -> np.ndarray:
    """p0[..., l, u]: the tau -> 0 limit of soft_bucket_probs (hard LSH).

    [SOCKET-es, Fundamento Teórico, Teorema 3: as tau -> 0 the soft score
    becomes the hard collision count] [SOCKET-de, Theoretische Grundlage]

    The logit of bucket u, (1/tau) * sum_j s_j(u) z[l, j], is largest exactly
    for the buckets whose bit j equals [z[l, j] > 0] wherever z[l, j] != 0
    (bits with z[l, j] == 0 contribute 0 either way). As tau -> 0 the softmax
    puts equal mass on those maximisers and none elsewhere: with m exactly-zero
    projections in table l, each of the 2^m maximising buckets gets 2^-m. The
    maximisers are found from the signs, not by comparing rounded sums.
    """
    z = query_projections(Q, R, L, P)                     # [..., L, P]
    u = np.arange(2 ** P)
    bits = ((u[:, None] >> np.arange(P)[None, :]) & 1).astype(bool)  # [2^P, P]
    pos = (z > 0)[..., None, :]                           # [..., L, 1, P]
    zero = (z == 0)[..., None, :]
    agree = zero | (bits[None, :, :] == pos)              # [..., L, 2^P, P]
    maximiser = agree.all(axis=-1)                        # [..., L, 2^P]
    m = zero.sum(axis=-1)                                 # [..., L, 1]
    return np.where(maximiser, np.ldexp(1.0, -m), 0.0)


# ---------------------------------------------------------------------------
# Step 3: soft collision score  [SOCKET-es, Mecanismo Central: LSH Suave, 3]
#                               [SOCKET-de, Kernmechanismus, Bewertung]
# ---------------------------------------------------------------------------

def soft_scores(p, ids, vnorm, G: int) -> np.ndarray:
    """s[b, h, n] = vnorm[b, g, n] * sum_l p[b, h, l, ids[b, g, n, l]].

    p [B, Hq, L, 2^P]; ids [B, Hkv, N, L]; vnorm [B, Hkv, N]; g = h // G.
    """
    p = _f64(p)
    ids = np.asarray(ids)
    vnorm = _f64(vnorm)
    B, Hq, L, _ = p.shape
    N = ids.shape[2]
    out = np.empty((B, Hq, N), dtype=np.float64)
    tables = np.arange(L)[None, :]
    for b in range(B):
        for h in range(Hq):
            g = h // G
            mass = p[b, h][tables, ids[b, g].astype(np.intp)]  # [N, L]
            out[b, h] = vnorm[b, g] * mass.sum(axis=-1)
    return out


def group_scores(p, ids, vnorm, G: int) -> np.ndarray:
    """GQA group-shared score (a reading: the pages leave GQA open): for KV
    head g, the sum of the soft scores of the G query heads of its group,
    s[b, g, n] = sum_j soft_scores[b, g*G + j, n]; one top-k of these gives
    the group one shared index set.

    p [B, Hq, L, 2^P]; ids [B, Hkv, N, L]; vnorm [B, Hkv, N] -> [B, Hkv, N].
    """
    s = soft_scores(p, ids, vnorm, G)
    B, Hq, N = s.shape
    return s.reshape(B, Hq // G, G, N).sum(axis=2)


# ---------------------------------------------------------------------------
# Step 4: deterministic top-k  [SOCKET-es, Mecanismo Central: LSH Suave, 4]
#                              [SOCKET-de, Kernmechanismus, Auswahl]
# ---------------------------------------------------------------------------

def topk_indices(s, k: int) -> np.ndarray:
    """The min(k, N) keys with the largest score, ascending by index.

    Keys are ordered by (score descending, index ascending), so equal scores
    go to the lower index. s has shape [..., N].
    """
    s = np.asarray(s)
    N = s.shape[-1]
    kk = min(int(k), N)
    flat = s.reshape(-1, N)
    out = np.empty((flat.shape[0], kk), dtype=np.int64)
    index = np.arange(N)
    for r in range(flat.shape[0]):
        order = np.lexsort((index, -flat[r].astype(np.float64)))
        out[r] = np.sort(order[:kk])
    return out.reshape(*s.shape[:-1], kk)


# ---------------------------------------------------------------------------
# Step 5: exact attention over the subset  [SOCKET-es, LSH Suave, item 4]
#                                          [SOCKET-de, Auswahl]
# ---------------------------------------------------------------------------

def subset_attention(Q, K, V, idx, G: int) -> np.ndarray:
    """out[b, h] = sum_{i in S} softmax_i(q . k_i / sqrt(d)) v_i over S only.

    Q [B, Hq, d]; K, V [B, Hkv, N, d]; idx [B, Hq, kk].
    """
    Q = _f64(Q)
    K = _f64(K)
    V = _f64(V)
    idx = np.asarray(idx)
    B, Hq, d = Q.shape
    out = np.empty((B, Hq, d), dtype=np.float64)
    scale = 1.0 / math.sqrt(d)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            sel = idx[b, h].astype(np.intp)
            a = (K[b, g, sel] @ Q[b, h]) * scale
            a = a - a.max()
            w = np.exp(a)
            w = w / w.sum()
            out[b, h] = w @ V[b, g, sel]
    return out


def decode(Q, K, V, R, ids, vnorm, L: int, P: int, tau: float, k: int):
    """One decode step: (out, idx, scores, probs)."""
    Q = _f64(Q)
    G = Q.shape[1] // np.asarray(ids).shape[1]
    p = soft_bucket_probs(Q, R, L, P, tau)
    s = soft_scores(p, ids, vnorm, G)
    idx = topk_indices(s, k)
    out = subset_attention(Q, K, V, idx, G)
    return out, idx, s, p
