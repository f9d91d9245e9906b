"""Python binding of the SOCKET decode library (argument marshalling only).

Every function takes contiguous torch tensors that live on a ROCm device,
passes their device pointers and the current HIP stream to the C ABI and
returns the outputs it allocated with torch. All computation happens in the
HIP kernels; nothing here falls back to the CPU.
"""

from __future__ import annotations

import torch

from . import _lib
from ._lib import DTYPE_BF16, DTYPE_F32, check

_DTYPES = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)") from None


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a ROCm device (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _expect(t, name: str, shape, dtype=None) -> None:
    """Shape and dtype check of an argument before its pointer reaches the C
    ABI, which cannot see either (a wrong one would be read or written out of
    bounds on the device)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _heads(Hq: int, Hkv: int) -> int:
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    return Hq // Hkv


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def hash_keys(K: torch.Tensor, V: torch.Tensor, R: torch.Tensor, L: int,
              P: int, n_keys: int | None = None, ids: torch.Tensor | None = None,
              vnorm: torch.Tensor | None = None, row_offset: int = 0):
    """Prefill hashing. K, V: [..., S, d] (S = head stride rows), R: [d, L*P].

    Returns (ids uint8 [..., S, L], vnorm float32 [..., S]). Rows
    [row_offset, row_offset + n_keys) of every head are hashed (default: all
    S rows); pass the existing ids / vnorm to append to a cache.
    """
    lib = _lib.load()
    _dtype_code(K)
    if K.dim() < 2:
        raise ValueError("K must be [..., S, d]")
    _expect(V, "V", K.shape, K.dtype)
    *lead, S, d = K.shape
    _expect(R, "R", (d, L * P), K.dtype)
    n_heads = 1
    for x in lead:
        n_heads *= x
    o = int(row_offset)
    n = S - o if n_keys is None else int(n_keys)
    if o < 0 or n < 0 or o + n > S:
        raise ValueError(f"rows [{o}, {o + n}) do not fit the {S} rows per head")
    if ids is None:
        ids = torch.empty((*lead, S, L), dtype=torch.uint8, device=K.device)
    if vnorm is None:
        vnorm = torch.empty((*lead, S), dtype=torch.float32, device=K.device)
    _expect(ids, "ids", (*lead, S, L), torch.uint8)
    _expect(vnorm, "vnorm", (*lead, S), torch.float32)
    esz = K.element_size()
    dt = _dtype_code(K)
    ws_bytes = lib.socket_hash_keys_workspace_bytes(dt, n_heads, n, d, L, P)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=K.device)
    st = lib.socket_hash_keys(_dev(K, "K") + o * d * esz, _dev(V, "V") + o * d * esz,
                              _dev(R, "R"), dt, n_heads, n, S, d, L, P,
                              _dev(ids, "ids") + o * L, _dev(vnorm, "vnorm") + o * 4,
                              ws.data_ptr() if ws_bytes else None, ws_bytes, _stream(K))
    check(st, "socket_hash_keys")
    return ids, vnorm


def bucket_probs(Q: torch.Tensor, R: torch.Tensor, Hkv: int, L: int, P: int,
                 tau: float) -> torch.Tensor:
    """Soft bucket table [B, Hkv, 2^P, L, G] (float32) for queries Q [B, Hq, d]."""
    lib = _lib.load()
    B, Hq, d = Q.shape
    G = _heads(Hq, Hkv)
    _expect(R, "R", (d, L * P), Q.dtype)
    table = torch.empty((B, Hkv, 2 ** P, L, G), dtype=torch.float32, device=Q.device)
    st = lib.socket_bucket_probs(_dev(Q, "Q"), _dev(R, "R"), _dtype_code(Q), B,
                                 Hq, Hkv, d, L, P, float(tau),
                                 _dev(table, "table"), _stream(Q))
    check(st, "socket_bucket_probs")
    return table


def hard_bucket_table(Q: torch.Tensor, R: torch.Tensor, Hkv: int, L: int,
                      P: int) -> torch.Tensor:
    """One-hot table [B, Hkv, 2^P, L, G] (float32) at the queries' own buckets:
    the tau -> 0 limit of bucket_probs (hard LSH)."""
    lib = _lib.load()
    B, Hq, d = Q.shape
    G = _heads(Hq, Hkv)
    _expect(R, "R", (d, L * P), Q.dtype)
    table = torch.empty((B, Hkv, 2 ** P, L, G), dtype=torch.float32, device=Q.device)
    st = lib.socket_hard_bucket_table(_dev(Q, "Q"), _dev(R, "R"), _dtype_code(Q), B, Hq, Hkv,
                                      d, L, P, _dev(table, "table"), _stream(Q))
    check(st, "socket_hard_bucket_table")
    return table


def score(table: torch.Tensor, ids: torch.Tensor, vnorm: torch.Tensor,
          Hq: int, n_keys: int | None = None) -> torch.Tensor:
    """Soft collision scores [B, Hq, n_keys] from a table and the hash cache.

    table [B, Hkv, 2^P, L, G]; ids [B, Hkv, S, L]; vnorm [B, Hkv, S].
    """
    lib = _lib.load()
    _expect(table, "table", None, torch.float32)
    if table.dim() != 5:
        raise ValueError("table must be [B, Hkv, 2^P, L, G]")
    B, Hkv, nb, L, G = table.shape
    P = nb.bit_length() - 1
    if nb != 1 << P or Hq != Hkv * G:
        raise ValueError(f"table {tuple(table.shape)} does not fit Hq={Hq} (2^P buckets, "
                         "G = Hq / Hkv heads per slot)")
    if ids.dim() != 4:
        raise ValueError("ids must be [B, Hkv, S, L]")
    S = ids.shape[-2]
    _expect(ids, "ids", (B, Hkv, S, L), torch.uint8)
    _expect(vnorm, "vnorm", (B, Hkv, S), torch.float32)
    n = S if n_keys is None else int(n_keys)
    if not 0 <= n <= S:
        raise ValueError(f"n_keys={n} outside [0, {S}]")
    scores = torch.empty((B, Hq, n), dtype=torch.float32, device=table.device)
    st = lib.socket_score(_dev(table, "table"), _dev(ids, "ids"),
                          _dev(vnorm, "vnorm"), B, Hq, Hkv, n, S, L, P,
                          _dev(scores, "scores"), _stream(table))
    check(st, "socket_score")
    return scores


def topk(scores: torch.Tensor, k: int) -> torch.Tensor:
    """Deterministic top-k of each row of scores [..., n] -> int32 [..., min(k, n)]."""
    lib = _lib.load()
    _expect(scores, "scores", None, torch.float32)
    *lead, n = scores.shape
    rows = 1
    for x in lead:
        rows *= x
    kk = min(int(k), n)
    idx = torch.empty((*lead, kk), dtype=torch.int32, device=scores.device)
    ws = _workspace(lib.socket_topk_workspace_bytes(rows, n, int(k)), scores.device)
    st = lib.socket_topk(_dev(scores, "scores"), rows, n, int(k), _dev(idx, "idx"),
                         ws.data_ptr(), ws.numel(), _stream(scores))
    check(st, "socket_topk")
    return idx


def sparse_attn(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                idx: torch.Tensor) -> torch.Tensor:
    """Attention of Q [B, Hq, d] over the keys idx [B, Hq, kk] of K, V [B, Hkv, S, d]."""
    lib = _lib.load()
    _dtype_code(Q)
    B, Hq, d = Q.shape
    if K.dim() != 4:
        raise ValueError("K must be [B, Hkv, S, d]")
    _, Hkv, S, _ = K.shape
    _heads(Hq, Hkv)
    _expect(K, "K", (B, Hkv, S, d), Q.dtype)
    _expect(V, "V", (B, Hkv, S, d), Q.dtype)
    kk = idx.shape[-1]
    _expect(idx, "idx", (B, Hq, kk), torch.int32)
    out = torch.empty_like(Q)
    ws = _workspace(lib.socket_sparse_attn_workspace_bytes(B, Hq, d, kk), Q.device)
    st = lib.socket_sparse_attn(_dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"),
                                _dtype_code(Q), B, Hq, Hkv, d, S, _dev(idx, "idx"),
                                kk, _dev(out, "out"), ws.data_ptr(), ws.numel(),
                                _stream(Q))
    check(st, "socket_sparse_attn")
    return out


def dense_attn(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
               n: int | None = None) -> torch.Tensor:
    """Dense attention of Q [B, Hq, d] over the first n keys of K, V [B, Hkv, S, d]."""
    lib = _lib.load()
    _dtype_code(Q)
    B, Hq, d = Q.shape
    if K.dim() != 4:
        raise ValueError("K must be [B, Hkv, S, d]")
    _, Hkv, S, _ = K.shape
    _heads(Hq, Hkv)
    _expect(K, "K", (B, Hkv, S, d), Q.dtype)
    _expect(V, "V", (B, Hkv, S, d), Q.dtype)
    n = S if n is None else int(n)
    out = torch.empty_like(Q)
    ws = _workspace(lib.socket_dense_attn_workspace_bytes(B, Hq, d, n), Q.device)
    st = lib.socket_dense_attn(_dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _dtype_code(Q),
                               B, Hq, Hkv, d, n, S, _dev(out, "out"), ws.data_ptr(),
                               ws.numel(), _stream(Q))
    check(st, "socket_dense_attn")
    return out


def _check_decode_args(Q, K, V, R, ids, vnorm, L, P, k, n_keys, out, idx_out, scores_out,
                       group_shared):
    """Shapes and dtypes of a decode call; returns (B, Hq, Hkv, d, S, n)."""
    _dtype_code(Q)
    if Q.dim() != 3 or K.dim() != 4:
        raise ValueError("Q must be [B, Hq, d] and K [B, Hkv, S, d]")
    B, Hq, d = Q.shape
    _, Hkv, S, _ = K.shape
    _heads(Hq, Hkv)
    _expect(K, "K", (B, Hkv, S, d), Q.dtype)
    _expect(V, "V", (B, Hkv, S, d), Q.dtype)
    _expect(R, "R", (d, L * P), Q.dtype)
    _expect(ids, "ids", (B, Hkv, S, L), torch.uint8)
    _expect(vnorm, "vnorm", (B, Hkv, S), torch.float32)
    n = S if n_keys is None else int(n_keys)
    if not 1 <= n <= S:
        raise ValueError(f"n_keys={n} outside [1, {S}]")
    rows = Hkv if group_shared else Hq
    if out is not None:
        _expect(out, "out", (B, Hq, d), Q.dtype)
    if idx_out is not None:
        _expect(idx_out, "idx_out", (B, rows, min(int(k), n)), torch.int32)
    if scores_out is not None:
        _expect(scores_out, "scores_out", (B, rows, n), torch.float32)
    return B, Hq, Hkv, d, S, n


def decode_workspace_bytes(B: int, Hq: int, Hkv: int, d: int, n_keys: int,
                           L: int, P: int, k: int) -> int:
    return int(_lib.load().socket_decode_workspace_bytes(B, Hq, Hkv, d, n_keys, L, P, k))


def decode(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, R: torch.Tensor,
           ids: torch.Tensor, vnorm: torch.Tensor, L: int, P: int, tau: float,
           k: int, n_keys: int | None = None, out: torch.Tensor | None = None,
           idx_out: torch.Tensor | None = None,
           scores_out: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None):
    """One decode step; returns (out, idx_out, scores_out).

    Q [B, Hq, d]; K, V [B, Hkv, S, d]; R [d, L*P]; ids [B, Hkv, S, L];
    vnorm [B, Hkv, S]. idx_out / scores_out are returned only if given.
    A workspace of decode_workspace_bytes(...) bytes may be passed to avoid
    an allocation per call.
    """
    lib = _lib.load()
    B, Hq, Hkv, d, S, n = _check_decode_args(Q, K, V, R, ids, vnorm, L, P, k, n_keys, out,
                                             idx_out, scores_out, False)
    if out is None:
        out = torch.empty_like(Q)
    need = lib.socket_decode_workspace_bytes(B, Hq, Hkv, d, n, L, P, int(k))
    if workspace is None:
        workspace = _workspace(need, Q.device)
    _expect(workspace, "workspace", None, torch.uint8)
    st = lib.socket_decode(
        _dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _dev(R, "R"), _dev(ids, "ids"),
        _dev(vnorm, "vnorm"), _dtype_code(Q), B, Hq, Hkv, d, n, S, L, P,
        float(tau), int(k), _dev(out, "out"),
        _dev(idx_out, "idx_out") if idx_out is not None else None,
        _dev(scores_out, "scores_out") if scores_out is not None else None,
        _dev(workspace, "workspace"), workspace.numel(), _stream(Q))
    check(st, "socket_decode")
    return out, idx_out, scores_out


def decode_group_shared(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, R: torch.Tensor,
                        ids: torch.Tensor, vnorm: torch.Tensor, L: int, P: int, tau: float,
                        k: int, n_keys: int | None = None, out: torch.Tensor | None = None,
                        idx_out: torch.Tensor | None = None,
                        scores_out: torch.Tensor | None = None):
    """GQA group-shared variant of decode: one index set [B, Hkv, kk] per KV
    head from the group's summed scores; returns (out, idx_out, scores_out)."""
    lib = _lib.load()
    B, Hq, Hkv, d, S, n = _check_decode_args(Q, K, V, R, ids, vnorm, L, P, k, n_keys, out,
                                             idx_out, scores_out, True)
    if out is None:
        out = torch.empty_like(Q)
    need = lib.socket_decode_group_shared_workspace_bytes(B, Hq, Hkv, d, n, L, P, int(k))
    ws = _workspace(need, Q.device)
    st = lib.socket_decode_group_shared(
        _dev(Q, "Q"), _dev(K, "K"), _dev(V, "V"), _dev(R, "R"), _dev(ids, "ids"),
        _dev(vnorm, "vnorm"), _dtype_code(Q), B, Hq, Hkv, d, n, S, L, P, float(tau), int(k),
        _dev(out, "out"), _dev(idx_out, "idx_out") if idx_out is not None else None,
        _dev(scores_out, "scores_out") if scores_out is not None else None,
        _dev(ws, "workspace"), ws.numel(), _stream(Q))
    check(st, "socket_decode_group_shared")
    return out, idx_out, scores_out
