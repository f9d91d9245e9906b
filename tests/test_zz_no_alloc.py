"""The allocation-free decode entry point against socket_decode.

socket_decode_noalloc runs the same kernels as socket_decode with the
workspace in the library's own device array, so its outputs (attention,
selected indices, score rows) must equal socket_decode's bit for bit. Two
calls in a row on the same GPU, the second smaller than the first (the array
keeps the first call's contents), both through the C ABI; then a call too
large for the array is rejected on the host."""

import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle as O
import soft_lsh_sparse_amd as S
import synthetic as W
from soft_lsh_sparse_amd import _lib

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _call(lib, fn, w, Q, K, V, R, ids, vn, out, idx, sc, ws=None):
    args = [Q.data_ptr(), K.data_ptr(), V.data_ptr(), R.data_ptr(), ids.data_ptr(),
            vn.data_ptr(), _lib.DTYPE_BF16 if w.dtype == "bf16" else _lib.DTYPE_F32,
            w.B, w.Hq, w.Hkv, w.d, w.N, w.N, w.L, w.P, w.tau, w.k, out.data_ptr(),
            _ptr(idx), _ptr(sc)]
    if ws is not None:
        args += [ws.data_ptr(), ws.numel()]
    args.append(torch.cuda.current_stream().cuda_stream)
    return fn(*args)


def _run_both(lib, w, seed):
    Q, K, V, R = W.make_decode_inputs(w, DEV, seed=seed)
    ids, vn = S.hash_keys(K, V, R, w.L, w.P)
    outs = []
    for fn in ("socket_decode", "socket_decode_noalloc"):
        out = torch.empty_like(Q)
        idx = torch.empty((w.B, w.Hq, w.kk), dtype=torch.int32, device=DEV)
        sc = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=DEV)
        idx2 = torch.empty((w.B, w.Hq, w.kk), dtype=torch.int32, device=DEV)
        out2 = torch.empty_like(Q)
        ws = None
        if fn == "socket_decode":
            ws = torch.empty(lib.socket_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.N, w.L,
                                                               w.P, w.k), dtype=torch.uint8,
                             device=DEV)
        # with score rows, then the benched form (no score rows)
        st = _call(lib, getattr(lib, fn), w, Q, K, V, R, ids, vn, out, idx, sc, ws)
        _lib.check(st, fn)
        st = _call(lib, getattr(lib, fn), w, Q, K, V, R, ids, vn, out2, idx2, None, ws)
        _lib.check(st, fn)
        torch.cuda.synchronize()
        outs.append((out, idx, sc, out2, idx2))
    return Q, K, V, outs


def test_noalloc_decode_equals_decode_on_two_calls_in_a_row():
    lib = _lib.load()
    big = W.WORKLOADS["llama3_8b_32k"]
    small = W.custom_workload(B=2, Hq=8, Hkv=2, d=128, N=5000, dtype="bf16", L=32, P=8,
                              tau=0.3, k=300, outlier_channels=4, outlier_scale=8.0,
                              lognormal_v=True, planted=16, name="noalloc_small")
    for w, seed in ((big, 21), (small, 22)):
        need = lib.socket_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.N, w.L, w.P, w.k)
        assert need <= _lib.DECODE_NOALLOC_SCRATCH_BYTES
        _log(f"noalloc decode {w.name} (workspace {need} bytes)")
        Q, K, V, outs = _run_both(lib, w, seed)
        (o_ref, i_ref, s_ref, o2_ref, i2_ref), (o, i, s, o2, i2) = outs
        assert torch.equal(i, i_ref), f"{w.name}: selected indices differ"
        assert torch.equal(s, s_ref), f"{w.name}: score rows differ"
        assert torch.equal(o, o_ref), f"{w.name}: attention outputs differ"
        assert torch.equal(i2, i_ref) and torch.equal(o2, o_ref), f"{w.name}: benched form"
        # and the selection is the oracle's on those scores
        sc_np = s.cpu().numpy()
        assert np.array_equal(i.cpu().numpy(), O.topk_indices(sc_np, w.k))


def test_noalloc_decode_gathers_large_k():
    """k large enough that the selection gathers each row's candidates into
    the workspace first (inside the device array here): same results as
    socket_decode, then a smaller call."""
    lib = _lib.load()
    big = W.custom_workload(B=1, Hq=8, Hkv=2, d=128, N=30000, dtype="bf16", L=32, P=8,
                            tau=0.3, k=6000, lognormal_v=True, name="noalloc_gathered")
    small = W.custom_workload(B=1, Hq=4, Hkv=1, d=128, N=20000, dtype="bf16", L=32, P=8,
                              tau=0.3, k=5500, lognormal_v=True, name="noalloc_gathered_small")
    for w, seed in ((big, 23), (small, 24)):
        assert lib.socket_decode_kernels(0x1000, _lib.DTYPE_BF16, w.B, w.Hq, w.Hkv, w.d, w.N,
                                         w.N, w.L, w.P, w.k, 0, None, 0) == 5  # + gather
        _log(f"noalloc decode {w.name}")
        Q, K, V, outs = _run_both(lib, w, seed)
        (o_ref, i_ref, s_ref, o2_ref, i2_ref), (o, i, s, o2, i2) = outs
        assert torch.equal(i, i_ref) and torch.equal(s, s_ref) and torch.equal(o, o_ref)
        assert torch.equal(i2, i_ref) and torch.equal(o2, o_ref), f"{w.name}: benched form"
        assert np.array_equal(i.cpu().numpy(), O.topk_indices(s.cpu().numpy(), w.k))


def test_noalloc_decode_rejects_a_call_larger_than_its_array():
    lib = _lib.load()
    w = W.WORKLOADS["llama3_8b_128k_b4"]
    need = lib.socket_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.N, w.L, w.P, w.k)
    assert need > _lib.DECODE_NOALLOC_SCRATCH_BYTES
    fake = 0x1000  # never dereferenced: the size check comes first
    st = lib.socket_decode_noalloc(fake, fake, fake, fake, fake, fake, _lib.DTYPE_BF16, w.B,
                                   w.Hq, w.Hkv, w.d, w.N, w.N, w.L, w.P, w.tau, w.k, fake,
                                   None, None, None)
    assert st == _lib.SOCKET_ERR_UNSUPPORTED
    assert b"device array" in lib.socket_last_error()
