"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/socket_lsh.h, and rejects invalid arguments on the host
before anything is enqueued (fake non-null pointers are never dereferenced
because validation fails first)."""

import ctypes
import os
import re

import pytest

from soft_lsh_sparse_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x1000  # 16-byte aligned, never dereferenced (validation fails first)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "socket_lsh.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(socket_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_typed(lib):
    names = _declared_functions()
    assert len(names) >= 12
    for name in names:
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"{name} has no ctypes signature"
    assert set(_lib.SIGNATURES) == set(names)


def test_version_and_status_strings(lib):
    assert lib.socket_version() == (0 << 16) | (1 << 8) | 0
    for st in range(5):
        assert lib.socket_status_string(st)
    assert lib.socket_status_string(99) == b"unknown status"


def _decode(lib, **over):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, R=FAKE, ids=FAKE, vnorm=FAKE, dt=1, B=1,
             Hq=32, Hkv=8, d=128, n=1024, stride=1024, L=32, P=8, tau=0.3,
             k=64, out=FAKE, idx=None, scores=None, ws=FAKE, ws_bytes=0)
    a.update(over)
    return lib.socket_decode(a["Q"], a["K"], a["V"], a["R"], a["ids"], a["vnorm"],
                             a["dt"], a["B"], a["Hq"], a["Hkv"], a["d"], a["n"],
                             a["stride"], a["L"], a["P"], a["tau"], a["k"],
                             a["out"], a["idx"], a["scores"], a["ws"],
                             a["ws_bytes"], None)


@pytest.mark.parametrize("over,status", [
    (dict(dt=7), _lib.SOCKET_ERR_INVALID_ARGUMENT),
    (dict(Hq=30), _lib.SOCKET_ERR_INVALID_ARGUMENT),
    (dict(Hq=48, Hkv=8), _lib.SOCKET_ERR_UNSUPPORTED),       # G = 6
    (dict(d=96), _lib.SOCKET_ERR_UNSUPPORTED),
    (dict(d=0), _lib.SOCKET_ERR_INVALID_ARGUMENT),
    (dict(P=0), _lib.SOCKET_ERR_INVALID_ARGUMENT),
    (dict(P=9), _lib.SOCKET_ERR_INVALID_ARGUMENT),
    (dict(L=0), _lib.SOCKET_ERR_INVALID_ARGUMENT),
    (dict(L=200, P=8), _lib.SOCKET_ERR_UNSUPPORTED),         # L*P > 1024
    (dict(tau=0.0), _lib.SOCKET_ERR_INVALID_ARGUMENT),
    (dict(tau=-1.0), _lib.SOCKET_ERR_INVALID_ARGUMENT),
    (dict(tau=float("inf")), _lib.SOCKET_ERR_INVALID_ARGUMENT),
    (dict(tau=float("nan")), _lib.SOCKET_ERR_INVALID_ARGUMENT),
    (dict(k=0), _lib.SOCKET_ERR_INVALID_ARGUMENT),
    (dict(n=0), _lib.SOCKET_ERR_INVALID_ARGUMENT),
    (dict(stride=100), _lib.SOCKET_ERR_INVALID_ARGUMENT),    # stride < n
    (dict(Q=None), _lib.SOCKET_ERR_INVALID_ARGUMENT),
    (dict(ids=None), _lib.SOCKET_ERR_INVALID_ARGUMENT),
    (dict(out=None), _lib.SOCKET_ERR_INVALID_ARGUMENT),
    (dict(K=FAKE + 2), _lib.SOCKET_ERR_INVALID_ARGUMENT),    # misaligned
    (dict(ws=None), _lib.SOCKET_ERR_WORKSPACE),
    (dict(ws_bytes=1000), _lib.SOCKET_ERR_WORKSPACE),
])
def test_decode_rejects_bad_arguments(lib, over, status):
    assert _decode(lib, **over) == status
    assert lib.socket_last_error()


def test_decode_packs_query_heads_when_the_group_table_overflows_lds(lib):
    """L=64, P=8, G=4 needs 256 KB for a group's tables: the score blocks then
    take 2 query heads each (G-pack) instead of the call being rejected. The
    host-only launch query and the workspace check show the call accepted
    (the fake pointers are never used)."""
    n, names = _kernels(lib, L=64, P=8)
    assert n == 5 and names[:3] == ["bucket_probs_kernel", "score_kernel",
                                    "topk_select_kernel"]
    assert _kernels(lib, L=128, P=8, Hq=64, Hkv=8)[0] == 5     # G = 8 -> one head per block
    assert _decode(lib, L=64, P=8) == _lib.SOCKET_ERR_WORKSPACE   # accepted up to the workspace
    ws = lib.socket_decode_workspace_bytes(1, 32, 8, 128, 1024, 64, 8, 64)
    assert ws >= 256 * 64 * 32 * 4                                   # tables of all 32 heads


def _group(lib, **over):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, R=FAKE, ids=FAKE, vnorm=FAKE, dt=1, B=1,
             Hq=4, Hkv=1, d=128, n=1024, stride=1024, L=32, P=8, tau=0.3,
             k=64, out=FAKE, idx=None, scores=None, ws=FAKE, ws_bytes=0)
    a.update(over)
    return lib.socket_decode_group_shared(
        a["Q"], a["K"], a["V"], a["R"], a["ids"], a["vnorm"], a["dt"], a["B"], a["Hq"],
        a["Hkv"], a["d"], a["n"], a["stride"], a["L"], a["P"], a["tau"], a["k"], a["out"],
        a["idx"], a["scores"], a["ws"], a["ws_bytes"], None)


def test_group_shared_checks_the_geometry_it_launches(lib):
    """The group-shared variant scores one summed table per KV head, so its
    score kernel fits twice the blocks per CU of the per-head kernel: with
    one KV head and 600,000 keys that geometry needs more candidate sub-lists
    per row than the selection holds (the per-head geometry would not). The
    call must be rejected on the host, before any launch."""
    n = 600_000
    assert _group(lib, n=n, stride=n) == _lib.SOCKET_ERR_UNSUPPORTED
    assert b"sub-lists" in lib.socket_last_error()
    # the per-head decode of the same shape is within its own geometry
    assert _decode(lib, Hq=4, Hkv=1, n=n, stride=n) == _lib.SOCKET_ERR_WORKSPACE
    # a shape within both geometries reaches the workspace check
    assert _group(lib, n=400_000, stride=400_000) == _lib.SOCKET_ERR_WORKSPACE


def test_decode_profiled_needs_an_event_pair(lib):
    ws_bytes = lib.socket_decode_workspace_bytes(1, 32, 8, 128, 1024, 32, 8, 64)
    events = (ctypes.c_void_p * 1)(FAKE)
    st = lib.socket_decode_profiled(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 32, 8,
                                    128, 1024, 1024, 32, 8, 0.3, 64, FAKE, None,
                                    None, FAKE, ws_bytes, None, events, 1)
    assert st == _lib.SOCKET_ERR_INVALID_ARGUMENT
    assert b"n_events" in lib.socket_last_error()


def test_hash_keys_validation(lib):
    f = lib.socket_hash_keys
    ws = lib.socket_hash_keys_workspace_bytes(1, 8, 1024, 128, 64, 8)
    assert ws > 0 and lib.socket_hash_keys_workspace_bytes(0, 8, 1024, 128, 64, 8) == 0
    ok_args = [FAKE, FAKE, FAKE, 1, 8, 1024, 1024, 128, 64, 8, FAKE, FAKE, FAKE, ws, None]
    bad = list(ok_args); bad[7] = 80
    assert f(*bad) == _lib.SOCKET_ERR_UNSUPPORTED
    bad = list(ok_args); bad[9] = 9
    assert f(*bad) == _lib.SOCKET_ERR_INVALID_ARGUMENT
    bad = list(ok_args); bad[8] = 128          # L*P = 1024 > 512 for bf16
    assert f(*bad) == _lib.SOCKET_ERR_UNSUPPORTED
    bad = list(ok_args); bad[6] = 10           # stride < n_keys
    assert f(*bad) == _lib.SOCKET_ERR_INVALID_ARGUMENT
    bad = list(ok_args); bad[10] = None
    assert f(*bad) == _lib.SOCKET_ERR_INVALID_ARGUMENT
    bad = list(ok_args); bad[0] = FAKE + 4
    assert f(*bad) == _lib.SOCKET_ERR_INVALID_ARGUMENT
    bad = list(ok_args); bad[2] = FAKE + 8     # R must be 16-byte aligned
    assert f(*bad) == _lib.SOCKET_ERR_INVALID_ARGUMENT
    bad = list(ok_args); bad[13] = ws - 1      # workspace too small
    assert f(*bad) == _lib.SOCKET_ERR_WORKSPACE
    bad = list(ok_args); bad[12] = FAKE + 16   # workspace not 256-byte aligned
    assert f(*bad) == _lib.SOCKET_ERR_WORKSPACE
    bad = list(ok_args); bad[12] = None
    assert f(*bad) == _lib.SOCKET_ERR_WORKSPACE
    # nothing to hash: OK without touching any pointer or the GPU
    empty = list(ok_args); empty[5] = 0
    assert f(*empty) == _lib.SOCKET_OK
    empty = [None, None, None, 1, 0, 5, 5, 128, 64, 8, None, None, None, 0, None]
    assert f(*empty) == _lib.SOCKET_OK


def test_stage_validation(lib):
    assert lib.socket_bucket_probs(FAKE, FAKE, 1, 1, 32, 8, 128, 32, 8, 0.0,
                                   FAKE, None) == _lib.SOCKET_ERR_INVALID_ARGUMENT
    assert lib.socket_score(FAKE, FAKE, FAKE, 1, 32, 8, 10, 5, 32, 8, FAKE,
                            None) == _lib.SOCKET_ERR_INVALID_ARGUMENT
    assert lib.socket_topk(FAKE, 4, 100, 0, FAKE, FAKE, 1 << 30,
                           None) == _lib.SOCKET_ERR_INVALID_ARGUMENT
    assert lib.socket_topk(FAKE, 4, 100, 10, FAKE, None, 0,
                           None) == _lib.SOCKET_ERR_WORKSPACE
    assert lib.socket_topk(None, 0, 100, 10, None, None, 0, None) == _lib.SOCKET_OK
    assert lib.socket_sparse_attn(FAKE, FAKE, FAKE, 1, 1, 32, 8, 128, 1024, FAKE,
                                  0, FAKE, FAKE, 1 << 30,
                                  None) == _lib.SOCKET_ERR_INVALID_ARGUMENT
    assert lib.socket_sparse_attn(FAKE, FAKE, FAKE, 1, 1, 32, 8, 128, 1024, FAKE,
                                  16, FAKE, FAKE, 4,
                                  None) == _lib.SOCKET_ERR_WORKSPACE


def test_workspace_sizes_are_sane(lib):
    # 128K-key decode, batch 4, 32/8 heads, L=32, P=8, k=4096
    ws = lib.socket_decode_workspace_bytes(4, 32, 8, 128, 131072, 32, 8, 4096)
    rows, n = 4 * 32, 131072
    assert ws >= rows * n * 4          # scores
    assert ws < 512 * 1024 * 1024
    assert lib.socket_decode_workspace_bytes(0, 32, 8, 128, 1, 32, 8, 1) == 0
    assert lib.socket_topk_workspace_bytes(128, 131072, 4096) >= 128 * 2048 * 4
    assert lib.socket_sparse_attn_workspace_bytes(4, 32, 128, 4096) >= 4 * 32 * 130 * 4


def _kernels(lib, ids=FAKE, dtype=_lib.DTYPE_BF16, B=4, Hq=32, Hkv=8, d=128, N=131072,
             L=32, P=8, k=4096, with_scores=0, cap=512):
    buf = ctypes.create_string_buffer(cap)
    n = lib.socket_decode_kernels(ids, dtype, B, Hq, Hkv, d, N, N, L, P, k, with_scores,
                                  buf, cap)
    return n, buf.value.decode().split(",") if n > 0 else []


def test_decode_kernel_sequence(lib):
    """The launch sequence socket_decode reports (host-only query): the score
    kernel builds the tables itself for bf16, P = 8, aligned id rows; the
    table kernel runs otherwise; k >= n_keys skips selection."""
    tail = ["sparse_attn_kernel", "attn_merge_kernel"]
    assert _kernels(lib) == (4, ["score_kernel", "topk_select_kernel"] + tail)
    n, names = _kernels(lib, dtype=_lib.DTYPE_F32)
    assert names == ["bucket_probs_kernel", "score_kernel", "topk_select_kernel"] + tail
    assert n == 5
    assert _kernels(lib, P=6)[1][0] == "bucket_probs_kernel"
    assert _kernels(lib, ids=FAKE + 8)[1][0] == "bucket_probs_kernel"  # unaligned id rows
    assert _kernels(lib, L=24, P=8)[1][0] == "bucket_probs_kernel"     # not the rotated path
    # large k: the candidates are gathered before the select
    gathered = ["score_kernel", "topk_gather_kernel", "topk_select_kernel"] + tail
    assert _kernels(lib, k=16384) == (5, gathered)
    assert _kernels(lib, k=5462)[1] == gathered
    assert _kernels(lib, k=5461)[1] == ["score_kernel", "topk_select_kernel"] + tail
    assert _kernels(lib, k=131072) == (3, ["iota_rows_kernel"] + tail)
    assert _kernels(lib, k=131072, with_scores=1)[1] == ["score_kernel", "iota_rows_kernel"] + tail
    # a row of one chunk (at most 256 keys with 4 waves): no merge kernel
    assert _kernels(lib, B=1, Hq=1, Hkv=1, k=64)[1][-2:] == ["topk_select_kernel",
                                                             "sparse_attn_kernel"]
    assert _kernels(lib, B=1, Hq=1, Hkv=1, k=257)[1][-1] == "attn_merge_kernel"
    assert _kernels(lib, Hq=30)[0] == -1      # G not an integer
    assert _kernels(lib, cap=8)[0] == -2      # names do not fit
    assert lib.socket_decode_kernels(FAKE, _lib.DTYPE_BF16, 4, 32, 8, 128, 131072, 131072,
                                     32, 8, 4096, 0, None, 0) == 4


def _dense(lib, **over):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, dt=1, B=1, Hq=32, Hkv=8, d=128, n=1024,
             stride=1024, out=FAKE, ws=FAKE, ws_bytes=0)
    a.update(over)
    return lib.socket_dense_attn(a["Q"], a["K"], a["V"], a["dt"], a["B"], a["Hq"],
                                 a["Hkv"], a["d"], a["n"], a["stride"], a["out"],
                                 a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("over,status", [
    (dict(dt=7), _lib.SOCKET_ERR_INVALID_ARGUMENT),
    (dict(Hq=30), _lib.SOCKET_ERR_INVALID_ARGUMENT),
    (dict(d=96), _lib.SOCKET_ERR_UNSUPPORTED),
    (dict(n=0), _lib.SOCKET_ERR_INVALID_ARGUMENT),
    (dict(n=(1 << 20) + 1, stride=(1 << 20) + 1), _lib.SOCKET_ERR_UNSUPPORTED),
    (dict(stride=100), _lib.SOCKET_ERR_INVALID_ARGUMENT),    # stride < n
    (dict(Q=None), _lib.SOCKET_ERR_INVALID_ARGUMENT),
    (dict(out=None), _lib.SOCKET_ERR_INVALID_ARGUMENT),
    (dict(V=FAKE + 4), _lib.SOCKET_ERR_INVALID_ARGUMENT),    # misaligned
    (dict(ws=None), _lib.SOCKET_ERR_WORKSPACE),
    (dict(ws_bytes=1000), _lib.SOCKET_ERR_WORKSPACE),
])
def test_dense_attn_rejects_invalid_arguments(lib, over, status):
    assert _dense(lib, **over) == status


def test_dense_attn_workspace_covers_every_chunk(lib):
    # partials of (m, l, acc[d]) per query row and 1024-key chunk
    assert lib.socket_dense_attn_workspace_bytes(4, 32, 128, 131072) == 4 * 32 * 128 * 130 * 4
    assert lib.socket_dense_attn_workspace_bytes(1, 1, 64, 1) == 66 * 4
    assert lib.socket_dense_attn_workspace_bytes(1, 1, 64, 0) == 0


def test_hard_bucket_table_rejects_invalid_arguments(lib):
    args = dict(Q=FAKE, R=FAKE, dt=1, B=1, Hq=8, Hkv=2, d=128, L=8, P=4, table=FAKE)

    def call(**over):
        a = dict(args)
        a.update(over)
        return lib.socket_hard_bucket_table(a["Q"], a["R"], a["dt"], a["B"], a["Hq"], a["Hkv"],
                                            a["d"], a["L"], a["P"], a["table"], None)

    assert call(dt=7) == _lib.SOCKET_ERR_INVALID_ARGUMENT
    assert call(Hq=7) == _lib.SOCKET_ERR_INVALID_ARGUMENT
    assert call(P=0) == _lib.SOCKET_ERR_INVALID_ARGUMENT
    assert call(Q=None) == _lib.SOCKET_ERR_INVALID_ARGUMENT
    assert call(table=None) == _lib.SOCKET_ERR_INVALID_ARGUMENT
    assert call(R=FAKE + 8) == _lib.SOCKET_ERR_INVALID_ARGUMENT
