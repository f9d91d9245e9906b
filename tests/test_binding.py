"""Python binding checks that need no GPU: every wrapper rejects tensors of
the wrong shape or dtype with a ValueError naming the argument, before any
pointer reaches the C ABI (which cannot see shapes or dtypes, so a wrong
tensor would be read or written out of bounds on the device). CPU tensors
are used: the checks run before the device check, and the messages are
matched so that the device check cannot stand in for them."""

import pytest
import torch

import soft_lsh_sparse_amd as S

B, Hq, Hkv, d, N, L, P, k = 1, 8, 2, 128, 64, 8, 4, 16


def _decode_args(**over):
    a = dict(
        Q=torch.zeros(B, Hq, d, dtype=torch.bfloat16),
        K=torch.zeros(B, Hkv, N, d, dtype=torch.bfloat16),
        V=torch.zeros(B, Hkv, N, d, dtype=torch.bfloat16),
        R=torch.zeros(d, L * P, dtype=torch.bfloat16),
        ids=torch.zeros(B, Hkv, N, L, dtype=torch.uint8),
        vnorm=torch.zeros(B, Hkv, N, dtype=torch.float32),
    )
    a.update(over)
    return a


@pytest.mark.parametrize("over,match", [
    (dict(ids=torch.zeros(B, Hkv, N, L, dtype=torch.int64)), "ids must be torch.uint8"),
    (dict(ids=torch.zeros(B, Hkv, N, L + 1, dtype=torch.uint8)), "ids must have shape"),
    (dict(vnorm=torch.zeros(B, Hkv, N, dtype=torch.float16)), "vnorm must be torch.float32"),
    (dict(vnorm=torch.zeros(B, Hkv, N - 1)), "vnorm must have shape"),
    (dict(R=torch.zeros(d, L * P - 1, dtype=torch.bfloat16)), "R must have shape"),
    (dict(R=torch.zeros(d, L * P, dtype=torch.float32)), "R must be torch.bfloat16"),
    (dict(V=torch.zeros(B, Hkv, N, d, dtype=torch.float32)), "V must be torch.bfloat16"),
    (dict(K=torch.zeros(B, Hkv, N, d // 2, dtype=torch.bfloat16)), "K must have shape"),
    (dict(Q=torch.zeros(B, 7, d, dtype=torch.bfloat16)), "not a multiple"),
])
def test_decode_rejects_mismatched_inputs(over, match):
    with pytest.raises(ValueError, match=match):
        S.decode(**_decode_args(**over), L=L, P=P, tau=0.3, k=k)


@pytest.mark.parametrize("kw,match", [
    (dict(idx_out=torch.zeros(B, Hq, k, dtype=torch.int64)), "idx_out must be torch.int32"),
    (dict(idx_out=torch.zeros(B, Hq, k - 1, dtype=torch.int32)), "idx_out must have shape"),
    (dict(scores_out=torch.zeros(B, Hq, N, dtype=torch.bfloat16)),
     "scores_out must be torch.float32"),
    (dict(scores_out=torch.zeros(B, Hq, N - 5)), "scores_out must have shape"),
    (dict(out=torch.zeros(B, Hq, d, dtype=torch.float32)), "out must be torch.bfloat16"),
    (dict(n_keys=N + 1), "n_keys"),
])
def test_decode_rejects_mismatched_outputs(kw, match):
    with pytest.raises(ValueError, match=match):
        S.decode(**_decode_args(), L=L, P=P, tau=0.3, k=k, **kw)


def test_group_shared_outputs_are_per_kv_head():
    with pytest.raises(ValueError, match="idx_out must have shape"):
        S.decode_group_shared(**_decode_args(), L=L, P=P, tau=0.3, k=k,
                              idx_out=torch.zeros(B, Hq, k, dtype=torch.int32))
    with pytest.raises(ValueError, match="scores_out must have shape"):
        S.decode_group_shared(**_decode_args(), L=L, P=P, tau=0.3, k=k,
                              scores_out=torch.zeros(B, Hq, N))


def test_stage_wrappers_check_their_tensors():
    a = _decode_args()
    with pytest.raises(ValueError, match="R must have shape"):
        S.hash_keys(a["K"], a["V"], a["R"][:, :-1], L, P)
    with pytest.raises(ValueError, match="ids must be torch.uint8"):
        S.hash_keys(a["K"], a["V"], a["R"], L, P, ids=torch.zeros(B, Hkv, N, L, dtype=torch.int32))
    with pytest.raises(ValueError, match="V must have shape"):
        S.hash_keys(a["K"], a["V"][:, :, :-1], a["R"], L, P)
    with pytest.raises(ValueError, match="R must be torch.bfloat16"):
        S.bucket_probs(a["Q"], a["R"].float(), Hkv, L, P, 0.3)
    with pytest.raises(ValueError, match="R must have shape"):
        S.hard_bucket_table(a["Q"], a["R"][:-1], Hkv, L, P)
    table = torch.zeros(B, Hkv, 2 ** P, L, Hq // Hkv)
    with pytest.raises(ValueError, match="table must be torch.float32"):
        S.score(table.double(), a["ids"], a["vnorm"], Hq)
    with pytest.raises(ValueError, match="does not fit Hq"):
        S.score(table, a["ids"], a["vnorm"], Hq * 2)
    with pytest.raises(ValueError, match="vnorm must have shape"):
        S.score(table, a["ids"], a["vnorm"][..., :-1], Hq)
    with pytest.raises(ValueError, match="scores must be torch.float32"):
        S.topk(torch.zeros(4, 100, dtype=torch.bfloat16), 10)
    idx = torch.zeros(B, Hq, k, dtype=torch.int32)
    with pytest.raises(ValueError, match="idx must be torch.int32"):
        S.sparse_attn(a["Q"], a["K"], a["V"], idx.long())
    with pytest.raises(ValueError, match="V must be torch.bfloat16"):
        S.sparse_attn(a["Q"], a["K"], a["V"].float(), idx)
    with pytest.raises(ValueError, match="K must have shape"):
        S.dense_attn(a["Q"], a["K"][..., :64], a["V"])
