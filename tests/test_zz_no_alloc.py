"""csa2_select_topk_noalloc (no workspace: the library's static scratch)
against csa2_select_topk with a caller's workspace, through the C ABI, on
consecutive calls of decreasing size, and its refusal of a size beyond the
static scratch."""
import pytest
import torch

import long_context_sparse_csa2_amd as C

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _both(Q, n_cols, k, n_valid, col_ids, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    scores = torch.rand(Q, n_cols, generator=g, device=DEV) * 100
    scores[:, ::97] = scores[:, 1:2]                 # exact ties across each row
    nv = torch.tensor(n_valid, dtype=torch.int64, device=DEV)
    ref = torch.full((Q, k), -7, dtype=torch.int32, device=DEV)
    got = torch.full((Q, k), -9, dtype=torch.int32, device=DEV)
    ws = C.workspace(C.CSA2_OP_TOPK, Q, n_cols, k, DEV)
    C.csa2_select_topk(scores, nv, col_ids, n_cols, k, ref, ws)
    C.csa2_select_topk_noalloc(scores, nv, col_ids, n_cols, k, got)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_workspace_call():
    # 1M-column rows (the decode Full layer's size), ragged valid counts
    print("[noalloc] Q=4 n_cols=2^20 k=512", flush=True)
    ref, got = _both(4, 1 << 20, 512, [1 << 20, (1 << 20) - 5, 700001, 300], None, 1)
    assert torch.equal(ref, got)
    assert (got[3, 300:] == -1).all()
    # then a smaller call with mapped column ids (a pool-shaped row)
    print("[noalloc] Q=3 n_cols=20000 k=100 col_ids", flush=True)
    ids = torch.stack([torch.sort(torch.randperm(1 << 18, generator=torch.Generator().manual_seed(s))[:20000])[0]
                       for s in range(3)]).to(torch.int32).to(DEV)
    ref, got = _both(3, 20000, 100, [20000, 19999, 64], ids, 2)
    assert torch.equal(ref, got)
    # and one that needs no maxima at all
    print("[noalloc] Q=2 n_cols=3000 k=512", flush=True)
    ref, got = _both(2, 3000, 512, [3000, 2000], None, 3)
    assert torch.equal(ref, got)


def test_noalloc_refuses_beyond_scratch():
    Q, n = 64, 1 << 19                              # 18 MiB of maxima > 16 MiB
    assert C.csa2_workspace_bytes(C.CSA2_OP_TOPK, Q, n, 512) > 16 << 20
    scores = torch.zeros(Q, n, device=DEV)
    nv = torch.full((Q,), n, dtype=torch.int64, device=DEV)
    out = torch.empty(Q, 512, dtype=torch.int32, device=DEV)
    with pytest.raises(C.Csa2Error, match="static"):
        C.csa2_select_topk_noalloc(scores, nv, None, n, 512, out)
