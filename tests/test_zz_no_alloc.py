"""csa2_index_topk_noalloc (static device scratch, no allocation) against
csa2_index_topk (caller workspace) on the same inputs: Top-k indices, block
maxima and score rows bit for bit, on two calls in a row, the second with a
smaller input, in both key formats."""
import numpy as np
import pytest
import torch

from tests._conv import np_

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _g(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def _inputs(nq, N, seed, fp4):
    import kv_cache_compression_csa2_amd as K
    g = _g(seed)
    q = torch.randn((nq, 32, 128), generator=g, device=DEV).to(torch.bfloat16)
    w = torch.rand((nq, 32), generator=g, device=DEV)
    k = torch.randn((nq, N, 128), generator=g, device=DEV).to(torch.bfloat16)
    nv = torch.randint(N // 2, N + 1, (nq,), generator=g, device=DEV).to(torch.int32)
    if fp4:
        return q, w, None, K.kidx_fp4_pack(k.reshape(-1, 128)).view(nq, N, 68), nv
    return q, w, k, None, nv


@pytest.mark.parametrize("fp4", [False, True])
def test_noalloc_equals_workspace_call_twice_shrinking(fp4):
    import kv_cache_compression_csa2_amd as K
    print("case: noalloc fp4=%s" % fp4, flush=True)
    assert K.csa2_index_topk_noalloc_scratch_bytes() == 16 << 20
    for call, (nq, N, k, seed) in enumerate([(16, 300000, 512, 41), (3, 40000, 100, 42)]):
        q, w, kb, kf, nv = _inputs(nq, N, seed + (10 if fp4 else 0), fp4)
        assert 0 < K.csa2_index_topk_workspace_bytes(nq, N, k) <= K.csa2_index_topk_noalloc_scratch_bytes()
        top = torch.full((nq, k), -7, dtype=torch.int32, device=DEV)
        blk = torch.full((nq, (N + 7) // 8), 7.0, dtype=torch.float32, device=DEV)
        sc = torch.full((nq, N), 7.0, dtype=torch.float32, device=DEV)
        torch.cuda.synchronize()
        K.csa2_index_topk_noalloc(q, w, kb, N, k, n_visible=nv, block_size=8, top=top, block_scores=blk, scores=sc,
                                  k_fp4=kf)
        ref_top, ref_blk = K.csa2_index_topk(q, w, kb, N, k, n_visible=nv, block_size=8, k_fp4=kf)
        ref_sc = torch.empty_like(sc)
        K.csa2_index_topk(q, w, kb, N, k, n_visible=nv, scores=ref_sc, k_fp4=kf)
        torch.cuda.synchronize()
        assert torch.equal(top, ref_top), call
        assert torch.equal(blk, ref_blk), call
        assert torch.equal(sc, ref_sc), call
        # the selection is exactly Top-k of the score row it scored
        own = K.csa2_topk(sc, k, row_len=nv)
        torch.cuda.synchronize()
        assert torch.equal(own, top), call
        print("  call %d ok (nq %d, N %d, k %d)" % (call, nq, N, k), flush=True)
