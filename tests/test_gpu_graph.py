"""A whole step of the hot path captured in a HIP graph and replayed. The
library enqueues every launch on the caller's stream, allocates nothing and
issues no memset, so a captured step is the same work: every replay, with
eager work on the stream between replays (the outputs cleared), must give the
eager step's indices, attention outputs and lse bit for bit. Workloads at
reduced sizes: the headline decode (fused Full scoring + Top-512, split
attention), the hierarchical decode with MXFP4 indexer Q and FP8 window rows
(query packing, pool selection, Reindex layers), and the MXFP4-Q prefill
chunk (fused scoring + Top-512 over chunks, unsplit attention)."""
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("name,nq,N", [("encoder64k", 16, 32768), ("decode1m_fp4qk_fp8w", 8, 65536),
                                       ("prefill128k_fp4qk", 64, 65536)])
def test_step_graph_replays_equal_eager(name, nq, N):
    from kv_cache_compression_csa2_amd.pipeline import Step, pack_workload_kv, workload_kidx
    from kv_cache_compression_csa2_amd.workloads import make_workload
    print("case: graph replay", name, nq, N, flush=True)
    wl = make_workload(name, device=DEV, nq=nq, N=N)
    kv = pack_workload_kv(wl, DEV)
    kk = workload_kidx(wl)
    st = Step(wl, DEV)
    st.prepare(kk)
    st.run(kk, kv)
    torch.cuda.synchronize()
    ref = [t.clone() for t in st.top + st.out + st.lse]

    # warm-up on a side stream, then capture (the usual torch recipe)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.run(kk, kv)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run(kk, kv)
    torch.cuda.synchronize()

    for rep in range(3):
        for t in st.top:
            t.fill_(-7)
        for t in st.out + st.lse:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = st.top + st.out + st.lse
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), (name, rep, i)
    del g
