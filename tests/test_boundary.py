"""The C-ABI library loads, exports every declared call, and rejects bad
arguments on the host before touching the GPU. CPU only (no kernel launches)."""
import ctypes
import os
import re

import pytest

import kv_cache_compression_csa2_amd as K
from kv_cache_compression_csa2_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "csa2.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ["fp4_kv_pack", "fp4_kv_unpack", "csa2_index_full", "csa2_index_reindex", "csa2_topk",
              "csa2_topk_workspace_bytes", "csa2_sparse_attn", "csa2_sparse_attn_workspace_bytes",
              "csa2_format_version", "csa2_last_error", "kidx_fp4_pack", "csa2_index_full_fp4k",
              "csa2_index_reindex_fp4k"]:
        assert n in names
    assert sorted(L.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    lib = K.load()
    for n in _declared():
        assert hasattr(lib, n), n
    assert K.format_version() == 1


P = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation first
S = ctypes.c_void_p(0)


def _err(rc):
    return rc, K.load().csa2_last_error().decode()


@pytest.mark.parametrize("args,frag", [
    ((P, -1, P, S), "n < 0"),
    ((None, 5, P, S), "null"),
])
def test_pack_rejects(args, frag):
    rc, msg = _err(K.load().fp4_kv_pack(*args))
    assert rc == L.CSA2_EINVAL and frag in msg
    rc, msg = _err(K.load().swa_fp8_pack(*args))
    assert rc == L.CSA2_EINVAL and frag in msg and msg.startswith("swa_fp8_pack")


@pytest.mark.parametrize("kw,frag", [
    (dict(N=0), "N must be"),
    (dict(nq=-1), "nq < 0"),
    (dict(q_per_seq=0), "q_per_seq < 1"),
    (dict(nq=6, q_per_seq=4), "divide"),
    (dict(block_size=4), "block_size"),
    (dict(block_size=8, block=None), "block_scores"),
    (dict(scores=None), "null scores"),
    (dict(q=None), "null pointer"),
])
def test_index_full_rejects(kw, frag):
    a = dict(q=P, w=P, k=P, N=100, nq=2, q_per_seq=1, nv=None, scores=P, block_size=0, block=P)
    a.update(kw)
    rc, msg = _err(K.load().csa2_index_full(a["q"], a["w"], a["k"], a["N"], a["nq"], a["q_per_seq"], a["nv"],
                                            a["scores"], a["block_size"], a["block"], S))
    assert rc == L.CSA2_EINVAL and frag in msg, msg


@pytest.mark.parametrize("kw,frag", [
    (dict(N=0), "N must be"),
    (dict(q_per_seq=4), "divide"),
    (dict(block_size=8, block=None), "block_scores"),
    (dict(k=None), "null pointer"),
])
def test_index_fp4k_rejects(kw, frag):
    a = dict(q=P, w=P, k=P, N=100, nq=6, q_per_seq=1, scores=P, block_size=0, block=P)
    a.update(kw)
    L_ = K.load()
    rc, msg = _err(L_.csa2_index_full_fp4k(a["q"], a["w"], a["k"], a["N"], a["nq"], a["q_per_seq"], None,
                                          a["scores"], a["block_size"], a["block"], S))
    assert rc == L.CSA2_EINVAL and frag in msg and "fp4k" in msg, msg
    rc, msg = _err(L_.csa2_index_reindex_fp4k(a["q"], a["w"], a["k"], a["N"], a["nq"], a["q_per_seq"], None, P, 4,
                                             8, P, None, S))
    if kw.get("block_size") is None:
        assert rc == L.CSA2_EINVAL and frag in msg, msg
    rc, msg = _err(L_.kidx_fp4_pack(None, 3, P, S))
    assert rc == L.CSA2_EINVAL and "null" in msg


@pytest.mark.parametrize("kw,frag", [
    (dict(N=0), "N must be"),
    (dict(q_per_seq=1), "multiple of 8"),
    (dict(nq=24, q_per_seq=12), "multiple of 8"),
    (dict(q_per_seq=3), "divide"),
    (dict(block_size=8, block=None), "block_scores"),
    (dict(scores=None), "null scores"),
    (dict(k=None), "null pointer"),
    (dict(q=None), "null pointer"),
])
def test_index_fp4qk_rejects(kw, frag):
    a = dict(q=P, w=P, k=P, N=100, nq=8, q_per_seq=8, scores=P, block_size=0, block=P)
    a.update(kw)
    L_ = K.load()
    if frag != "multiple of 8":  # only the prefill-chunk call scores 8 queries of a sequence together
        rc, msg = _err(L_.csa2_index_full_fp4qk(a["q"], a["w"], a["k"], a["N"], a["nq"], a["q_per_seq"], None,
                                               a["scores"], a["block_size"], a["block"], S))
        assert rc == L.CSA2_EINVAL and frag in msg and "fp4qk" in msg, msg
    if "scores" not in kw and "block_size" not in kw:
        rc, msg = _err(L_.csa2_index_prefill_topk_fp4qk(a["q"], a["w"], a["k"], a["N"], a["nq"], a["q_per_seq"], None,
                                                       512, P, None, P, 1 << 30, S))
        assert rc == L.CSA2_EINVAL and frag in msg and "fp4qk" in msg, msg
    rc, msg = _err(L_.csa2_index_prefill_topk_fp4qk(P, P, P, 100, 8, 8, None, 513, P, None, P, 1 << 30, S))
    assert rc == L.CSA2_EINVAL and "k must be" in msg
    # the decode and Reindex MXFP4-Q calls check as their FP4-K siblings
    rc, msg = _err(L_.csa2_index_topk_fp4qk(P, P, P, 100, 2, None, 0, P, 0, None, None, P, 1 << 30, S))
    assert rc == L.CSA2_EINVAL and "k must be" in msg and "fp4qk" in msg, msg
    rc, msg = _err(L_.csa2_index_topk_select_fp4qk(None, P, P, 100, 2, None, 512, P, 0, None, None, P, 1 << 30, S))
    assert rc == L.CSA2_EINVAL and "null pointer" in msg, msg
    rc, msg = _err(L_.csa2_index_reindex_fp4qk(P, P, P, 100, 2, 1, None, P, 0, 8, P, None, S))
    assert rc == L.CSA2_EINVAL and "nb must be" in msg and "fp4qk" in msg, msg
    rc, msg = _err(L_.csa2_index_reindex_topk_fp4qk(P, P, P, 100, 2, 1, None, P, 4, 0, P, None, P, 1 << 30, S))
    assert rc == L.CSA2_EINVAL and "k must be" in msg and "fp4qk" in msg, msg


@pytest.mark.parametrize("kw,frag", [
    (dict(block_size=16), "block_size"),
    (dict(nb=0), "nb must be"),
    (dict(nb=70000), "nb must be"),
    (dict(cand=None), "null pointer"),
])
def test_reindex_rejects(kw, frag):
    a = dict(nb=2048, block_size=8, cand=P)
    a.update(kw)
    rc, msg = _err(K.load().csa2_index_reindex(P, P, P, 1000, 2, 1, None, a["cand"], a["nb"], a["block_size"], P,
                                               None, S))
    assert rc == L.CSA2_EINVAL and frag in msg, msg


@pytest.mark.parametrize("kw,frag,code", [
    (dict(k=0), "k must be", L.CSA2_EINVAL),
    (dict(k=4097), "k must be", L.CSA2_EINVAL),
    (dict(ncols=0), "ncols", L.CSA2_EINVAL),
    (dict(ld=10), "ld < ncols", L.CSA2_EINVAL),
    (dict(rows=-2), "rows < 0", L.CSA2_EINVAL),
    (dict(ncols=1 << 20, ld=1 << 20, ws=None), "workspace", L.CSA2_EWORKSPACE),
    (dict(ncols=1 << 20, ld=1 << 20, wsb=8), "workspace", L.CSA2_EWORKSPACE),
])
def test_topk_rejects(kw, frag, code):
    a = dict(rows=8, ncols=1000, ld=1000, k=512, ws=P, wsb=1 << 40)
    a.update(kw)
    rc, msg = _err(K.load().csa2_topk(P, a["rows"], a["ncols"], a["ld"], None, a["k"], None, P, a["ws"], a["wsb"],
                                      S))
    assert rc == code and frag in msg, msg


@pytest.mark.parametrize("kw,frag,code", [
    (dict(k=0), "k must be", L.CSA2_EINVAL),
    (dict(k=4097), "k must be", L.CSA2_EINVAL),
    (dict(N=0), "N must be", L.CSA2_EINVAL),
    (dict(N=5_000_000), "too large", L.CSA2_EINVAL),          # 611 chunks of 8192: beyond two merge levels at k=512
    (dict(N=70000, k=4096), "too large", L.CSA2_EINVAL),
    (dict(top=None), "null top_idx", L.CSA2_EINVAL),
    (dict(block_size=4), "block_size", L.CSA2_EINVAL),
    (dict(block_size=8, block=None), "block_scores", L.CSA2_EINVAL),
    (dict(ws=None), "workspace", L.CSA2_EWORKSPACE),
    (dict(wsb=8), "workspace", L.CSA2_EWORKSPACE),
])
def test_index_topk_rejects(kw, frag, code):
    a = dict(N=40000, nq=4, k=512, top=P, block_size=0, block=P, ws=P, wsb=1 << 40)
    a.update(kw)
    L_ = K.load()
    for name, fn in [("csa2_index_topk", L_.csa2_index_topk), ("csa2_index_topk_fp4k", L_.csa2_index_topk_fp4k)]:
        rc, msg = _err(fn(P, P, P, a["N"], a["nq"], None, a["k"], a["top"], a["block_size"], a["block"], None,
                          a["ws"], a["wsb"], S))
        assert rc == code and frag in msg and msg.startswith(name), msg
    rc, msg = _err(L_.csa2_index_topk_select(P, P, P, 1, a["N"], a["nq"], None, a["k"], a["top"], a["block_size"],
                                            a["block"], None, a["ws"], a["wsb"], S))
    assert rc == code and frag in msg, msg
    if "block" not in frag:
        rc, msg = _err(L_.csa2_index_topk_merge(a["N"], a["nq"], a["k"], a["top"], a["ws"], a["wsb"], S))
        assert rc == code and frag in msg, msg


@pytest.mark.parametrize("kw,frag,code", [
    (dict(k=0), "k must be", L.CSA2_EINVAL),
    (dict(k=4097), "k must be", L.CSA2_EINVAL),
    (dict(pool_k=0), "pool_k must be", L.CSA2_EINVAL),
    (dict(pool_k=4097), "pool_k must be", L.CSA2_EINVAL),
    (dict(N=0), "N must be", L.CSA2_EINVAL),
    (dict(nq=-1), "nq < 0", L.CSA2_EINVAL),
    (dict(N=5_000_000), "too large", L.CSA2_EINVAL),
    (dict(top=None), "null pointer", L.CSA2_EINVAL),
    (dict(block=None), "null pointer", L.CSA2_EINVAL),
    (dict(cand=None), "null pointer", L.CSA2_EINVAL),
    (dict(ws=None), "workspace", L.CSA2_EWORKSPACE),
    (dict(wsb=8), "workspace", L.CSA2_EWORKSPACE),
])
def test_index_topk_merge_pool_rejects(kw, frag, code):
    a = dict(N=1 << 20, nq=8, k=512, pool_k=2048, top=P, block=P, cand=P, ws=P, wsb=1 << 40)
    a.update(kw)
    rc, msg = _err(K.load().csa2_index_topk_merge_pool(a["N"], a["nq"], a["k"], a["top"], a["block"], a["pool_k"],
                                                       a["cand"], a["ws"], a["wsb"], S))
    assert rc == code and frag in msg and msg.startswith("csa2_index_topk_merge_pool"), msg


def test_index_topk_pool_workspace_covers_both_selections():
    L_ = K.load()
    for nq, N, k, pk in [(8, 1 << 20, 512, 2048), (32, 262144, 512, 2048), (3, 20000, 100, 3000), (2, 4096, 512, 2048)]:
        a = L_.csa2_index_topk_workspace_bytes(nq, N, k)
        b = L_.csa2_topk_workspace_bytes(nq, (N + 7) // 8, pk)
        got = L_.csa2_index_topk_pool_workspace_bytes(nq, N, k, pk)
        assert got == ((a + 255) // 256) * 256 + b, (nq, N, k, pk, got, a, b)
    assert L_.csa2_index_topk_pool_workspace_bytes(8, 1 << 20, 512, 0) == 0
    assert L_.csa2_index_topk_pool_workspace_bytes(8, 5_000_000, 512, 2048) == 0


@pytest.mark.parametrize("kw,frag,code", [
    (dict(k=0), "k must be", L.CSA2_EINVAL),
    (dict(k=4097), "k must be", L.CSA2_EINVAL),
    (dict(N=0), "N must be", L.CSA2_EINVAL),
    (dict(nb=0), "nb must be", L.CSA2_EINVAL),
    (dict(nb=65537), "nb must be", L.CSA2_EINVAL),
    (dict(nq=3, qps=2), "q_per_seq", L.CSA2_EINVAL),
    (dict(nb=65536, k=4096), "too large", L.CSA2_EINVAL),   # 64 chunks of 8192 x 4096 slots: beyond the merge
    (dict(top=None), "null pointer", L.CSA2_EINVAL),
    (dict(blocks=None), "null pointer", L.CSA2_EINVAL),
    (dict(ws=None), "workspace", L.CSA2_EWORKSPACE),
    (dict(wsb=8), "workspace", L.CSA2_EWORKSPACE),
])
def test_index_reindex_topk_rejects(kw, frag, code):
    a = dict(N=40000, nq=4, qps=1, nb=2048, k=512, blocks=P, top=P, ws=P, wsb=1 << 40)
    a.update(kw)
    L_ = K.load()
    for name in ("csa2_index_reindex_topk", "csa2_index_reindex_topk_fp4k"):
        rc, msg = _err(getattr(L_, name)(P, P, P, a["N"], a["nq"], a["qps"], None, a["blocks"], a["nb"], a["k"],
                                         a["top"], None, a["ws"], a["wsb"], S))
        assert rc == code and frag in msg and msg.startswith(name), msg


def test_index_reindex_topk_workspace_sizes():
    # 32 x 2048 blocks (16384 positions): chunks of 1024 (512 workgroups), 16 x 512 candidates per row
    assert K.csa2_index_reindex_topk_workspace_bytes(32, 2048, 512) == 32 * 16 * 512 * 8
    # 64 queries: chunks of 2048 keep the grid at 512 workgroups
    assert K.csa2_index_reindex_topk_workspace_bytes(64, 2048, 512) == 64 * 8 * 512 * 8
    # k = 2048: chunks of at least 4096 positions
    assert K.csa2_index_reindex_topk_workspace_bytes(8, 2048, 2048) == 8 * 4 * 2048 * 8
    # a pool of one chunk: no workspace
    assert K.csa2_index_reindex_topk_workspace_bytes(4, 100, 512) == 0


def test_index_topk_workspace_sizes():
    # 64 x 32768: chunks of 4096 (8192 would give only 256 workgroups), candidates (key + id) of every chunk
    assert K.csa2_index_topk_workspace_bytes(64, 32768, 512) == 64 * 8 * 512 * 8
    # 8 x 2^20: 128 chunks, two merge levels of 4-chunk groups (32 groups of 2048 candidates)
    assert K.csa2_index_topk_workspace_bytes(8, 1 << 20, 512) == 8 * 512 * (128 + 32) * 8
    # k = 1024 at 2^20: 2048-candidate groups would leave 64 x 1024 for the second level;
    # 8-chunk groups of 8192 candidates keep it at 16 x 1024
    assert K.csa2_index_topk_workspace_bytes(8, 1 << 20, 1024) == 8 * 1024 * (128 + 16) * 8
    # one chunk per query: no workspace
    assert K.csa2_index_topk_workspace_bytes(64, 4096, 512) == 0
    # few queries: chunks of 4096
    assert K.csa2_index_topk_workspace_bytes(2, 20000, 512) == 2 * 5 * 512 * 8


def test_workspace_sizes():
    assert K.csa2_topk_workspace_bytes(4096, 16384, 512) == 0  # many rows, one 16384-key chunk: one pass per row
    # longer rows: chunks of <= 16384 keys, candidates of every chunk (key + column)
    assert K.csa2_topk_workspace_bytes(4096, 32768, 512) == 4096 * 2 * 512 * 8
    assert K.csa2_topk_workspace_bytes(4096, 65536, 512) == 4096 * 4 * 512 * 8
    # 1M-entry rows need 32768-key chunks to keep the merge within 16384 candidates
    assert K.csa2_topk_workspace_bytes(8, 1 << 20, 512) == 8 * 32 * 512 * 8
    big = K.csa2_topk_workspace_bytes(8, 1 << 20, 512)
    assert big > 0 and big % 8 == 0
    assert K.csa2_topk_workspace_bytes(1, 1000, 512) == 0
    assert K.csa2_sparse_attn_workspace_bytes(4096, 512) == 256  # the status word only
    assert K.csa2_sparse_attn_workspace_bytes(8, 512) > 256


@pytest.mark.parametrize("kw,frag,code", [
    (dict(k=-1), "k must be", L.CSA2_EINVAL),
    (dict(N=0), "N must be", L.CSA2_EINVAL),
    (dict(q_per_seq=3), "q_per_seq", L.CSA2_EINVAL),
    (dict(idx=None), "null idx", L.CSA2_EINVAL),
    (dict(T=0), "window", L.CSA2_EINVAL),
    (dict(start=None), "window", L.CSA2_EINVAL),
    (dict(scale=float("nan")), "NaN", L.CSA2_EINVAL),
    (dict(ws=None), "workspace", L.CSA2_EWORKSPACE),
])
def test_attn_rejects(kw, frag, code):
    a = dict(N=1000, nq=8, q_per_seq=1, idx=P, k=512, swa=P, T=128, start=P, len_=P, scale=0.04, ws=P, wsb=1 << 40)
    a.update(kw)
    rc, msg = _err(K.load().csa2_sparse_attn(P, P, a["N"], a["nq"], a["q_per_seq"], a["idx"], a["k"], a["swa"],
                                             a["T"], a["start"], a["len_"], a["scale"], P, None, a["ws"], a["wsb"],
                                             S))
    assert rc == code and frag in msg, msg
    # the FP8-window variant checks the same arguments
    rc, msg = _err(K.load().csa2_sparse_attn_fp8w(P, P, a["N"], a["nq"], a["q_per_seq"], a["idx"], a["k"], a["swa"],
                                                  a["T"], a["start"], a["len_"], a["scale"], P, None, a["ws"],
                                                  a["wsb"], S))
    assert rc == code and frag in msg and msg.startswith("csa2_sparse_attn_fp8w"), msg


def test_index_topk_noalloc_rejects_calls_beyond_its_scratch():
    """The no-allocation call refuses (before touching the device) any call
    whose candidates would not fit the static scratch."""
    import kv_cache_compression_csa2_amd._lib as L
    lib = L.load()
    cap = lib.csa2_index_topk_noalloc_scratch_bytes()
    assert cap == 16 << 20
    assert lib.csa2_index_topk_workspace_bytes(64, 1 << 20, 512) > cap
    rc = lib.csa2_index_topk_noalloc(1, 1, 1, 0, 1 << 20, 64, None, 512, 1, 0, None, None, None)
    assert rc == L.CSA2_EINVAL
    assert b"static scratch holds" in lib.csa2_last_error()
    # the usual argument checks come first
    rc = lib.csa2_index_topk_noalloc(1, 1, 1, 0, 1024, 4, None, 0, 1, 0, None, None, None)
    assert rc == L.CSA2_EINVAL and b"k must be in" in lib.csa2_last_error()
