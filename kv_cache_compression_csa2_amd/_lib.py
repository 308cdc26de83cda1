"""ctypes binding of libcsa2.so (the C ABI in include/csa2.h).

Argument marshalling only: tensors are passed as raw device pointers, the
stream is torch's current stream; every step runs in the HIP kernels. Loading
fails loudly when the built library is missing -- there is no fallback.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

CSA2_OK, CSA2_EINVAL, CSA2_ELAUNCH, CSA2_EWORKSPACE = 0, -1, -2, -3
DIM, HEADS, IDX_HEADS, IDX_DIM, RECORD = 512, 64, 32, 128, 288
KIDX_RECORD = 68  # FP4 indexer-K entry (OCP MXFP4): 64 code bytes + 4 E8M0 block scales
SWA_RECORD = 528  # FP8 window-KV row: 512 E4M3 codes + 16 E8M0 scales

_lib = None


class Csa2Error(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (code %d)" % (msg, code))
        self.code = code


def load():
    """Load libcsa2.so (built by kv_cache_compression_csa2_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libcsa2.so is not built: run `python -m kv_cache_compression_csa2_amd.build` "
                          "(or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    L.csa2_format_version.restype = ctypes.c_int
    L.csa2_last_error.restype = ctypes.c_char_p
    L.fp4_kv_pack.argtypes = [vp, i64, vp, vp]
    L.fp4_kv_unpack.argtypes = [vp, i64, vp, vp]
    L.csa2_index_full.argtypes = [vp, vp, vp, i64, i32, i32, vp, vp, i32, vp, vp]
    L.csa2_index_reindex.argtypes = [vp, vp, vp, i64, i32, i32, vp, vp, i32, i32, vp, vp, vp]
    L.kidx_fp4_pack.argtypes = [vp, i64, vp, vp]
    L.csa2_index_full_fp4k.argtypes = [vp, vp, vp, i64, i32, i32, vp, vp, i32, vp, vp]
    L.csa2_index_reindex_fp4k.argtypes = [vp, vp, vp, i64, i32, i32, vp, vp, i32, i32, vp, vp, vp]
    L.swa_fp8_pack.argtypes = [vp, i64, vp, vp]
    L.csa2_index_topk_workspace_bytes.argtypes = [i32, i64, i32]
    L.csa2_index_topk_workspace_bytes.restype = sz
    L.csa2_index_topk.argtypes = [vp, vp, vp, i64, i32, vp, i32, vp, i32, vp, vp, vp, sz, vp]
    L.csa2_index_topk_fp4k.argtypes = [vp, vp, vp, i64, i32, vp, i32, vp, i32, vp, vp, vp, sz, vp]
    L.csa2_index_topk_select.argtypes = [vp, vp, vp, i32, i64, i32, vp, i32, vp, i32, vp, vp, vp, sz, vp]
    L.csa2_index_topk_merge.argtypes = [i64, i32, i32, vp, vp, sz, vp]
    L.csa2_index_topk_pool_workspace_bytes.argtypes = [i32, i64, i32, i32]
    L.csa2_index_topk_pool_workspace_bytes.restype = sz
    L.csa2_index_topk_merge_pool.argtypes = [i64, i32, i32, vp, vp, i32, vp, vp, sz, vp]
    L.csa2_index_topk_noalloc_scratch_bytes.argtypes = []
    L.csa2_index_topk_noalloc_scratch_bytes.restype = sz
    L.csa2_index_topk_noalloc.argtypes = [vp, vp, vp, i32, i64, i32, vp, i32, vp, i32, vp, vp, vp]
    L.csa2_index_prefill_topk_workspace_bytes.argtypes = [i32, i64, i32]
    L.csa2_index_prefill_topk_workspace_bytes.restype = sz
    L.csa2_index_prefill_topk.argtypes = [vp, vp, vp, i64, i32, i32, vp, i32, vp, vp, vp, sz, vp]
    L.csa2_index_prefill_topk_fp4k.argtypes = [vp, vp, vp, i64, i32, i32, vp, i32, vp, vp, vp, sz, vp]
    L.csa2_index_full_fp4qk.argtypes = [vp, vp, vp, i64, i32, i32, vp, vp, i32, vp, vp]
    L.csa2_index_reindex_fp4qk.argtypes = [vp, vp, vp, i64, i32, i32, vp, vp, i32, i32, vp, vp, vp]
    L.csa2_index_topk_fp4qk.argtypes = [vp, vp, vp, i64, i32, vp, i32, vp, i32, vp, vp, vp, sz, vp]
    L.csa2_index_topk_select_fp4qk.argtypes = [vp, vp, vp, i64, i32, vp, i32, vp, i32, vp, vp, vp, sz, vp]
    L.csa2_index_reindex_topk_fp4qk.argtypes = [vp, vp, vp, i64, i32, i32, vp, vp, i32, i32, vp, vp, vp, sz, vp]
    L.csa2_index_prefill_topk_fp4qk.argtypes = [vp, vp, vp, i64, i32, i32, vp, i32, vp, vp, vp, sz, vp]
    L.csa2_index_reindex_topk_workspace_bytes.argtypes = [i32, i32, i32]
    L.csa2_index_reindex_topk_workspace_bytes.restype = sz
    L.csa2_index_reindex_topk.argtypes = [vp, vp, vp, i64, i32, i32, vp, vp, i32, i32, vp, vp, vp, sz, vp]
    L.csa2_index_reindex_topk_fp4k.argtypes = [vp, vp, vp, i64, i32, i32, vp, vp, i32, i32, vp, vp, vp, sz, vp]
    L.csa2_topk_workspace_bytes.argtypes = [i32, i64, i32]
    L.csa2_topk_workspace_bytes.restype = sz
    L.csa2_topk.argtypes = [vp, i32, i64, i64, vp, i32, vp, vp, vp, sz, vp]
    L.csa2_sparse_attn_workspace_bytes.argtypes = [i32, i32]
    L.csa2_sparse_attn_workspace_bytes.restype = sz
    L.csa2_sparse_attn.argtypes = [vp, vp, i64, i32, i32, vp, i32, vp, i64, vp, vp, f32, vp, vp, vp, sz, vp]
    L.csa2_sparse_attn_fp8w.argtypes = [vp, vp, i64, i32, i32, vp, i32, vp, i64, vp, vp, f32, vp, vp, vp, sz, vp]
    for name in ["fp4_kv_pack", "fp4_kv_unpack", "csa2_index_full", "csa2_index_reindex", "csa2_topk",
                 "csa2_sparse_attn", "kidx_fp4_pack", "csa2_index_full_fp4k", "csa2_index_reindex_fp4k",
                 "swa_fp8_pack", "csa2_sparse_attn_fp8w", "csa2_index_topk", "csa2_index_topk_fp4k",
                 "csa2_index_topk_select", "csa2_index_topk_merge", "csa2_index_topk_merge_pool",
                 "csa2_index_reindex_topk", "csa2_index_reindex_topk_fp4k", "csa2_index_topk_noalloc", "csa2_index_prefill_topk",
                 "csa2_index_prefill_topk_fp4k", "csa2_index_full_fp4qk", "csa2_index_prefill_topk_fp4qk",
                 "csa2_index_reindex_fp4qk", "csa2_index_topk_fp4qk", "csa2_index_topk_select_fp4qk",
                 "csa2_index_reindex_topk_fp4qk"]:
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


EXPORTS = ["csa2_format_version", "csa2_last_error", "fp4_kv_pack", "fp4_kv_unpack", "csa2_index_full",
           "csa2_index_reindex", "csa2_topk_workspace_bytes", "csa2_topk", "csa2_sparse_attn_workspace_bytes",
           "csa2_sparse_attn", "kidx_fp4_pack", "csa2_index_full_fp4k", "csa2_index_reindex_fp4k", "swa_fp8_pack",
           "csa2_sparse_attn_fp8w", "csa2_index_topk_workspace_bytes", "csa2_index_topk", "csa2_index_topk_fp4k",
           "csa2_index_topk_select", "csa2_index_topk_merge", "csa2_index_topk_pool_workspace_bytes",
           "csa2_index_topk_merge_pool", "csa2_index_reindex_topk_workspace_bytes",
           "csa2_index_reindex_topk", "csa2_index_reindex_topk_fp4k", "csa2_index_topk_noalloc_scratch_bytes",
           "csa2_index_topk_noalloc", "csa2_index_prefill_topk_workspace_bytes", "csa2_index_prefill_topk",
           "csa2_index_prefill_topk_fp4k", "csa2_index_full_fp4qk", "csa2_index_prefill_topk_fp4qk",
           "csa2_index_reindex_fp4qk", "csa2_index_topk_fp4qk", "csa2_index_topk_select_fp4qk",
           "csa2_index_reindex_topk_fp4qk"]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(rc, name):
    if rc != CSA2_OK:
        msg = load().csa2_last_error().decode()
        raise Csa2Error(rc, msg or name)


def _need(t, dtype, name, cuda=True):
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if cuda and not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)


def format_version():
    return load().csa2_format_version()


def fp4_kv_pack(x, out=None, stream=None):
    """bf16 [n,512] -> uint8 [n,288] FP4 records."""
    _need(x, torch.bfloat16, "x")
    n = x.numel() // DIM
    if out is None:
        out = torch.empty((n, RECORD), dtype=torch.uint8, device=x.device)
    _need(out, torch.uint8, "out")
    _check(load().fp4_kv_pack(_ptr(x), n, _ptr(out), _stream(stream)), "fp4_kv_pack")
    return out


def fp4_kv_unpack(rec, out=None, stream=None):
    """uint8 [n,288] FP4 records -> bf16 [n,512]."""
    _need(rec, torch.uint8, "rec")
    n = rec.numel() // RECORD
    if out is None:
        out = torch.empty((n, DIM), dtype=torch.bfloat16, device=rec.device)
    _need(out, torch.bfloat16, "out")
    _check(load().fp4_kv_unpack(_ptr(rec), n, _ptr(out), _stream(stream)), "fp4_kv_unpack")
    return out


def _k_args(k_idx, k_fp4):
    """(pointer, call suffix) of the indexer-K operand: bf16 k_idx or FP4 k_fp4."""
    if (k_idx is None) == (k_fp4 is None):
        raise ValueError("pass exactly one of k_idx (bf16) and k_fp4 (uint8 [.., 68])")
    if k_fp4 is not None:
        _need(k_fp4, torch.uint8, "k_fp4")
        return _ptr(k_fp4), "_fp4k"
    _need(k_idx, torch.bfloat16, "k_idx")
    return _ptr(k_idx), ""


def _q_args(q_idx, q_fp4, suffix):
    """(pointer, query count, call suffix) of the indexer-Q operand: bf16 q_idx
    [nq,32,128], or MXFP4 entries q_fp4 [nq,32,68] (then the K must be FP4 too)."""
    if (q_idx is None) == (q_fp4 is None):
        raise ValueError("pass exactly one of q_idx (bf16) and q_fp4 (uint8 [nq, 32, 68])")
    if q_fp4 is None:
        _need(q_idx, torch.bfloat16, "q_idx")
        return _ptr(q_idx), q_idx.shape[0], suffix
    _need(q_fp4, torch.uint8, "q_fp4")
    if suffix != "_fp4k":
        raise ValueError("an MXFP4 indexer Q pairs with FP4 indexer-K entries (k_fp4)")
    return _ptr(q_fp4), q_fp4.numel() // (IDX_HEADS * KIDX_RECORD), "_fp4qk"


def kidx_fp4_pack(x, out=None, stream=None):
    """bf16 [n,128] indexer keys -> uint8 [n,68] FP4 entries (OCP MXFP4: 64 code bytes + one E8M0
    scale per 32 channels)."""
    _need(x, torch.bfloat16, "x")
    n = x.numel() // IDX_DIM
    if out is None:
        out = torch.empty((n, KIDX_RECORD), dtype=torch.uint8, device=x.device)
    _need(out, torch.uint8, "out")
    _check(load().kidx_fp4_pack(_ptr(x), n, _ptr(out), _stream(stream)), "kidx_fp4_pack")
    return out


def swa_fp8_pack(x, out=None, stream=None):
    """bf16 [n,512] window rows -> uint8 [n,528] FP8 rows (512 E4M3 codes + 16 E8M0 scales)."""
    _need(x, torch.bfloat16, "x")
    n = x.numel() // DIM
    if out is None:
        out = torch.empty((n, SWA_RECORD), dtype=torch.uint8, device=x.device)
    _need(out, torch.uint8, "out")
    _check(load().swa_fp8_pack(_ptr(x), n, _ptr(out), _stream(stream)), "swa_fp8_pack")
    return out


def csa2_index_full(q_idx, w, k_idx, N, q_per_seq, n_visible=None, block_size=0, scores=None, block_scores=None,
                    stream=None, k_fp4=None, q_fp4=None):
    """Full-mode indexer scores [nq,N] fp32 (and block maxima [nq,ceil(N/8)] when block_size == 8).
    The indexer K is bf16 `k_idx` [nseq,N,128], or FP4 entries `k_fp4` [nseq,N,68] (pass k_idx=None);
    with `q_fp4` [nq,32,68] (MXFP4 query entries, q_idx=None, k_fp4 required) the call is
    csa2_index_full_fp4qk."""
    for t, dt, nm in [(w, torch.float32, "w"), (n_visible, torch.int32, "n_visible")]:
        _need(t, dt, nm)
    kp, suffix = _k_args(k_idx, k_fp4)
    qp, nq, suffix = _q_args(q_idx, q_fp4, suffix)
    dev = w.device
    if scores is None:
        scores = torch.empty((nq, N), dtype=torch.float32, device=dev)
    if block_size and block_scores is None:
        block_scores = torch.empty((nq, (N + 7) // 8), dtype=torch.float32, device=dev)
    fn = getattr(load(), "csa2_index_full" + suffix)
    _check(fn(qp, _ptr(w), kp, N, nq, q_per_seq, _ptr(n_visible), _ptr(scores), block_size,
              _ptr(block_scores) if block_size else None, _stream(stream)), "csa2_index_full" + suffix)
    return (scores, block_scores) if block_size else scores


def csa2_index_topk_workspace_bytes(nq, N, k):
    return load().csa2_index_topk_workspace_bytes(nq, N, k)


def csa2_index_topk(q_idx, w, k_idx, N, k, n_visible=None, block_size=0, top=None, block_scores=None,
                    scores=None, workspace=None, stream=None, k_fp4=None, stage="both", q_fp4=None):
    """Full-mode scores fused with Top-k (decode, one query per sequence):
    int32 [nq,k] (and block maxima [nq,ceil(N/8)] when block_size == 8).
    `scores` [nq,N] fp32, when given, also receives the score rows.
    stage: "both" (complete), "select" (scoring + per-chunk selection, the
    candidates stay in `workspace`) or "merge" (completes a "select" call
    with the same top/workspace; the other inputs are ignored). `q_fp4`
    [nq,32,68] (with k_fp4, q_idx=None) selects the MXFP4-Q calls."""
    for t, dt, nm in [(w, torch.float32, "w"), (n_visible, torch.int32, "n_visible"), (scores, torch.float32, "scores")]:
        _need(t, dt, nm)
    kp, suffix = _k_args(k_idx, k_fp4)
    qp, nq, suffix = _q_args(q_idx, q_fp4, suffix)
    dev = w.device
    if top is None:
        top = torch.empty((nq, k), dtype=torch.int32, device=dev)
    if block_size and block_scores is None:
        block_scores = torch.empty((nq, (N + 7) // 8), dtype=torch.float32, device=dev)
    need = csa2_index_topk_workspace_bytes(nq, N, k)
    if workspace is None and need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stage == "merge":
        _check(load().csa2_index_topk_merge(N, nq, k, _ptr(top), _ptr(workspace), wsb, _stream(stream)),
               "csa2_index_topk_merge")
        return top
    args = (N, nq, _ptr(n_visible), k, _ptr(top), block_size, _ptr(block_scores) if block_size else None,
            _ptr(scores), _ptr(workspace), wsb, _stream(stream))
    if stage == "select" and suffix == "_fp4qk":
        _check(load().csa2_index_topk_select_fp4qk(qp, _ptr(w), kp, *args), "csa2_index_topk_select_fp4qk")
    elif stage == "select":
        _check(load().csa2_index_topk_select(qp, _ptr(w), kp, 1 if suffix else 0, *args), "csa2_index_topk_select")
    else:
        fn = getattr(load(), "csa2_index_topk" + suffix)
        _check(fn(qp, _ptr(w), kp, *args), "csa2_index_topk" + suffix)
    return (top, block_scores) if block_size else top


def csa2_index_topk_pool_workspace_bytes(nq, N, k, pool_k):
    return load().csa2_index_topk_pool_workspace_bytes(nq, N, k, pool_k)


def csa2_index_topk_merge_pool(N, k, top, block_scores, pool_k, cand_blocks=None, workspace=None, stream=None):
    """Completes a csa2_index_topk(stage="select", block_size=8) call: its
    Top-k into `top` and the pool's Top-pool_k blocks of `block_scores` into
    `cand_blocks` (int32 [nq,pool_k]). `workspace` is the select call's, of at
    least csa2_index_topk_pool_workspace_bytes(nq, N, k, pool_k) bytes."""
    for t, dt, nm in [(top, torch.int32, "top"), (block_scores, torch.float32, "block_scores"),
                      (cand_blocks, torch.int32, "cand_blocks")]:
        _need(t, dt, nm)
    nq = top.shape[0]
    if cand_blocks is None:
        cand_blocks = torch.empty((nq, pool_k), dtype=torch.int32, device=top.device)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().csa2_index_topk_merge_pool(N, nq, k, _ptr(top), _ptr(block_scores), pool_k, _ptr(cand_blocks),
                                             _ptr(workspace), wsb, _stream(stream)), "csa2_index_topk_merge_pool")
    return top, cand_blocks


def csa2_index_prefill_topk_workspace_bytes(nq, N, k):
    return load().csa2_index_prefill_topk_workspace_bytes(nq, N, k)


def csa2_index_prefill_topk(q_idx, w, k_idx, N, q_per_seq, k, n_visible=None, top=None, scores=None, workspace=None,
                            stream=None, k_fp4=None, q_fp4=None):
    """Prefill-chunk scores fused with Top-k (q_per_seq a multiple of 8,
    k <= 512): int32 [nq,k]. `scores` [nq,N] fp32, when given, also receives
    the score rows. `q_fp4` [nq,32,68] (with k_fp4) selects the MXFP4-Q call."""
    for t, dt, nm in [(w, torch.float32, "w"), (n_visible, torch.int32, "n_visible"),
                      (scores, torch.float32, "scores"), (top, torch.int32, "top")]:
        _need(t, dt, nm)
    kp, suffix = _k_args(k_idx, k_fp4)
    qp, nq, suffix = _q_args(q_idx, q_fp4, suffix)
    dev = w.device
    if top is None:
        top = torch.empty((nq, k), dtype=torch.int32, device=dev)
    need = csa2_index_prefill_topk_workspace_bytes(nq, N, k)
    if workspace is None and need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    fn = getattr(load(), "csa2_index_prefill_topk" + suffix)
    _check(fn(qp, _ptr(w), kp, N, nq, q_per_seq, _ptr(n_visible), k, _ptr(top), _ptr(scores),
              _ptr(workspace), wsb, _stream(stream)), "csa2_index_prefill_topk" + suffix)
    return top


def csa2_index_topk_noalloc_scratch_bytes():
    return load().csa2_index_topk_noalloc_scratch_bytes()


def csa2_index_topk_noalloc(q_idx, w, k_idx, N, k, n_visible=None, block_size=0, top=None, block_scores=None,
                            scores=None, stream=None, k_fp4=None):
    """csa2_index_topk without a workspace: the library's static device scratch
    holds the candidates (calls overlapping on one GPU race). Outputs must be
    passed in (`top`, and `block_scores` when block_size == 8) for a call that
    allocates nothing; missing ones are allocated here, outside the call."""
    for t, dt, nm in [(q_idx, torch.bfloat16, "q_idx"), (w, torch.float32, "w"), (n_visible, torch.int32, "n_visible"),
                      (scores, torch.float32, "scores"), (top, torch.int32, "top"),
                      (block_scores, torch.float32, "block_scores")]:
        _need(t, dt, nm)
    kp, suffix = _k_args(k_idx, k_fp4)
    nq = q_idx.shape[0]
    dev = q_idx.device
    if top is None:
        top = torch.empty((nq, k), dtype=torch.int32, device=dev)
    if block_size and block_scores is None:
        block_scores = torch.empty((nq, (N + 7) // 8), dtype=torch.float32, device=dev)
    _check(load().csa2_index_topk_noalloc(_ptr(q_idx), _ptr(w), kp, 1 if suffix else 0, N, nq, _ptr(n_visible), k,
                                          _ptr(top), block_size, _ptr(block_scores) if block_size else None,
                                          _ptr(scores), _stream(stream)), "csa2_index_topk_noalloc")
    return (top, block_scores) if block_size else top


def csa2_index_reindex(q_idx, w, k_idx, N, q_per_seq, cand_blocks, n_visible=None, block_size=8, pool_scores=None,
                       pool_ids=None, want_ids=True, stream=None, k_fp4=None, q_fp4=None):
    """Reindex-mode scores over the pool [nq, nb*8] fp32 (+ entry ids [nq, nb*8] int32).
    The indexer K is bf16 `k_idx`, or FP4 entries `k_fp4` (pass k_idx=None); `q_fp4`
    [nq,32,68] (with k_fp4, q_idx=None) selects csa2_index_reindex_fp4qk."""
    for t, dt, nm in [(w, torch.float32, "w"), (cand_blocks, torch.int32, "cand_blocks"),
                      (n_visible, torch.int32, "n_visible")]:
        _need(t, dt, nm)
    kp, suffix = _k_args(k_idx, k_fp4)
    qp, _, suffix = _q_args(q_idx, q_fp4, suffix)
    nq, nb = cand_blocks.shape
    dev = w.device
    if pool_scores is None:
        pool_scores = torch.empty((nq, nb * block_size), dtype=torch.float32, device=dev)
    if want_ids and pool_ids is None:
        pool_ids = torch.empty((nq, nb * block_size), dtype=torch.int32, device=dev)
    fn = getattr(load(), "csa2_index_reindex" + suffix)
    _check(fn(qp, _ptr(w), kp, N, nq, q_per_seq, _ptr(n_visible), _ptr(cand_blocks), nb, block_size,
              _ptr(pool_scores), _ptr(pool_ids), _stream(stream)), "csa2_index_reindex" + suffix)
    return pool_scores, pool_ids


def csa2_index_reindex_topk_workspace_bytes(nq, nb, k):
    return load().csa2_index_reindex_topk_workspace_bytes(nq, nb, k)


def csa2_index_reindex_topk(q_idx, w, k_idx, N, q_per_seq, cand_blocks, k, n_visible=None, top=None,
                            pool_scores=None, workspace=None, stream=None, k_fp4=None, q_fp4=None):
    """Reindex-mode scores over the pool fused with the Top-k: int32 [nq, k]
    entry ids (csa2_topk of csa2_index_reindex's pool row through its ids).
    `pool_scores` [nq, nb*8] fp32, when given, also receives the pool row.
    `q_fp4` [nq,32,68] (with k_fp4, q_idx=None) selects the MXFP4-Q call."""
    for t, dt, nm in [(w, torch.float32, "w"), (cand_blocks, torch.int32, "cand_blocks"),
                      (n_visible, torch.int32, "n_visible"), (pool_scores, torch.float32, "pool_scores")]:
        _need(t, dt, nm)
    kp, suffix = _k_args(k_idx, k_fp4)
    qp, _, suffix = _q_args(q_idx, q_fp4, suffix)
    nq, nb = cand_blocks.shape
    dev = w.device
    if top is None:
        top = torch.empty((nq, k), dtype=torch.int32, device=dev)
    need = csa2_index_reindex_topk_workspace_bytes(nq, nb, k)
    if workspace is None and need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    fn = getattr(load(), "csa2_index_reindex_topk" + suffix)
    _check(fn(qp, _ptr(w), kp, N, nq, q_per_seq, _ptr(n_visible), _ptr(cand_blocks), nb, k, _ptr(top),
              _ptr(pool_scores), _ptr(workspace), wsb, _stream(stream)), "csa2_index_reindex_topk" + suffix)
    return top


def csa2_topk_workspace_bytes(rows, ncols, k):
    return load().csa2_topk_workspace_bytes(rows, ncols, k)


def csa2_topk(scores, k, row_len=None, id_map=None, out=None, workspace=None, stream=None):
    """Per-row Top-K columns ascending, -1 padded: int32 [rows, k]."""
    _need(scores, torch.float32, "scores")
    _need(row_len, torch.int32, "row_len")
    _need(id_map, torch.int32, "id_map")
    rows, ncols = scores.shape
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=scores.device)
    need = csa2_topk_workspace_bytes(rows, ncols, k)
    if workspace is None and need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=scores.device)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().csa2_topk(_ptr(scores), rows, ncols, ncols, _ptr(row_len), k, _ptr(id_map), _ptr(out),
                            _ptr(workspace), wsb, _stream(stream)), "csa2_topk")
    return out


STATUS_IDX, STATUS_WIN_LEN, STATUS_WIN_RANGE, STATUS_NONFINITE = 1, 2, 4, 8


def attn_status(workspace):
    """The status word of an attention workspace (CSA2_STATUS_* bits; the
    caller zeroes it before the calls it covers and reads it after them)."""
    return int(workspace[:4].view(torch.int32)[0].item())


def csa2_sparse_attn_workspace_bytes(nq, k):
    return load().csa2_sparse_attn_workspace_bytes(nq, k)


def csa2_sparse_attn(q, kv, N, q_per_seq, idx, swa=None, swa_start=None, swa_len=None, softmax_scale=None,
                     out=None, lse=None, want_lse=True, workspace=None, stream=None, swa_fp8=None):
    """Sparse MQA attention: bf16 out [nq,64,512] (and lse [nq,64] fp32).
    The window rows are bf16 `swa` [nseq,T,512], or FP8 rows `swa_fp8`
    [nseq,T,528] (pass swa=None)."""
    if swa is not None and swa_fp8 is not None:
        raise ValueError("pass at most one of swa (bf16) and swa_fp8 (uint8 [.., 528])")
    for t, dt, nm in [(q, torch.bfloat16, "q"), (kv, torch.uint8, "kv"), (idx, torch.int32, "idx"),
                      (swa, torch.bfloat16, "swa"), (swa_fp8, torch.uint8, "swa_fp8"),
                      (swa_start, torch.int32, "swa_start"), (swa_len, torch.int32, "swa_len")]:
        _need(t, dt, nm)
    nq = q.shape[0]
    k = idx.shape[1]
    win = swa if swa_fp8 is None else swa_fp8
    T = win.shape[-2] if win is not None else 0
    if softmax_scale is None:
        softmax_scale = DIM ** -0.5
    if out is None:
        out = torch.empty((nq, HEADS, DIM), dtype=torch.bfloat16, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty((nq, HEADS), dtype=torch.float32, device=q.device)
    need = csa2_sparse_attn_workspace_bytes(nq, k)
    if workspace is None and need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    name = "csa2_sparse_attn" if swa_fp8 is None else "csa2_sparse_attn_fp8w"
    _check(getattr(load(), name)(_ptr(q), _ptr(kv), N, nq, q_per_seq, _ptr(idx), k, _ptr(win), T, _ptr(swa_start),
                                 _ptr(swa_len), float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace), wsb,
                                 _stream(stream)), name)
    return out, lse
