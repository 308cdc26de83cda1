"""ctypes front-end of the CSA2 CPU oracle (``csa2_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark. The product package never imports it and
shares no code with it. Arrays are numpy; bf16 travels as ``uint16`` bit
patterns.

Every function states the passage of the pages it follows; the C source holds
the full citations.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libcsa2_oracle.so")
_lib = None

RECORD_BYTES = 288
KIDX_RECORD_BYTES = 68  # FP4 indexer-K entry (OCP MXFP4): 64 code bytes + 4 E8M0 scales (one per 32 channels)
SWA_RECORD_BYTES = 528  # FP8 window row: 512 E4M3 codes + 16 E8M0 scales (one per 32 channels)
IDX_HEADS, IDX_DIM, HEADS, DIM = 32, 128, 64, 512


def build(force=True):
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
             _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        vp, i64, i32, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        L.orc_e4m3_value.restype = f64
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_value.restype = f64
        L.orc_e2m1_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_encode_nonneg.restype = ctypes.c_uint8
        L.orc_e4m3_encode_nonneg.argtypes = [ctypes.c_float]
        L.orc_e2m1_encode.restype = ctypes.c_uint8
        L.orc_e2m1_encode.argtypes = [f64, f64]
        L.orc_fp4_pack.argtypes = [vp, i64, vp]
        L.orc_fp4_unpack.argtypes = [vp, i64, vp]
        L.orc_index_full.argtypes = [vp, vp, vp, i64, i32, i32, vp, vp, i32, vp]
        L.orc_index_full_fp4k.argtypes = [vp, vp, vp, i64, i32, i32, vp, vp, i32, vp]
        L.orc_index_full_fp4qk.argtypes = [vp, vp, vp, i64, i32, i32, vp, vp, i32, vp]
        L.orc_index_reindex_fp4qk.argtypes = [vp, vp, vp, i64, i32, i32, vp, vp, i64, vp]
        L.orc_kidx_fp4_pack.argtypes = [vp, i64, vp]
        L.orc_kidx_fp4_unpack.argtypes = [vp, i64, vp]
        L.orc_index_reindex_fp4k.argtypes = [vp, vp, vp, i64, i32, i32, vp, vp, i64, vp]
        L.orc_pool_ids.argtypes = [vp, i32, i32, i32, vp]
        L.orc_index_reindex.argtypes = [vp, vp, vp, i64, i32, i32, vp, vp, i64, vp]
        L.orc_topk.argtypes = [vp, i32, i64, i64, vp, i32, vp, vp]
        L.orc_sparse_attn.argtypes = [vp, vp, i64, i32, i32, vp, i32, vp, i64, vp, vp, f64, vp, vp]
        L.orc_sparse_attn_fp8w.argtypes = [vp, vp, i64, i32, i32, vp, i32, vp, i64, vp, vp, f64, vp, vp]
        L.orc_swa_fp8_pack.argtypes = [vp, i64, vp]
        L.orc_swa_fp8_unpack.argtypes = [vp, i64, vp]
        L.orc_e8m0_value.restype = f64
        L.orc_e8m0_value.argtypes = [ctypes.c_uint8]
        L.orc_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def num_threads():
    return lib().orc_num_threads()


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def e4m3_value(b):
    """OCP E4M3 byte -> value (NaN for 0x7F / 0xFF)."""
    return lib().orc_e4m3_value(int(b))


def e2m1_value(n):
    """OCP E2M1 nibble -> value."""
    return lib().orc_e2m1_value(int(n))


def e4m3_encode(v):
    """Nearest non-negative E4M3 code to float32 v, ties to even, saturating."""
    return lib().orc_e4m3_encode_nonneg(float(np.float32(v)))


def e2m1_encode(x, S):
    """Nearest E2M1 code for x on the grid scaled by S, ties to even."""
    return lib().orc_e2m1_encode(float(x), float(S))


def fp4_pack(x_bf16):
    """FP4 main-KV record of each 512-channel bf16 row (eogee.com report 3.4)."""
    x = _c(x_bf16, np.uint16).reshape(-1, DIM)
    out = np.zeros((x.shape[0], RECORD_BYTES), np.uint8)
    lib().orc_fp4_pack(_p(x), x.shape[0], _p(out))
    return out


def fp4_unpack(rec):
    """Exact values of FP4 records, float64 [n, 512]."""
    r = _c(rec, np.uint8).reshape(-1, RECORD_BYTES)
    out = np.zeros((r.shape[0], DIM), np.float64)
    lib().orc_fp4_unpack(_p(r), r.shape[0], _p(out))
    return out


def kidx_fp4_pack(x_bf16):
    """FP4 indexer-K entry of each 128-channel bf16 row [n, 68] uint8, read as
    OCP MXFP4 (eogee.com report 3.4 names the standard; the 68 B size comes
    from the 890 B/token accounting): 64 code bytes + one E8M0 scale per 32
    channels."""
    x = _c(x_bf16, np.uint16).reshape(-1, IDX_DIM)
    out = np.zeros((x.shape[0], KIDX_RECORD_BYTES), np.uint8)
    lib().orc_kidx_fp4_pack(_p(x), x.shape[0], _p(out))
    return out


def kidx_fp4_unpack(rec):
    """Exact values of FP4 indexer-K entries, float64 [n, 128]."""
    r = _c(rec, np.uint8).reshape(-1, KIDX_RECORD_BYTES)
    out = np.zeros((r.shape[0], IDX_DIM), np.float64)
    lib().orc_kidx_fp4_unpack(_p(r), r.shape[0], _p(out))
    return out


def index_full(q_idx, w, k_idx, N, q_per_seq, n_visible=None, block_size=0, k_fp4=None, q_fp4=None):
    """Full-mode indexer scores [nq, N] float32 (+ block maxima when block_size>0).
    The indexer K is bf16 `k_idx` [nseq, N, 128], or FP4 entries `k_fp4`
    [nseq, N, 68] when given (then k_idx is ignored). With `q_fp4` [nq, 32, 68]
    (MXFP4 indexer Q, one entry per head; eogee.com report 3.4: the indexer Q/K
    ran in FP4) the query is read from those entries (q_idx is ignored) and the
    K must be FP4 entries too."""
    if q_fp4 is not None:
        qq = _c(q_fp4, np.uint8).reshape(-1, IDX_HEADS * KIDX_RECORD_BYTES)
        nq = qq.shape[0]
        assert k_fp4 is not None, "the MXFP4-Q scoring reads FP4 K entries"
        scores = np.zeros((nq, N), np.float32)
        nb = (N + block_size - 1) // block_size if block_size > 0 else 0
        blocks = np.zeros((nq, nb), np.float32) if block_size > 0 else None
        lib().orc_index_full_fp4qk(_p(qq), _p(_c(w, np.float32)), _p(_c(k_fp4, np.uint8)), N, nq, q_per_seq,
                                   _p(_c(n_visible, np.int32)), _p(scores), block_size, _p(blocks))
        return (scores, blocks) if block_size > 0 else scores
    q = _c(q_idx, np.uint16)
    nq = q.shape[0]
    ww = _c(w, np.float32)
    nv = _c(n_visible, np.int32)
    scores = np.zeros((nq, N), np.float32)
    nb = (N + block_size - 1) // block_size if block_size > 0 else 0
    blocks = np.zeros((nq, nb), np.float32) if block_size > 0 else None
    if k_fp4 is not None:
        k = _c(k_fp4, np.uint8)
        lib().orc_index_full_fp4k(_p(q), _p(ww), _p(k), N, nq, q_per_seq, _p(nv), _p(scores), block_size,
                                  _p(blocks))
    else:
        k = _c(k_idx, np.uint16)
        lib().orc_index_full(_p(q), _p(ww), _p(k), N, nq, q_per_seq, _p(nv), _p(scores), block_size, _p(blocks))
    return (scores, blocks) if block_size > 0 else scores


def pool_ids(blocks, block_size):
    """Candidate-pool entry ids from chosen block ids (eogee.com report 3.3)."""
    b = _c(blocks, np.int32)
    nq, nb = b.shape
    out = np.zeros((nq, nb * block_size), np.int32)
    lib().orc_pool_ids(_p(b), nq, nb, block_size, _p(out))
    return out


def index_reindex(q_idx, w, k_idx, N, q_per_seq, pool, n_visible=None, k_fp4=None, q_fp4=None):
    """Reindex-mode scores over pool positions [nq, pool_len] float32 (FP4
    indexer K from `k_fp4` when given; MXFP4 indexer Q from `q_fp4`
    [nq, 32, 68] when given, which needs the FP4 K)."""
    pl = _c(pool, np.int32)
    out = np.zeros(pl.shape, np.float32)
    if q_fp4 is not None:
        assert k_fp4 is not None, "the MXFP4-Q scoring reads FP4 K entries"
        qq = _c(q_fp4, np.uint8).reshape(-1, IDX_HEADS * KIDX_RECORD_BYTES)
        lib().orc_index_reindex_fp4qk(_p(qq), _p(_c(w, np.float32)), _p(_c(k_fp4, np.uint8)), N, qq.shape[0],
                                      q_per_seq, _p(_c(n_visible, np.int32)), _p(pl), pl.shape[1], _p(out))
        return out
    q = _c(q_idx, np.uint16)
    nq = q.shape[0]
    if k_fp4 is not None:
        lib().orc_index_reindex_fp4k(_p(q), _p(_c(w, np.float32)), _p(_c(k_fp4, np.uint8)), N, nq, q_per_seq,
                                     _p(_c(n_visible, np.int32)), _p(pl), pl.shape[1], _p(out))
    else:
        lib().orc_index_reindex(_p(q), _p(_c(w, np.float32)), _p(_c(k_idx, np.uint16)), N, nq, q_per_seq,
                                _p(_c(n_visible, np.int32)), _p(pl), pl.shape[1], _p(out))
    return out


def topk(scores, k, row_len=None, id_map=None):
    """Per-row Top-K positions, ascending, -1 padded [rows, k] int32."""
    s = _c(scores, np.float32)
    rows, ncols = s.shape
    out = np.zeros((rows, k), np.int32)
    lib().orc_topk(_p(s), rows, ncols, ncols, _p(_c(row_len, np.int32)), k, _p(_c(id_map, np.int32)), _p(out))
    return out


def sparse_attn(q, kv, N, q_per_seq, idx, swa, T, swa_start, swa_len, softmax_scale=1.0 / np.sqrt(512.0),
                swa_fp8=None):
    """Sparse MQA attention; returns (out [nq,64,512] float64, lse [nq,64] float64).
    The window rows are bf16 `swa` [nseq,T,512], or FP8 rows `swa_fp8`
    [nseq,T,528] when given (then swa is ignored)."""
    qq = _c(q, np.uint16)
    nq = qq.shape[0]
    ii = _c(idx, np.int32)
    k = ii.shape[1]
    out = np.zeros((nq, HEADS, DIM), np.float64)
    lse = np.zeros((nq, HEADS), np.float64)
    args = (_p(_c(swa_start, np.int32)), _p(_c(swa_len, np.int32)), float(softmax_scale), _p(out), _p(lse))
    if swa_fp8 is not None:
        lib().orc_sparse_attn_fp8w(_p(qq), _p(_c(kv, np.uint8)), N, nq, q_per_seq, _p(ii), k,
                                   _p(_c(swa_fp8, np.uint8)), T, *args)
    else:
        lib().orc_sparse_attn(_p(qq), _p(_c(kv, np.uint8)), N, nq, q_per_seq, _p(ii), k, _p(_c(swa, np.uint16)), T,
                              *args)
    return out, lse


def e8m0_value(b):
    """OCP E8M0 scale byte -> value (2^(b-127); 255 is NaN)."""
    return lib().orc_e8m0_value(int(b))


def swa_fp8_pack(x_bf16):
    """FP8 window rows [n, 528] uint8 of bf16 rows [n, 512] ([EOG] 3.4 FP8 SWA
    KV, read as OCP MXFP8: E4M3 elements, one E8M0 scale per 32 channels)."""
    x = _c(x_bf16, np.uint16).reshape(-1, DIM)
    out = np.zeros((x.shape[0], SWA_RECORD_BYTES), np.uint8)
    lib().orc_swa_fp8_pack(_p(x), x.shape[0], _p(out))
    return out


def swa_fp8_unpack(rec):
    """Exact values of FP8 window rows, float64 [n, 512]."""
    r = _c(rec, np.uint8).reshape(-1, SWA_RECORD_BYTES)
    out = np.zeros((r.shape[0], DIM), np.float64)
    lib().orc_swa_fp8_unpack(_p(r), r.shape[0], _p(out))
    return out
