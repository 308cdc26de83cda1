"""GPU parity of each C-ABI call against the CPU oracle on seeded inputs, at
sizes the oracle finishes in seconds that still span several tiles and a
ragged tail, plus the degenerate cases. Bars: bit-exact for FP4 records,
decoded values and Top-K indices; indexer scores within 1e-3 relative (floor
1e-5 * max|ref|); attention within 1e-2 * max|ref|."""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as O
from tests._conv import bf16_bits_to_f64, dev_i32, np_, rel_close, u16

pytestmark = pytest.mark.gpu
DEV = "cuda"
SCALE = 1.0 / math.sqrt(512.0)


def K():
    import kv_cache_compression_csa2_amd as k
    return k


def _g(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def _bf16(shape, seed, scale=1.0):
    return (torch.randn(shape, generator=_g(seed), device=DEV) * scale).to(torch.bfloat16)


def _records(n, seed):
    from kv_cache_compression_csa2_amd.workloads import random_records
    return random_records(n, _g(seed), DEV)


# ------------------------------------------------------------------ FP4

def test_pack_bit_exact_random_scales():
    print("case: pack random", flush=True)
    x = _bf16((3000, 512), 1) * torch.exp2(torch.randint(-20, 12, (3000, 1), generator=_g(2), device=DEV)).to(
        torch.bfloat16)
    x[0] = 0
    x[1, :16] = -0.0
    x[2, :16] = 1e-30
    x[3, :32] = 3e4  # saturating group
    rec = K().fp4_kv_pack(x.contiguous())
    torch.cuda.synchronize()
    ref = O.fp4_pack(u16(x))
    assert np.array_equal(np_(rec), ref)


def test_pack_bit_exact_ties():
    """Inputs exactly on the E2M1 midpoints of their group's scale."""
    print("case: pack ties", flush=True)
    rng = np.random.default_rng(3)
    S = torch.tensor(np.exp2(rng.integers(-9, 8, (512, 32, 1))).astype(np.float32))
    mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], dtype=torch.float32)
    pick = torch.tensor(rng.integers(0, 8, (512, 32, 16)))
    sign = torch.tensor(rng.choice([-1.0, 1.0], (512, 32, 16)).astype(np.float32))
    v = (mids[pick] * sign * S)
    v[:, :, 0] = 6.0 * S[:, :, 0]  # amax = 6S so the scale is exactly S
    x = v.reshape(512, 512).to(torch.bfloat16).to(DEV)
    rec = K().fp4_kv_pack(x)
    torch.cuda.synchronize()
    assert np.array_equal(np_(rec), O.fp4_pack(u16(x)))


def test_unpack_exhaustive_and_roundtrip():
    print("case: unpack exhaustive", flush=True)
    # every (code, scale byte) pair: record r, group g uses scale byte (r*32+g) % 256
    n = 64
    rec = np.zeros((n, 288), np.uint8)
    for r in range(n):
        rec[r, :256] = np.arange(256, dtype=np.uint8)  # each byte = two codes: all 16x16 pairs
    for r in range(n):
        sc = (r * 32 + np.arange(32)) % 256
        sc[(sc == 0x7F) | (sc == 0xFF)] = 0x7E
        rec[r, 256:] = sc
        rec[r, :256] = np.arange(256, dtype=np.uint8)
    y = K().fp4_kv_unpack(torch.tensor(rec, device=DEV))
    torch.cuda.synchronize()
    got = bf16_bits_to_f64(u16(y))
    ref = O.fp4_unpack(rec)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))
    # pack(unpack(x)) keeps values (grid points with any scale)
    x = _bf16((256, 512), 5)
    r1 = K().fp4_kv_pack(x)
    back = K().fp4_kv_unpack(r1)
    r2 = K().fp4_kv_pack(back)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits_to_f64(u16(K().fp4_kv_unpack(r2))), bf16_bits_to_f64(u16(back)))


def test_pack_empty():
    out = torch.empty((0, 288), dtype=torch.uint8, device=DEV)
    K().fp4_kv_pack(torch.empty((0, 512), dtype=torch.bfloat16, device=DEV), out=out)
    torch.cuda.synchronize()


# ------------------------------------------------------ FP4 indexer K

def test_kidx_pack_bit_exact():
    print("case: kidx pack", flush=True)
    x = _bf16((5000, 128), 11) * torch.exp2(torch.randint(-30, 20, (5000, 1), generator=_g(12), device=DEV)).to(
        torch.bfloat16)
    x[0] = 0
    x[1, :] = -0.0
    x[2, :64] = 1e-35
    x[3, :32] = 1e-39  # a block of bf16 subnormals (scale byte 0, codes up to 2)
    x[3, 32:64] = -3e-39
    x[4, 96:] = 3e38   # the largest binades
    # exact ties: amax 6 * 2^e so the scale is 2^e, the rest on the grid midpoints
    rng = np.random.default_rng(13)
    e = torch.tensor(np.exp2(rng.integers(-20, 20, (100, 1))).astype(np.float32))
    mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
    v = mids[torch.tensor(rng.integers(0, 8, (100, 128)))] * torch.tensor(
        rng.choice([-1.0, 1.0], (100, 128)).astype(np.float32)) * e
    v[:, 0] = 6.0 * e[:, 0]
    x[100:200] = v.to(torch.bfloat16).to(DEV)
    x = x.contiguous()
    rec = K().kidx_fp4_pack(x)
    torch.cuda.synchronize()
    assert np.array_equal(np_(rec), O.kidx_fp4_pack(u16(x)))
    out = torch.empty((0, 68), dtype=torch.uint8, device=DEV)
    K().kidx_fp4_pack(torch.empty((0, 128), dtype=torch.bfloat16, device=DEV), out=out)  # n == 0
    torch.cuda.synchronize()


@pytest.mark.parametrize("nq,N,qps", [(1, 1024, 1), (3, 1000, 1), (5, 77, 1), (2, 40000, 1), (4, 1, 1),
                                      (16, 5003, 16), (24, 4096 * 2 + 100, 8)])
def test_index_full_fp4k_matches_oracle(nq, N, qps):
    """Scores over FP4 indexer-K entries packed by the oracle; the decode
    kernel (one sequence per query) and the prefill kernel (8 | q_per_seq)."""
    print("case: index_full_fp4k", nq, N, qps, flush=True)
    q, w, k = _idx_inputs(nq, N, nq // qps, 20 + N)
    kf_host = O.kidx_fp4_pack(u16(k)).reshape(nq // qps, N, 68)
    kf = torch.tensor(kf_host, device=DEV)
    rng = np.random.default_rng(N + 1)
    nv = rng.integers(0, N + 1, nq).astype(np.int32)
    nv[0] = N
    s, b = K().csa2_index_full(q, w, None, N, qps, n_visible=dev_i32(nv, DEV), block_size=8, k_fp4=kf)
    torch.cuda.synchronize()
    rs, rb = O.index_full(u16(q), np_(w), None, N, qps, n_visible=nv, block_size=8, k_fp4=kf_host)
    ok, msg = rel_close(np_(s), rs)
    assert ok, msg
    ok, msg = rel_close(np_(b), rb)
    assert ok, msg
    s2 = K().csa2_index_full(q, w, None, N, qps, n_visible=dev_i32(nv, DEV), k_fp4=kf)  # no blocks
    torch.cuda.synchronize()
    ok, msg = rel_close(np_(s2), rs)
    assert ok, msg


@pytest.mark.parametrize("qps", [1, 8])
def test_index_fp4k_decodes_every_code_and_scale_exactly(qps):
    """Every E2M1 code under every E8M0 scale byte 2..252 (the bytes whose
    decoded values are normal numbers; the packer never writes more than 252),
    in every channel position: entry i holds one nonzero code in channel
    i % 128 and scale byte b in all four blocks. Head 0 of the query is all
    ones and head 1 all minus ones, so with w = (1, 1) the score is |v| and
    with w = (1, 0) it is max(v, 0): the decoded value v = E2M1 * 2^(b-127)
    must come out bit-exact. qps 1: the decode kernel; 8: the prefill kernel."""
    print("case: fp4k exhaustive decode", qps, flush=True)
    bs = np.arange(2, 253)
    codes = np.arange(16)
    n = len(bs) * len(codes)
    ent = np.zeros((n, 68), np.uint8)
    i = np.arange(n)
    b, c = bs[i // 16], codes[i % 16]
    ch = i % 128
    ent[i, ch // 2] = (c << (4 * (ch % 2))).astype(np.uint8)
    ent[:, 64:] = b[:, None].astype(np.uint8)
    nq = 2 if qps == 1 else 8
    nseq = nq // qps
    kf_host = np.ascontiguousarray(np.broadcast_to(ent, (nseq, n, 68)))
    q = torch.zeros((nq, 32, 128), dtype=torch.bfloat16)
    q[:, 0] = 1.0
    q[:, 1] = -1.0
    w = torch.zeros((nq, 32), dtype=torch.float32)
    w[:, 0] = 1.0
    w[0::2, 1] = 1.0
    q, w = q.to(DEV), w.to(DEV)
    s = K().csa2_index_full(q, w, None, n, qps, k_fp4=torch.tensor(kf_host, device=DEV))
    torch.cuda.synchronize()
    ref = O.index_full(u16(q), np_(w), None, n, qps, k_fp4=kf_host)
    assert np.array_equal(np_(s), ref)
    v = O.kidx_fp4_unpack(ent)[i, ch]
    assert np.array_equal(ref[0], np.abs(v).astype(np.float32))
    assert np.array_equal(ref[1], np.maximum(v, 0).astype(np.float32))


# ------------------------------------------- MXFP4 indexer Q and K


def _fp4qk_inputs(nq, N, nseq, seed):
    """bf16 queries and keys packed by the oracle's own packer into MXFP4
    entries (one per query head / per key), and the GPU packer's query entries,
    which must be the same bytes."""
    q, w, k = _idx_inputs(nq, N, nseq, seed)
    qf_host = O.kidx_fp4_pack(u16(q).reshape(-1, 128)).reshape(nq, 32, 68)
    kf_host = O.kidx_fp4_pack(u16(k).reshape(-1, 128)).reshape(nseq, N, 68)
    qf = K().kidx_fp4_pack(q.reshape(-1, 128)).reshape(nq, 32, 68)
    torch.cuda.synchronize()
    assert np.array_equal(np_(qf), qf_host)
    return qf, qf_host, w, torch.tensor(kf_host, device=DEV), kf_host


@pytest.mark.parametrize("nq,N,qps", [(8, 1000, 8), (16, 5003, 16), (24, 4096 * 2 + 100, 8), (8, 1, 8),
                                      (8, 64, 8), (32, 4097, 32), (1, 1024, 1), (3, 1000, 1), (5, 77, 1),
                                      (2, 40000, 1), (4, 1, 1), (12, 3000, 3)])
def test_index_full_fp4qk_matches_oracle(nq, N, qps):
    """MXFP4 query and key entries on the scaled FP4 matrix instruction: scores
    and block maxima within the score tolerance of the oracle (exact products,
    fp32 sums), with causal-like visible lengths and ragged tails; the prefill
    kernel (8 | q_per_seq) and the streaming kernel (the rest)."""
    print("case: index_full_fp4qk", nq, N, qps, flush=True)
    qf, qf_host, w, kf, kf_host = _fp4qk_inputs(nq, N, nq // qps, 30 + N + nq)
    rng = np.random.default_rng(N + 7)
    nv = rng.integers(0, N + 1, nq).astype(np.int32)
    nv[0] = N
    s, b = K().csa2_index_full(None, w, None, N, qps, n_visible=dev_i32(nv, DEV), block_size=8, k_fp4=kf, q_fp4=qf)
    s2 = K().csa2_index_full(None, w, None, N, qps, k_fp4=kf, q_fp4=qf)  # every entry visible, no blocks
    torch.cuda.synchronize()
    rs, rb = O.index_full(None, np_(w), None, N, qps, n_visible=nv, block_size=8, k_fp4=kf_host, q_fp4=qf_host)
    ok, msg = rel_close(np_(s), rs)
    assert ok, msg
    ok, msg = rel_close(np_(b), rb)
    assert ok, msg
    ok, msg = rel_close(np_(s2), O.index_full(None, np_(w), None, N, qps, k_fp4=kf_host, q_fp4=qf_host))
    assert ok, msg


@pytest.mark.parametrize("qps", [1, 8])
def test_index_fp4qk_products_exact_for_every_code_and_scale(qps):
    """Every E2M1 key code under every E8M0 scale byte 2..252 in every channel
    position (as the FP4-K exhaustive test), against queries whose four blocks
    carry different scales: head 0 is +1 in every channel with block scales
    1, 2, 1/2, 4, head 1 is -1 everywhere. The score with w = (1, 1) is
    v*m if v > 0 else -v, and with w = (1, 0) max(v*m, 0), for the decoded key
    value v and the channel's block multiplier m: bit-exact."""
    print("case: fp4qk exhaustive products", qps, flush=True)
    bs = np.arange(2, 253)
    n = len(bs) * 16
    i = np.arange(n)
    b, c, ch = bs[i // 16], i % 16, i % 128
    ent = np.zeros((n, 68), np.uint8)
    ent[i, ch // 2] = (c << (4 * (ch % 2))).astype(np.uint8)
    ent[:, 64:] = b[:, None].astype(np.uint8)
    nq = 8
    qent = np.zeros((nq, 32, 68), np.uint8)
    qent[:, 0, :64] = 0x22          # code 2 = +1.0 in both nibbles
    qent[:, 0, 64:] = [127, 128, 126, 129]
    qent[:, 1, :64] = 0xAA          # code 10 = -1.0
    qent[:, 1, 64:] = 127
    qent[:, 2:, 64:] = 127          # zero codes elsewhere
    w = torch.zeros((nq, 32), dtype=torch.float32)
    w[:, 0] = 1.0
    w[0::2, 1] = 1.0
    kent = np.ascontiguousarray(np.broadcast_to(ent, (nq // qps, n, 68)))
    s = K().csa2_index_full(None, w.to(DEV), None, n, qps, k_fp4=torch.tensor(kent, device=DEV),
                            q_fp4=torch.tensor(qent, device=DEV))
    torch.cuda.synchronize()
    ref = O.index_full(None, np_(w), None, n, qps, k_fp4=kent, q_fp4=qent)
    assert np.array_equal(np_(s), ref)
    v = O.kidx_fp4_unpack(ent)[i, ch]
    m = np.array([1.0, 2.0, 0.5, 4.0])[ch // 32]
    assert np.array_equal(ref[0], np.where(v > 0, v * m, -v).astype(np.float32))
    assert np.array_equal(ref[1], np.maximum(v * m, 0).astype(np.float32))


def _fp4qk_exact_entries(n, rng):
    """Random MXFP4 entries with scale bytes 126..127: every product of a
    query and a key value is a multiple of 1/16 below 36 in magnitude, so with
    power-of-two weights of at most 1 every score is exact in fp32."""
    e = rng.integers(0, 256, (n, 68)).astype(np.uint8)
    e[:, 64:] = rng.integers(126, 128, (n, 4))
    return e


@pytest.mark.parametrize("nq,qps,N,k", [(8, 8, 5003, 512), (16, 8, 70000, 512), (24, 24, 20000, 100),
                                        (8, 8, 600, 512), (64, 64, 4096, 512)])
def test_index_prefill_topk_fp4qk_bit_exact_on_exact_scores(nq, qps, N, k):
    """Prefill scoring with MXFP4 Q and K fused with Top-k, on exact-score
    entries: the selection equals the oracle's Top-K of the oracle's score row
    (one chunk, several chunks, rows with fewer visible entries than k or none)."""
    print("case: prefill_topk fp4qk exact", nq, qps, N, k, flush=True)
    rng = np.random.default_rng(1500 + N + nq)
    qf_host = _fp4qk_exact_entries(nq * 32, rng).reshape(nq, 32, 68)
    kf_host = _fp4qk_exact_entries((nq // qps) * N, rng).reshape(nq // qps, N, 68)
    w_host = np.exp2(rng.integers(-2, 1, (nq, 32))).astype(np.float32)
    nv = rng.integers(N // 2, N + 1, nq).astype(np.int32)
    nv[0], nv[-1], nv[1] = N, min(k // 2, N), 0
    top = K().csa2_index_prefill_topk(None, torch.tensor(w_host, device=DEV), None, N, qps, k,
                                      n_visible=dev_i32(nv, DEV), k_fp4=torch.tensor(kf_host, device=DEV),
                                      q_fp4=torch.tensor(qf_host, device=DEV))
    torch.cuda.synchronize()
    rs = O.index_full(None, w_host, None, N, qps, n_visible=nv, k_fp4=kf_host, q_fp4=qf_host)
    assert np.array_equal(np_(top), O.topk(rs, k, row_len=nv))


@pytest.mark.parametrize("nq,N,k", [(3, 20000, 512), (2, 8192, 512), (4, 1000, 512), (2, 70000, 2048),
                                    (3, 20000, 100), (8, 65536, 512)])
def test_index_topk_fp4qk_bit_exact_on_exact_scores(nq, N, k):
    """Decode Full scoring with MXFP4 Q and K fused with Top-k, on exact-score
    entries: the oracle's Top-K of the oracle's score row (one chunk, several,
    a ragged tail, the two-level merge, rows with fewer visible entries than k
    or none), with the block maxima, and the select + merge launches apart."""
    print("case: index_topk fp4qk exact", nq, N, k, flush=True)
    rng = np.random.default_rng(1700 + N + k + nq)
    qf_host = _fp4qk_exact_entries(nq * 32, rng).reshape(nq, 32, 68)
    kf_host = _fp4qk_exact_entries(nq * N, rng).reshape(nq, N, 68)
    w_host = np.exp2(rng.integers(-2, 1, (nq, 32))).astype(np.float32)
    nv = rng.integers(N // 2, N + 1, nq).astype(np.int32)
    nv[0], nv[1] = N, 0
    if nq > 2:
        nv[2] = min(k // 2, N)
    qf, kf, w, nvd = (torch.tensor(qf_host, device=DEV), torch.tensor(kf_host, device=DEV),
                      torch.tensor(w_host, device=DEV), dev_i32(nv, DEV))
    top, blk = K().csa2_index_topk(None, w, None, N, k, n_visible=nvd, block_size=8, k_fp4=kf, q_fp4=qf)
    ws = torch.empty((max(K().csa2_index_topk_workspace_bytes(nq, N, k), 1),), dtype=torch.uint8, device=DEV)
    top2 = torch.empty_like(top)
    K().csa2_index_topk(None, w, None, N, k, n_visible=nvd, top=top2, workspace=ws, k_fp4=kf, q_fp4=qf,
                        stage="select")
    K().csa2_index_topk(None, w, None, N, k, top=top2, workspace=ws, k_fp4=kf, q_fp4=qf, stage="merge")
    torch.cuda.synchronize()
    rs, rb = O.index_full(None, w_host, None, N, 1, n_visible=nv, block_size=8, k_fp4=kf_host, q_fp4=qf_host)
    top_o = O.topk(rs, k, row_len=nv)
    assert np.array_equal(np_(top), top_o)
    assert np.array_equal(np_(top2), top_o)
    assert np.array_equal(np_(blk), rb)


@pytest.mark.parametrize("nq,N,nb,k,qps", [(2, 1 << 20, 2048, 512, 1), (3, 9000, 300, 512, 1),
                                           (16, 40000, 1000, 100, 8)])
def test_index_reindex_fp4qk_matches_oracle_and_topk_is_exact(nq, N, nb, k, qps):
    """Reindex with MXFP4 Q and K: pool scores within the score tolerance of
    the oracle on random entries (pool ids exact), and on exact-score entries
    the fused Reindex + Top-k equals the oracle's Top-K through the pool ids
    (padding blocks, blocks shared by sequences of several queries)."""
    print("case: reindex fp4qk", nq, N, nb, k, qps, flush=True)
    rng = np.random.default_rng(1800 + N + nb)
    blocks = np.sort(np.stack([rng.choice((N + 7) // 8, nb, replace=False) for _ in range(nq)]), 1).astype(np.int32)
    blocks[0, -3:] = -1
    nv = rng.integers(N // 2, N + 1, nq).astype(np.int32)
    pool = O.pool_ids(blocks, 8)
    # random entries: scores
    qf, qf_host, w, kf, kf_host = _fp4qk_inputs(nq, N, nq // qps, 1900 + nb)
    ps, pid = K().csa2_index_reindex(None, w, None, N, qps, dev_i32(blocks, DEV), n_visible=dev_i32(nv, DEV),
                                     k_fp4=kf, q_fp4=qf)
    torch.cuda.synchronize()
    ref = O.index_reindex(None, np_(w), None, N, qps, pool, n_visible=nv, k_fp4=kf_host, q_fp4=qf_host)
    ok, msg = rel_close(np_(ps), ref)
    assert ok, msg
    assert np.array_equal(np_(pid), np.where((pool >= 0) & (pool < nv[:, None]), pool, -1))
    # exact-score entries: the fused selection
    qx = _fp4qk_exact_entries(nq * 32, rng).reshape(nq, 32, 68)
    kx = _fp4qk_exact_entries((nq // qps) * N, rng).reshape(nq // qps, N, 68)
    wx = np.exp2(rng.integers(-2, 1, (nq, 32))).astype(np.float32)
    top = K().csa2_index_reindex_topk(None, torch.tensor(wx, device=DEV), None, N, qps, dev_i32(blocks, DEV), k,
                                      n_visible=dev_i32(nv, DEV), k_fp4=torch.tensor(kx, device=DEV),
                                      q_fp4=torch.tensor(qx, device=DEV))
    torch.cuda.synchronize()
    rx = O.index_reindex(None, wx, None, N, qps, pool, n_visible=nv, k_fp4=kx, q_fp4=qx)
    assert np.array_equal(np_(top), O.topk(rx, k, id_map=pool))


def test_index_prefill_topk_fp4qk_matches_the_unfused_path():
    """Random MXFP4 entries at the prefill chunk's row length: the fused call's
    debug score rows equal csa2_index_full_fp4qk's bit for bit, and its
    selection is csa2_topk of that row with the causal row lengths."""
    print("case: prefill_topk fp4qk random", flush=True)
    nq, N, k = 64, 65536, 512
    qf, _, w, kf, _ = _fp4qk_inputs(nq, N, 1, 1600)
    nv = dev_i32(np.arange(N - nq + 1, N + 1), DEV)
    sc = torch.empty((nq, N), dtype=torch.float32, device=DEV)
    top = K().csa2_index_prefill_topk(None, w, None, N, nq, k, n_visible=nv, scores=sc, k_fp4=kf, q_fp4=qf)
    ref_sc = K().csa2_index_full(None, w, None, N, nq, n_visible=nv, k_fp4=kf, q_fp4=qf)
    ref_top = K().csa2_topk(ref_sc, k, row_len=nv)
    torch.cuda.synchronize()
    assert torch.equal(sc, ref_sc)
    assert torch.equal(top, ref_top)


def test_index_reindex_fp4k_matches_oracle():
    print("case: reindex fp4k", flush=True)
    nq, N, nb = 3, 9000, 300
    q, w, k = _idx_inputs(nq, N, nq, 78)
    kf_host = O.kidx_fp4_pack(u16(k)).reshape(nq, N, 68)
    kf = torch.tensor(kf_host, device=DEV)
    rng = np.random.default_rng(8)
    blocks = np.sort(np.stack([rng.choice((N + 7) // 8, nb, replace=False) for _ in range(nq)]), 1).astype(np.int32)
    blocks[1, -5:] = -1
    nv = np.array([N, 5000, 8999], np.int32)
    ps, pid = K().csa2_index_reindex(q, w, None, N, 1, dev_i32(blocks, DEV), n_visible=dev_i32(nv, DEV), k_fp4=kf)
    torch.cuda.synchronize()
    pool = O.pool_ids(blocks, 8)
    pool_vis = np.where((pool >= 0) & (pool < nv[:, None]), pool, -1)
    ref = O.index_reindex(u16(q), np_(w), None, N, 1, pool, n_visible=nv, k_fp4=kf_host)
    ok, msg = rel_close(np_(ps), ref)
    assert ok, msg
    assert np.array_equal(np_(pid), pool_vis)


# ------------------------------------------------------ fused scoring + Top-K

def _int_idx_inputs(nq, N, seed, nseq=None):
    """Small-integer queries and keys and power-of-two weights: every score is
    an exact fp32 value whatever the summation order, with many ties."""
    g = _g(seed)
    q = torch.randint(-2, 3, (nq, 32, 128), generator=g, device=DEV).to(torch.bfloat16)
    w = torch.exp2(torch.randint(-2, 2, (nq, 32), generator=g, device=DEV).float())
    k = torch.randint(-2, 3, (nq if nseq is None else nseq, N, 128), generator=g, device=DEV).to(torch.bfloat16)
    return q, w, k


@pytest.mark.parametrize("nq,N,k,fp4", [(3, 20000, 512, False), (2, 8192, 512, False), (4, 1000, 512, False),
                                        (2, 70000, 2048, False), (3, 20000, 100, False), (3, 20000, 512, True),
                                        (2, 70000, 2048, True)])
def test_index_topk_bit_exact_on_exact_scores(nq, N, k, fp4):
    """With exact scores the fused selection must equal the oracle's Top-K of
    the oracle's score row, ties included (one chunk, several chunks, a
    ragged tail, the two-level merge at 70000 x 2048, FP4 keys)."""
    print("case: index_topk exact", nq, N, k, fp4, flush=True)
    q, w, kb = _int_idx_inputs(nq, N, 500 + N + k)
    nv = np.array([N, N // 3, 0, 7][:nq], np.int32)
    nvd = dev_i32(nv, DEV)
    if fp4:
        kf_host = O.kidx_fp4_pack(u16(kb)).reshape(nq, N, 68)
        kf = torch.tensor(kf_host, device=DEV)
        top, blk = K().csa2_index_topk(q, w, None, N, k, n_visible=nvd, block_size=8, k_fp4=kf)
        rs, rb = O.index_full(u16(q), np_(w), None, N, 1, n_visible=nv, block_size=8, k_fp4=kf_host)
    else:
        top, blk = K().csa2_index_topk(q, w, kb, N, k, n_visible=nvd, block_size=8)
        rs, rb = O.index_full(u16(q), np_(w), u16(kb), N, 1, n_visible=nv, block_size=8)
    torch.cuda.synchronize()
    assert np.array_equal(np_(blk), rb)
    assert np.array_equal(np_(top), O.topk(rs, k, row_len=nv))


def test_index_topk_matches_oracle_and_the_unfused_path():
    print("case: index_topk random", flush=True)
    nq, N, k = 4, 33000, 512
    q, w, kb = _idx_inputs(nq, N, nq, 600)
    nv = np.array([N, 30000, 513, 20], np.int32)
    nvd = dev_i32(nv, DEV)
    sc = torch.empty((nq, N), dtype=torch.float32, device=DEV)
    top = K().csa2_index_topk(q, w, kb, N, k, n_visible=nvd, scores=sc)
    s_ref = K().csa2_index_full(q, w, kb, N, 1, n_visible=nvd)
    t_ref = K().csa2_topk(s_ref, k, row_len=nvd)
    torch.cuda.synchronize()
    # the debug scores are the unfused kernel's, and so is the selection
    assert torch.equal(sc, s_ref)
    assert torch.equal(top, t_ref)
    # against the oracle: scores within 1e-3 relative, selections overlap
    rs = O.index_full(u16(q), np_(w), u16(kb), N, 1, n_visible=nv)
    ok, msg = rel_close(np_(sc), rs)
    assert ok, msg
    to = O.topk(rs, k, row_len=nv)
    for r in range(nq):
        a = set(np_(top[r]).tolist()) - {-1}
        b = set(to[r].tolist()) - {-1}
        assert len(a & b) >= 0.995 * len(b)


def _merge_pool(q, w, kb, kf, N, k, pool_k, nvd):
    """select (block maxima on) + csa2_index_topk_merge_pool, one workspace."""
    nq = q.shape[0]
    ws = torch.empty((max(K().csa2_index_topk_pool_workspace_bytes(nq, N, k, pool_k), 1),), dtype=torch.uint8,
                     device=DEV)
    top = torch.empty((nq, k), dtype=torch.int32, device=DEV)
    blk = torch.empty((nq, (N + 7) // 8), dtype=torch.float32, device=DEV)
    K().csa2_index_topk(q, w, kb, N, k, n_visible=nvd, block_size=8, top=top, block_scores=blk, workspace=ws,
                        k_fp4=kf, stage="select")
    _, cand = K().csa2_index_topk_merge_pool(N, k, top, blk, pool_k, workspace=ws)
    return top, blk, cand


@pytest.mark.parametrize("nq,N,k,pool_k,fp4", [(3, 20000, 512, 2048, False), (2, 70000, 512, 2048, False),
                                               (4, 1000, 512, 200, False), (2, 70000, 2048, 512, True),
                                               (3, 40000, 100, 3000, False)])
def test_index_topk_merge_pool_bit_exact_on_exact_scores(nq, N, k, pool_k, fp4):
    """The Top-k merge and the pool's block selection sharing launches give
    exactly the oracle's Top-k of the oracle's score row and its Top-pool_k of
    the oracle's block maxima (ties included; one chunk, two-level merges,
    pools wider than the block row)."""
    print("case: index_topk_merge_pool exact", nq, N, k, pool_k, fp4, flush=True)
    q, w, kb = _int_idx_inputs(nq, N, 900 + N + k)
    nv = np.array([N, N // 3, 0, 7][:nq], np.int32)
    kf_host = O.kidx_fp4_pack(u16(kb)).reshape(nq, N, 68) if fp4 else None
    top, blk, cand = _merge_pool(q, w, None if fp4 else kb, torch.tensor(kf_host, device=DEV) if fp4 else None, N, k,
                                 pool_k, dev_i32(nv, DEV))
    torch.cuda.synchronize()
    rs, rb = O.index_full(u16(q), np_(w), None if fp4 else u16(kb), N, 1, n_visible=nv, block_size=8, k_fp4=kf_host)
    assert np.array_equal(np_(blk), rb)
    assert np.array_equal(np_(top), O.topk(rs, k, row_len=nv))
    assert np.array_equal(np_(cand), O.topk(rb, pool_k))


@pytest.mark.parametrize("nq,N,k,pool_k", [(2, 7, 512, 3), (3, 13, 5, 1), (1, 8, 1, 1), (4, 4100, 512, 4096)])
def test_index_topk_merge_pool_degenerate_shapes(nq, N, k, pool_k):
    """Rows shorter than one block, k above the row length, pools wider than
    the block row, single entries: the oracle's Top-k and Top-pool_k, -1 padded."""
    print("case: index_topk_merge_pool degenerate", nq, N, k, pool_k, flush=True)
    q, w, kb = _int_idx_inputs(nq, N, 1300 + N)
    nv = np.array([N, max(N // 3, 1), 0, 1][:nq], np.int32)
    top, blk, cand = _merge_pool(q, w, kb, None, N, k, pool_k, dev_i32(nv, DEV))
    torch.cuda.synchronize()
    rs, rb = O.index_full(u16(q), np_(w), u16(kb), N, 1, n_visible=nv, block_size=8)
    assert np.array_equal(np_(blk), rb)
    assert np.array_equal(np_(top), O.topk(rs, k, row_len=nv))
    assert np.array_equal(np_(cand), O.topk(rb, pool_k))


@pytest.mark.parametrize("nq,N,pool_k", [(8, 1 << 20, 2048), (32, 262144, 2048), (1, 1 << 21, 4096),
                                         (2, 4096, 2048)])
def test_index_topk_merge_pool_matches_the_separate_calls(nq, N, pool_k):
    """At the decode shapes (8 x 1M: both selections two levels; 32 x 256K:
    one merge level against two block levels), a pool that needs the
    global-memory Top-K (1 x 2M, 4096 blocks: the calls run apart) and a row
    of one chunk: the same ids as csa2_index_topk + csa2_topk of its block
    maxima."""
    print("case: index_topk_merge_pool vs separate", nq, N, pool_k, flush=True)
    k = 512
    q, w, kb = _idx_inputs(nq, N, nq, 950 + nq)
    nv = np.full(nq, N, np.int32)
    nv[-1] = N - 12345 if N > 20000 else N
    nvd = dev_i32(nv, DEV)
    top, blk, cand = _merge_pool(q, w, kb, None, N, k, pool_k, nvd)
    t_ref, b_ref = K().csa2_index_topk(q, w, kb, N, k, n_visible=nvd, block_size=8)
    c_ref = K().csa2_topk(b_ref, pool_k)
    torch.cuda.synchronize()
    assert torch.equal(blk, b_ref)
    assert torch.equal(top, t_ref)
    assert torch.equal(cand, c_ref)
    del kb


# ------------------------------------------------------------------ indexer

def _idx_inputs(nq, N, nseq, seed):
    q = _bf16((nq, 32, 128), seed)
    w = torch.rand((nq, 32), generator=_g(seed + 1), device=DEV)
    k = _bf16((nseq, N, 128), seed + 2)
    return q, w, k


@pytest.mark.parametrize("nq,N,qps", [(1, 1024, 1), (3, 1000, 1), (5, 77, 1), (2, 40000, 1), (4, 1, 1),
                                      (16, 5003, 16), (24, 4096 * 2 + 100, 8)])
def test_index_full_matches_oracle(nq, N, qps):
    print("case: index_full", nq, N, qps, flush=True)
    q, w, k = _idx_inputs(nq, N, nq // qps, 10 + N)
    rng = np.random.default_rng(N)
    nv = rng.integers(0, N + 1, nq).astype(np.int32)
    nv[0] = N
    s, b = K().csa2_index_full(q, w, k, N, qps, n_visible=dev_i32(nv, DEV), block_size=8)
    torch.cuda.synchronize()
    rs, rb = O.index_full(u16(q), np_(w), u16(k), N, qps, n_visible=nv, block_size=8)
    ok, msg = rel_close(np_(s), rs)
    assert ok, msg
    ok, msg = rel_close(np_(b), rb)
    assert ok, msg
    s2 = K().csa2_index_full(q, w, k, N, qps)  # no visibility limit, no blocks
    torch.cuda.synchronize()
    ok, msg = rel_close(np_(s2), O.index_full(u16(q), np_(w), u16(k), N, qps))
    assert ok, msg


def test_index_reindex_matches_oracle():
    print("case: reindex", flush=True)
    nq, N, nb = 3, 9000, 300
    q, w, k = _idx_inputs(nq, N, nq, 77)
    rng = np.random.default_rng(7)
    blocks = np.sort(np.stack([rng.choice((N + 7) // 8, nb, replace=False) for _ in range(nq)]), 1).astype(np.int32)
    blocks[1, -5:] = -1
    nv = np.array([N, 5000, 8999], np.int32)
    ps, pid = K().csa2_index_reindex(q, w, k, N, 1, dev_i32(blocks, DEV), n_visible=dev_i32(nv, DEV))
    torch.cuda.synchronize()
    pool = O.pool_ids(blocks, 8)
    pool_vis = np.where((pool >= 0) & (pool < nv[:, None]), pool, -1)
    ref = O.index_reindex(u16(q), np_(w), u16(k), N, 1, pool, n_visible=nv)
    ok, msg = rel_close(np_(ps), ref)
    assert ok, msg
    assert np.array_equal(np_(pid), pool_vis)


def _pool_blocks(nq, N, nb, seed):
    """Ascending distinct block ids per query, the last rows' tails padded with -1."""
    rng = np.random.default_rng(seed)
    nblk = (N + 7) // 8
    b = np.sort(np.stack([rng.choice(nblk, min(nb, nblk), replace=False) for _ in range(nq)]), 1).astype(np.int32)
    if b.shape[1] < nb:
        b = np.concatenate([b, np.full((nq, nb - b.shape[1]), -1, np.int32)], 1)
    if nq > 1:
        b[1, -5:] = -1
    return b


@pytest.mark.parametrize("nq,N,nb,k,qps,fp4", [(3, 9000, 300, 512, 1, False), (2, 70000, 2048, 512, 1, False),
                                               (4, 70000, 2048, 512, 2, False), (2, 70000, 2048, 2048, 1, False),
                                               (3, 20000, 2048, 512, 1, True), (40, 40000, 2048, 512, 1, False),
                                               (2, 5000, 10, 512, 1, False), (3, 9000, 300, 100, 3, True)])
def test_index_reindex_topk_bit_exact_on_exact_scores(nq, N, nb, k, qps, fp4):
    """With exact scores the fused Reindex selection must equal the oracle's
    Top-K of the oracle's pool row through the pool ids, ties included (one
    and several chunks of each length, queries sharing a sequence, padding
    blocks, a pool smaller than k, FP4 keys)."""
    print("case: reindex_topk exact", nq, N, nb, k, qps, fp4, flush=True)
    q, w, kb = _int_idx_inputs(nq, N, 900 + N + nb + k, nseq=nq // qps)
    blocks = _pool_blocks(nq, N, nb, N + nb)
    nv = np.array([N, N // 2, 3 * N // 4, 9, N, N // 3] * 8, np.int32)[:nq]
    pool = O.pool_ids(blocks, 8)
    if fp4:
        kf_host = O.kidx_fp4_pack(u16(kb)).reshape(nq // qps, N, 68)
        kf = torch.tensor(kf_host, device=DEV)
        top = K().csa2_index_reindex_topk(q, w, None, N, qps, dev_i32(blocks, DEV), k, n_visible=dev_i32(nv, DEV),
                                          k_fp4=kf)
        ref = O.index_reindex(u16(q), np_(w), None, N, qps, pool, n_visible=nv, k_fp4=kf_host)
    else:
        top = K().csa2_index_reindex_topk(q, w, kb, N, qps, dev_i32(blocks, DEV), k, n_visible=dev_i32(nv, DEV))
        ref = O.index_reindex(u16(q), np_(w), u16(kb), N, qps, pool, n_visible=nv)
    torch.cuda.synchronize()
    assert np.array_equal(np_(top), O.topk(ref, k, id_map=pool))


@pytest.mark.parametrize("nq,qps,N,k,fp4", [(16, 16, 5003, 512, False), (8, 8, 70000, 512, False),
                                            (64, 32, 20000, 100, False), (256, 256, 16384, 512, False),
                                            (24, 8, 9000, 512, True), (8, 8, 600, 512, False),
                                            (8, 8, 4096, 512, False), (16, 8, 4000, 300, True)])
def test_index_prefill_topk_bit_exact_on_exact_scores(nq, qps, N, k, fp4):
    """Prefill scoring fused with Top-k, on exact-score inputs (small-integer Q
    and K, power-of-two w, many ties): the selection must equal the oracle's
    Top-K of the oracle's score row with causal row lengths (one chunk per
    row, several chunks, a ragged tail, rows with fewer visible entries than
    k or none, FP4 keys)."""
    print("case: prefill_topk exact", nq, qps, N, k, fp4, flush=True)
    q, w, kb = _int_idx_inputs(nq, N, 1300 + N + k + nq, nseq=nq // qps)
    rng = np.random.default_rng(N + nq)
    nv = rng.integers(N // 2, N + 1, nq).astype(np.int32)
    nv[0], nv[-1] = N, min(k // 2, N)
    if nq > 2:
        nv[1] = 0
    nvd = dev_i32(nv, DEV)
    if fp4:
        kf_host = O.kidx_fp4_pack(u16(kb)).reshape(nq // qps, N, 68)
        kf = torch.tensor(kf_host, device=DEV)
        top = K().csa2_index_prefill_topk(q, w, None, N, qps, k, n_visible=nvd, k_fp4=kf)
        rs = O.index_full(u16(q), np_(w), None, N, qps, n_visible=nv, k_fp4=kf_host)
    else:
        top = K().csa2_index_prefill_topk(q, w, kb, N, qps, k, n_visible=nvd)
        rs = O.index_full(u16(q), np_(w), u16(kb), N, qps, n_visible=nv)
    torch.cuda.synchronize()
    assert np.array_equal(np_(top), O.topk(rs, k, row_len=nv))


def test_index_prefill_topk_matches_the_unfused_path():
    """Random inputs at the prefill chunk's row length: the fused call's debug
    score rows equal csa2_index_full's bit for bit, and its selection is
    csa2_topk of that row with the causal row lengths."""
    print("case: prefill_topk random", flush=True)
    nq, N, k = 64, 65536, 512
    q, w, kb = _idx_inputs(nq, N, 1, 1400)
    nv = dev_i32(np.arange(N - nq + 1, N + 1) // 1, DEV)
    sc = torch.empty((nq, N), dtype=torch.float32, device=DEV)
    top = K().csa2_index_prefill_topk(q, w, kb, N, nq, k, n_visible=nv, scores=sc)
    ref_sc = K().csa2_index_full(q, w, kb, N, nq, n_visible=nv)
    ref_top = K().csa2_topk(ref_sc, k, row_len=nv)
    torch.cuda.synchronize()
    assert torch.equal(sc, ref_sc)
    assert torch.equal(top, ref_top)


def test_index_prefill_topk_rising_scores_compact_often():
    """Scores that never fall along the row (every entry beats the current
    k-th best, so the candidate buffers fill and are compacted every few
    tiles), with long runs of equal scores: still the oracle's Top-K."""
    print("case: prefill_topk rising", flush=True)
    nq, N, k = 8, 30000, 512
    q = torch.zeros((nq, 32, 128), dtype=torch.bfloat16, device=DEV)
    q[:, 0, 0] = 1.0
    q[:, 1, 1] = 1.0
    w = torch.zeros((nq, 32), dtype=torch.float32, device=DEV)
    w[:, 0] = 1.0
    w[1::2, 1] = 0.5
    kb = torch.zeros((1, N, 128), dtype=torch.float32, device=DEV)
    kb[0, :, 0] = torch.arange(N, device=DEV, dtype=torch.float32) / 7.0  # bf16 rounding makes runs of ties
    kb[0, :, 1] = torch.arange(N, device=DEV, dtype=torch.float32) % 13
    kb = kb.to(torch.bfloat16)
    nv = dev_i32(np.array([N, N - 1, 20000, 513, 512, 100, N, 7], np.int32), DEV)
    top = K().csa2_index_prefill_topk(q, w, kb, N, nq, k, n_visible=nv)
    torch.cuda.synchronize()
    rs = O.index_full(u16(q), np_(w), u16(kb), N, nq, n_visible=np_(nv))
    assert np.array_equal(np_(top), O.topk(rs, k, row_len=np_(nv)))


def test_index_reindex_topk_matches_the_unfused_path():
    """Random inputs at the pages' pool size (2048 blocks): the fused call's
    debug pool row is csa2_index_reindex's, and its selection is csa2_topk of
    that row through the pool ids."""
    print("case: reindex_topk random", flush=True)
    nq, N, nb = 8, 100000, 2048
    q, w, kb = _idx_inputs(nq, N, nq, 910)
    blocks = dev_i32(_pool_blocks(nq, N, nb, 911), DEV)
    nv = dev_i32(np.array([N, 90000, 513, 20, N, 70000, 99999, 50000], np.int32), DEV)
    ps = torch.empty((nq, nb * 8), dtype=torch.float32, device=DEV)
    top = K().csa2_index_reindex_topk(q, w, kb, N, 1, blocks, 512, n_visible=nv, pool_scores=ps)
    ps_ref, pid = K().csa2_index_reindex(q, w, kb, N, 1, blocks, n_visible=nv)
    t_ref = K().csa2_topk(ps_ref, 512, id_map=pid)
    torch.cuda.synchronize()
    assert torch.equal(ps, ps_ref)
    assert torch.equal(top, t_ref)


# ------------------------------------------------------------------ Top-K

def _topk_check(scores_np, k, row_len=None, id_map=None):
    s = torch.tensor(scores_np, device=DEV)
    got = K().csa2_topk(s, k, row_len=None if row_len is None else dev_i32(row_len, DEV),
                        id_map=None if id_map is None else dev_i32(id_map, DEV))
    torch.cuda.synchronize()
    ref = O.topk(scores_np, k, row_len=row_len, id_map=id_map)
    assert np.array_equal(np_(got), ref)


@pytest.mark.parametrize("rows,n,k", [(1, 1024, 512), (3, 1000, 512), (64, 32768, 512), (8, 131072, 2048),
                                      (4, 300001, 512), (2, 1 << 20, 512), (300, 5000, 512), (2, 100, 4096),
                                      (2, 32769, 512), (3, 65536, 2048), (2, 300000, 4096), (1, 40000, 3),
                                      (2, 40000, 4096)])
def test_topk_bit_exact_on_oracle_scores(rows, n, k):
    print("case: topk", rows, n, k, flush=True)
    rng = np.random.default_rng(rows * 7 + n)
    s = rng.normal(0, 10, (rows, n)).astype(np.float32)
    _topk_check(s, k)


def test_topk_ties_nonfinite_and_lengths():
    print("case: topk ties", flush=True)
    rng = np.random.default_rng(1)
    s = (rng.integers(-50, 50, (6, 70000)) / 4).astype(np.float32)
    s[0, ::2] = -np.inf
    s[1, ::3] = np.nan
    s[2, :30000] = -0.0
    s[2, 30000:] = 0.0
    s[3] = 2.5
    s[4, :] = -np.inf
    s[5, 10:] = np.inf
    row_len = np.array([70000, 60000, 70000, 70000, 70000, 311], np.int32)
    _topk_check(s, 512, row_len=row_len)
    _topk_check(s, 2048)
    _topk_check(s[:, :600], 512)  # fewer candidates than k in some rows


@pytest.mark.parametrize("rows,n,k", [(4, 1 << 20, 512), (8, 131072, 2048), (64, 32768, 512)])
def test_topk_narrow_band(rows, n, k):
    """Scores packed in a narrow band (shared sign, exponent and leading
    mantissa bits), plus exact ties: the merge stage sees candidates that
    differ only in low bits."""
    print("case: topk narrow", rows, n, k, flush=True)
    rng = np.random.default_rng(rows + n + k)
    s = (100.0 + rng.normal(0, 0.01, (rows, n))).astype(np.float32)
    s[:, ::7] = np.float32(100.0)  # many keys equal to one value inside the band
    _topk_check(s, k)


@pytest.mark.parametrize("n_tie,n_above", [(40, 500), (300, 300), (700, 100)])
def test_topk_threshold_bin_sizes(n_tie, n_above):
    """The k-th key's first-digit bin holding <= 64 keys (one key per lane),
    65..512 keys (ballot bit select) and > 512 keys (two more histogram
    digits): n_tie copies of the k-th value, n_above larger values in other
    bins, background below; ties resolved by lowest position."""
    print("case: topk bin sizes", n_tie, n_above, flush=True)
    rng = np.random.default_rng(n_tie + n_above)
    rows, n, k = 4, 20000, 512
    s = (1.0 + rng.random((rows, n))).astype(np.float32)  # [1, 2)
    for r in range(rows):
        pos = rng.permutation(n)
        s[r, pos[:n_tie]] = np.float32(10.0)
        s[r, pos[n_tie:n_tie + n_above]] = (16.0 + 16.0 * rng.random(n_above)).astype(np.float32)
    _topk_check(s, k)
    _topk_check(s, 2048)


def test_topk_id_map():
    print("case: topk id_map", flush=True)
    rng = np.random.default_rng(2)
    s = rng.normal(0, 1, (5, 16384)).astype(np.float32)
    ids = np.sort(rng.choice(1 << 20, (5, 16384), replace=False), 1).astype(np.int32)
    ids[0, 100:200] = -1
    s[0, 100:200] = -np.inf
    _topk_check(s, 512, id_map=ids)


# ------------------------------------------------------------------ attention

def _attn_case(nq, N, k, qps, seed, T=128, slen=None, sstart=None, pad=0):
    q = _bf16((nq, 64, 512), seed)
    kv = _records((nq // qps) * N, seed + 1).view(nq // qps, N, 288)
    rng = np.random.default_rng(seed)
    idx = np.sort(np.stack([rng.choice(N, k, replace=False) for _ in range(nq)]), 1).astype(np.int32)
    if pad:
        idx[:, -pad:] = -1
    swa = _bf16((nq // qps, T, 512), seed + 2)
    sl = np.full(nq, 128 if slen is None else slen, np.int32) if slen is None or np.isscalar(slen) else slen
    st = np.zeros(nq, np.int32) if sstart is None else sstart
    return q, kv, idx, swa, st, sl


def _attn_check(q, kv, idx, swa, st, sl, N, qps, T):
    out, lse = K().csa2_sparse_attn(q, kv, N, qps, dev_i32(idx, DEV), swa, dev_i32(st, DEV), dev_i32(sl, DEV))
    torch.cuda.synchronize()
    ro, rl = O.sparse_attn(u16(q), np_(kv), N, qps, idx, u16(swa), T, st, sl, SCALE)
    got = bf16_bits_to_f64(u16(out))
    err = np.abs(got - ro).max()
    assert err <= 1e-2 * np.abs(ro).max(), (err, np.abs(ro).max())
    glse = np_(lse).astype(np.float64)
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(glse))
    assert np.allclose(glse[fin], rl[fin], rtol=1e-3, atol=2e-3)


@pytest.mark.parametrize("nq,N,k,pad", [(1, 1024, 512, 0), (3, 2000, 512, 7), (8, 5000, 512, 0), (2, 700, 100, 0),
                                        (40, 3000, 512, 3)])
def test_sparse_attn_decode_matches_oracle(nq, N, k, pad):
    print("case: attn", nq, N, k, pad, flush=True)
    q, kv, idx, swa, st, sl = _attn_case(nq, N, k, 1, 100 + nq, pad=pad)
    _attn_check(q, kv, idx, swa, st, sl, N, 1, 128)


def test_sparse_attn_no_split_many_queries():
    """>= 512 queries: one workgroup per query, output written directly."""
    print("case: attn 520", flush=True)
    nq, N = 520, 600
    q, kv, idx, swa, st, sl = _attn_case(nq, N, 512, nq, 5, T=nq + 127)
    st = np.arange(nq, dtype=np.int32)
    sl = np.full(nq, 128, np.int32)
    sl[:5] = [0, 1, 31, 33, 127]
    _attn_check(q, kv, idx, swa, st, sl, N, nq, nq + 127)


def test_sparse_attn_split_path():
    """129..511 queries: each query's tiles split over workgroups and merged."""
    print("case: attn split path", flush=True)
    nq, N = 200, 800
    q, kv, idx, swa, st, sl = _attn_case(nq, N, 512, 1, 6, pad=5)
    sl[:6] = [0, 1, 31, 33, 64, 127]
    _attn_check(q, kv, idx, swa, st, sl, N, 1, 128)


@pytest.mark.parametrize("nq", [15, 16, 63, 64, 127, 128, 511, 512])
def test_sparse_attn_split_table_boundaries(nq):
    """Batches on both sides of each step of the split table (7 / 4 / 2 / 1
    workgroups per query from 16 / 64 / 128 / 512 queries), so every split
    count and the unsplit path run against the oracle, with empty slots and
    mixed window lengths."""
    print("case: attn split boundary", nq, flush=True)
    N, T = 1500, 300
    q, kv, idx, swa, st, sl = _attn_case(nq, N, 512, 1, 40 + nq, T=T, pad=5)
    rng = np.random.default_rng(41 + nq)
    sl = rng.choice(np.array([0, 1, 32, 33, 96, 128], np.int32), nq).astype(np.int32)
    st = rng.integers(0, T - 128, nq).astype(np.int32)
    _attn_check(q, kv, idx, swa, st, sl, N, 1, T)


@pytest.mark.parametrize("nq,k", [(12, 512), (12, 80)])
def test_sparse_attn_window_lengths(nq, k):
    """Window lengths at and around tile boundaries, window starts inside the
    buffer, and fewer selected entries than one tile per wave."""
    print("case: attn window lengths", nq, k, flush=True)
    N, T = 900, 300
    q, kv, idx, swa, st, sl = _attn_case(nq, N, k, 1, 7 + k, T=T, pad=3)
    sl = np.array([0, 1, 31, 32, 33, 63, 64, 65, 97, 127, 128, 5], np.int32)[:nq]
    st = np.random.default_rng(8).integers(0, T - 128, nq).astype(np.int32)
    _attn_check(q, kv, idx, swa, st, sl, N, 1, T)


def test_sparse_attn_q_of_any_magnitude():
    """Every finite bf16 Q enters the fp16 products exactly: heads scaled far
    above fp16's range (2^20 .. 2^100), far below it (2^-20 .. 2^-100) and an
    all-zero head still match the oracle (hard-max and uniform softmaxes
    included)."""
    print("case: attn q magnitudes", flush=True)
    nq, N, k = 3, 2000, 512
    q, kv, idx, swa, st, sl = _attn_case(nq, N, k, 1, 501)
    ex = torch.tensor([0, 20, 100, -100, -20, 60, -60, 10] * 8, dtype=torch.float32, device=DEV)
    qs = (q.float() * torch.exp2(ex).view(1, 64, 1)).to(torch.bfloat16)
    qs[1, 5] = 0
    assert torch.isfinite(qs.float()).all()
    _attn_check(qs.contiguous(), kv, idx, swa, st, sl, N, 1, 128)


def _attn_status_of(q, kv, idx, swa, st, sl, N, swa_fp8=None):
    import kv_cache_compression_csa2_amd._lib as L
    nq, k = q.shape[0], idx.shape[1]
    ws = torch.empty((L.csa2_sparse_attn_workspace_bytes(nq, k),), dtype=torch.uint8, device=DEV)
    ws[:4].zero_()
    K().csa2_sparse_attn(q, kv, N, 1, dev_i32(idx, DEV), swa, dev_i32(st, DEV), dev_i32(sl, DEV), workspace=ws,
                         swa_fp8=swa_fp8)
    torch.cuda.synchronize()
    return L.attn_status(ws)


@pytest.mark.parametrize("nq", [6, 600])
def test_sparse_attn_status_reports_out_of_domain_inputs(nq):
    """Inputs outside the documented domain set their status bit (ids outside
    [-1, N), swa_len above 128, window rows past the buffer, window values fp16
    cannot hold, which leave a non-finite output); in-domain calls leave the
    word at 0. Both the split (6 queries) and the unsplit (600) launch."""
    import kv_cache_compression_csa2_amd._lib as L
    print("case: attn status", nq, flush=True)
    N, k, T = 1000, 64, 200
    q, kv, idx, swa, st, sl = _attn_case(nq, N, k, 1, 600 + nq, T=T)
    assert _attn_status_of(q, kv, idx, swa, st, sl, N) == 0
    bad = idx.copy()
    bad[1, 3] = N
    assert _attn_status_of(q, kv, bad, swa, st, sl, N) == L.STATUS_IDX
    bad[1, 3] = -7
    assert _attn_status_of(q, kv, bad, swa, st, sl, N) == L.STATUS_IDX
    sl2 = sl.copy()
    sl2[2] = 130
    assert _attn_status_of(q, kv, idx, swa, st, sl2, N) == L.STATUS_WIN_LEN
    st2 = st.copy()
    st2[3] = T - 10
    assert _attn_status_of(q, kv, idx, swa, st2, sl, N) == L.STATUS_WIN_RANGE
    swa2 = swa.clone()
    swa2[4, 5, 100] = 70000.0
    assert _attn_status_of(q, kv, idx, swa2, st, sl, N) == L.STATUS_NONFINITE
    swa2[4, 5, 100] = 65280.0  # the largest bf16 below 65504 is in range
    assert _attn_status_of(q, kv, idx, swa2, st, sl, N) == 0
    # FP8 rows: a block scale that lifts its values past 65504
    w8 = K().swa_fp8_pack(swa.reshape(-1, 512).contiguous()).view(swa.shape[0], T, 528)
    assert _attn_status_of(q, kv, idx, None, st, sl, N, swa_fp8=w8) == 0
    w8b = w8.clone()
    w8b[0, 7, 512 + 3] = 135
    assert _attn_status_of(q, kv, idx, None, st, sl, N, swa_fp8=w8b) == L.STATUS_NONFINITE


def test_visible_lengths_are_clamped_like_the_oracle():
    """n_visible above N acts as N and below 0 as 0 in every scoring call (and
    row_len likewise in csa2_topk), exactly as in the oracle."""
    print("case: visibility clamps", flush=True)
    nq, N = 8, 3000
    q, w, kb = _idx_inputs(nq, N, nq, 700)
    nv = np.array([N + 5, -3, 100, 2 ** 31 - 1, 0, N, 1, -2 ** 31], np.int32)
    nvd = dev_i32(nv, DEV)
    s = K().csa2_index_full(q, w, kb, N, 1, n_visible=nvd)
    top = K().csa2_index_topk(q, w, kb, N, 512, n_visible=nvd)
    torch.cuda.synchronize()
    rs = O.index_full(u16(q), np_(w), u16(kb), N, 1, n_visible=nv)
    ok, msg = rel_close(np_(s), rs)
    assert ok, msg
    assert np.array_equal(np_(top), O.topk(rs, 512, row_len=nv))
    assert np.array_equal(np_(K().csa2_topk(s, 512, row_len=nvd)), O.topk(np_(s), 512, row_len=nv))
    # prefill: 8 queries of one sequence
    q1, w1, k1 = _idx_inputs(8, N, 1, 710)
    s1 = K().csa2_index_full(q1, w1, k1, N, 8, n_visible=nvd)
    t1 = K().csa2_index_prefill_topk(q1, w1, k1, N, 8, 512, n_visible=nvd)
    torch.cuda.synchronize()
    r1 = O.index_full(u16(q1), np_(w1), u16(k1), N, 8, n_visible=nv)
    ok, msg = rel_close(np_(s1), r1)
    assert ok, msg
    assert np.array_equal(np_(t1), O.topk(np_(s1), 512, row_len=nv))
    # reindex: pool positions past the clamped length score -inf
    blocks = np.tile(np.arange(0, 300, 2, dtype=np.int32), (nq, 1))
    ps, pid = K().csa2_index_reindex(q, w, kb, N, 1, dev_i32(blocks, DEV), n_visible=nvd)
    torch.cuda.synchronize()
    pool = O.pool_ids(blocks, 8)
    ref = O.index_reindex(u16(q), np_(w), u16(kb), N, 1, pool, n_visible=nv)
    ok, msg = rel_close(np_(ps), ref)
    assert ok, msg


def test_sparse_attn_degenerate():
    print("case: attn degenerate", flush=True)
    nq, N = 4, 300
    q, kv, idx, swa, st, sl = _attn_case(nq, N, 64, 1, 9)
    idx[0, :] = -1  # window only
    idx[1, :] = -1
    sl[1] = 0  # no keys at all -> zeros, -inf
    sl[2] = 0  # selected entries only
    _attn_check(q, kv, idx, swa, st, sl, N, 1, 128)
    out, lse = K().csa2_sparse_attn(q, kv, N, 1, dev_i32(idx, DEV), swa, dev_i32(st, DEV), dev_i32(sl, DEV))
    torch.cuda.synchronize()
    assert torch.all(out[1] == 0) and torch.all(torch.isneginf(lse[1]))
    # k = 0, no window at all
    out2, lse2 = K().csa2_sparse_attn(q, kv, N, 1, torch.empty((nq, 0), dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert torch.all(out2 == 0) and torch.all(torch.isneginf(lse2))


def test_zero_queries():
    """Every call accepts an empty batch and launches nothing."""
    print("case: zero queries", flush=True)
    e = lambda *shape, dt=torch.bfloat16: torch.empty(shape, dtype=dt, device=DEV)
    N = 4096
    q, w = e(0, 32, 128), e(0, 32, dt=torch.float32)
    kb = _bf16((1, N, 128), 31)
    blocks = e(0, 2048, dt=torch.int32)
    s = K().csa2_index_full(q, w, kb, N, 1)
    top = K().csa2_index_topk(q, w, kb, N, 512)
    ps, pid = K().csa2_index_reindex(q, w, kb, N, 1, blocks)
    rt = K().csa2_index_reindex_topk(q, w, kb, N, 1, blocks, 512)
    t = K().csa2_topk(e(0, N, dt=torch.float32), 512)
    out, lse = K().csa2_sparse_attn(e(0, 64, 512), _records(N, 32).view(1, N, 288), N, 1, e(0, 512, dt=torch.int32))
    torch.cuda.synchronize()
    for x in (s, top, ps, pid, rt, t, out, lse):
        assert x.shape[0] == 0


def test_sparse_attn_decode_exact():
    """A query that attends to one entry outputs that entry's value exactly
    (softmax weight 1): every decoded E2M1 x E4M3 product must equal the
    oracle's unpacked value bit for bit. 8 records cover all 254 non-NaN scale
    bytes x 16 codes at every nibble and byte position; a second set of
    queries attends to one window row only (bf16 values of magnitude >= 2^-14
    pass through the kernel exactly)."""
    print("case: attn decode exact", flush=True)
    scales = [b for b in range(256) if b not in (0x7F, 0xFF)]
    nrec = 8
    rec = np.zeros((nrec, 288), np.uint8)
    for r in range(nrec):
        for g in range(32):
            rec[r, 256 + g] = scales[(r * 32 + g) % len(scales)]
            for i in range(0, 16, 2):
                lo, hi = (i + r + g) % 16, (i + 1 + r + g) % 16
                rec[r, 8 * g + i // 2] = lo | (hi << 4)
    want = O.fp4_unpack(rec)  # exact in bf16; compared as values (the sum of 1 x -0 and +0 is +0)
    kv = torch.tensor(rec, device=DEV).view(1, nrec, 288)
    q = _bf16((nrec, 64, 512), 21)
    idx = torch.arange(nrec, dtype=torch.int32, device=DEV).view(nrec, 1)
    out, lse = K().csa2_sparse_attn(q, kv.expand(nrec, nrec, 288).contiguous(), nrec, 1, idx)
    torch.cuda.synchronize()
    got = bf16_bits_to_f64(u16(out))
    for r in range(nrec):
        assert np.array_equal(got[r], np.broadcast_to(want[r], (64, 512))), r
    # window only: one row per query
    swa = torch.randn((nrec, 1, 512), generator=_g(22), device=DEV)
    swa = torch.where(swa.abs() < 2.0 ** -14, torch.zeros_like(swa), swa).to(torch.bfloat16)
    none = torch.full((nrec, 1), -1, dtype=torch.int32, device=DEV)
    st = torch.zeros((nrec,), dtype=torch.int32, device=DEV)
    sl = torch.ones((nrec,), dtype=torch.int32, device=DEV)
    out2, _ = K().csa2_sparse_attn(q, kv.expand(nrec, nrec, 288).contiguous(), nrec, 1, none, swa, st, sl)
    torch.cuda.synchronize()
    assert torch.equal(out2, swa.expand(nrec, 64, 512))


def _fp8_rows(n, seed):
    """bf16 window rows spanning several binades, zero blocks and saturating blocks."""
    g = _g(seed)
    x = torch.randn((n, 512), generator=g, device=DEV)
    x = x * torch.exp2(torch.randint(-20, 20, (n, 1), generator=g, device=DEV).float())
    x[: n // 8, 64:96] = 0.0                      # an all-zero block
    x[n // 8: n // 4, 0] = 3.99 * x[n // 8: n // 4, 1:32].abs().amax(1)  # block max near 2^(k+1): saturation
    return x.to(torch.bfloat16)


def test_swa_fp8_pack_bit_exact():
    print("case: swa fp8 pack", flush=True)
    x = _fp8_rows(777, 41)
    got = K().swa_fp8_pack(x)
    torch.cuda.synchronize()
    assert np.array_equal(np_(got), O.swa_fp8_pack(u16(x)))
    assert K().swa_fp8_pack(torch.empty((0, 512), dtype=torch.bfloat16, device=DEV)).shape == (0, 528)


@pytest.mark.parametrize("nq,N,k,pad,qps", [(3, 2000, 512, 7, 1), (40, 3000, 512, 3, 1), (2, 700, 100, 0, 1),
                                            (64, 600, 512, 0, 64)])
def test_sparse_attn_fp8_window_matches_oracle(nq, N, k, pad, qps):
    print("case: attn fp8 window", nq, N, k, pad, qps, flush=True)
    T = 128 if qps == 1 else nq + 127
    q, kv, idx, swa, st, sl = _attn_case(nq, N, k, qps, 300 + nq, T=T, pad=pad)
    if qps > 1:
        st = np.arange(nq, dtype=np.int32)
        sl = np.full(nq, 128, np.int32)
        sl[:3] = [0, 1, 33]
    w8 = K().swa_fp8_pack(swa.reshape(-1, 512).contiguous()).view(nq // qps, T, 528)
    torch.cuda.synchronize()
    w8o = O.swa_fp8_pack(u16(swa).reshape(-1, 512)).reshape(nq // qps, T, 528)
    assert np.array_equal(np_(w8), w8o)
    out, lse = K().csa2_sparse_attn(q, kv, N, qps, dev_i32(idx, DEV), None, dev_i32(st, DEV), dev_i32(sl, DEV),
                                    swa_fp8=w8)
    torch.cuda.synchronize()
    ro, rl = O.sparse_attn(u16(q), np_(kv), N, qps, idx, None, T, st, sl, SCALE, swa_fp8=w8o)
    got = bf16_bits_to_f64(u16(out))
    err = np.abs(got - ro).max()
    assert err <= 1e-2 * np.abs(ro).max(), (err, np.abs(ro).max())
    glse = np_(lse).astype(np.float64)
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(glse))
    assert np.allclose(glse[fin], rl[fin], rtol=1e-3, atol=2e-3)


def test_sparse_attn_fp8_window_decode_exact():
    """A query attending to one FP8 window row outputs that row's decoded
    values exactly (block maxima within [2^-7, 2^16))."""
    print("case: attn fp8 window exact", flush=True)
    nq = 8
    x = torch.randn((nq, 512), generator=_g(43), device=DEV)
    x = (x.view(nq, 16, 32) * torch.exp2(torch.randint(-6, 14, (nq, 16, 1), generator=_g(44), device=DEV).float())
         ).view(nq, 512).to(torch.bfloat16)
    w8 = K().swa_fp8_pack(x).view(nq, 1, 528)
    torch.cuda.synchronize()
    want = O.swa_fp8_unpack(np_(w8).reshape(nq, 528))
    q = _bf16((nq, 64, 512), 45)
    kv = _records(nq * 4, 46).view(nq, 4, 288)
    none = torch.full((nq, 1), -1, dtype=torch.int32, device=DEV)
    st = torch.zeros((nq,), dtype=torch.int32, device=DEV)
    sl = torch.ones((nq,), dtype=torch.int32, device=DEV)
    out, _ = K().csa2_sparse_attn(q, kv, 4, 1, none, None, st, sl, swa_fp8=w8)
    torch.cuda.synchronize()
    got = bf16_bits_to_f64(u16(out))
    for r in range(nq):
        assert np.array_equal(got[r], np.broadcast_to(want[r], (64, 512))), r


def test_sparse_attn_deterministic():
    print("case: attn determinism", flush=True)
    q, kv, idx, swa, st, sl = _attn_case(16, 4000, 512, 1, 11)
    a = [K().csa2_sparse_attn(q, kv, 4000, 1, dev_i32(idx, DEV), swa, dev_i32(st, DEV), dev_i32(sl, DEV))[0]
         for _ in range(3)]
    torch.cuda.synchronize()
    assert torch.equal(a[0], a[1]) and torch.equal(a[1], a[2])
