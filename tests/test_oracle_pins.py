"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test ties one oracle function to a library routine, a published table, a
closed form, an invariant or brute force over exact rationals, so that a slip
in the oracle (a dropped term, a wrong sign, index or operand) fails here.
CPU only.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v = line.split()
        out[k] = v
    return out


def _e4m3_torch(byte_arr):
    """E4M3 decode by torch's float8_e4m3fn (library routine)."""
    t = torch.tensor(np.asarray(byte_arr, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _e2m1_table():
    g = _golden("e2m1_ocp_values.txt")
    return np.array([float(g[str(i)]) for i in range(16)])


def _bf16(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_to_f64(u16):
    return torch.tensor(np.asarray(u16, np.uint16).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def _deq_independent(rec):
    """Dequantize records with torch's E4M3 decode and the OCP E2M1 table."""
    rec = np.asarray(rec, np.uint8).reshape(-1, 288)
    codes = rec[:, :256]
    lo, hi = codes & 15, codes >> 4
    nib = np.stack([lo, hi], -1).reshape(rec.shape[0], 512)
    sc = _e4m3_torch(rec[:, 256:].reshape(-1)).reshape(rec.shape[0], 32)
    return _e2m1_table()[nib] * np.repeat(sc, 16, axis=1)


# ---------------------------------------------------------------- formats

def test_e4m3_decode_matches_torch_all_bytes():
    ref = _e4m3_torch(np.arange(256))
    got = np.array([O.e4m3_value(b) for b in range(256)])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    m = ~np.isnan(ref)
    assert np.array_equal(ref[m], got[m])
    assert np.isnan(got).sum() == 2  # 0x7F and 0xFF only
    assert O.e4m3_value(0x7E) == 448.0 and O.e4m3_value(0x01) == 2.0 ** -9


def test_e2m1_decode_matches_ocp_table():
    tab = _e2m1_table()
    got = np.array([O.e2m1_value(i) for i in range(16)])
    assert np.array_equal(got, tab)
    assert math.copysign(1.0, got[8]) == -1.0  # code 8 is -0


def test_record_is_288_bytes_and_890_accounting():
    g = _golden("byte_accounting.txt")
    d, grp = int(g["head_dim"]), int(g["scale_group"])
    code_b = d * 4 // 8
    scale_b = d // grp  # one 8-bit E4M3 per group
    assert code_b == int(g["main_entry_code_bytes"]) and scale_b == int(g["main_entry_scale_bytes"])
    assert code_b + scale_b == int(g["main_entry_bytes"]) == O.RECORD_BYTES
    rec = O.fp4_pack(np.zeros((3, 512), np.uint16))
    assert rec.shape == (3, 288)
    per_token = float(g["entries_per_token"]) * (int(g["main_entry_bytes"]) + int(g["indexer_key_bytes_read"]))
    assert per_token == float(g["global_kv_bytes_per_token"])


def test_e4m3_encode_matches_torch_rne_in_range():
    rng = np.random.default_rng(0)
    finite = _e4m3_torch(np.arange(0x7F))  # 0 .. 448
    mids = (finite[1:] + finite[:-1]) / 2  # exact ties (representable in fp32)
    vals = np.concatenate([
        finite, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
        np.nextafter(mids.astype(np.float32), np.float32(1e9)),
        rng.uniform(0, 448, 4000), np.exp2(rng.uniform(-14, 8.8, 4000)),
    ]).astype(np.float32)
    vals = vals[vals <= 448]
    ref = torch.tensor(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([O.e4m3_encode(v) for v in vals], np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates():
    for v in [448.0, 449.0, 463.9, 464.0, 480.0, 1e6, 3.0e38, float("inf")]:
        assert O.e4m3_encode(v) == 0x7E


def _e2m1_exact(x, S):
    """Nearest E2M1 code by exact rationals: tie -> even code; above 6S -> 6S."""
    grid = [Fraction(v) for v in _e2m1_table()[:8]]
    a = abs(Fraction(x))
    S = Fraction(S)
    best, bd = None, None
    for c, v in enumerate(grid):
        d = abs(a - v * S)
        if bd is None or d < bd or (d == bd and c % 2 == 0):
            best, bd = c, d
    if best != 0 and x < 0:
        best |= 8
    return best


def test_e2m1_encode_exact_brute_force():
    rng = np.random.default_rng(1)
    scales = _e4m3_torch(np.arange(1, 0x7F))
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    cases = []
    for S in scales[::7]:
        for m in mids:  # exact ties
            cases += [(m * S, S), (-m * S, S)]
        for v in rng.normal(0, 4 * S, 20):
            cases.append((float(np.float32(v)), S))
        cases += [(7 * S, S), (-100 * S, S), (0.0, S), (-0.0, S)]
    for x, S in cases:
        assert O.e2m1_encode(x, S) == _e2m1_exact(x, S), (x, S)


# ---------------------------------------------------------------- pack / unpack

def test_unpack_exhaustive_code_scale_table():
    """All 16 codes x 254 finite scales decode to E2M1 * E4M3 exactly."""
    recs = []
    pairs = []
    for sb in range(256):
        if sb in (0x7F, 0xFF):
            continue
        for code in range(16):
            pairs.append((code, sb))
    pairs = np.array(pairs)
    n = (len(pairs) + 511) // 512
    recs = np.zeros((n, 288), np.uint8)
    expect = np.zeros((n, 512))
    tab = _e2m1_table()
    for t, (code, sb) in enumerate(pairs):
        r, c = divmod(t, 512)
        recs[r, c // 2] |= code << (4 * (c & 1))
    # one scale per 16 channels: choose pairs so each group of 16 shares a scale
    for r in range(n):
        for g in range(32):
            t0 = r * 512 + g * 16
            sb = pairs[min(t0, len(pairs) - 1)][1]
            recs[r, 256 + g] = sb
    got = O.fp4_unpack(recs)
    sc = _e4m3_torch(recs[:, 256:].reshape(-1)).reshape(n, 32)
    for t in range(len(pairs)):
        r, c = divmod(t, 512)
        code = (recs[r, c // 2] >> (4 * (c & 1))) & 15
        expect[r, c] = tab[code] * sc[r, c // 16]
    assert np.array_equal(got, expect)
    # products are exact in bf16
    assert np.array_equal(_bf16_to_f64(_bf16(got)), got)


def test_pack_scale_is_rne_of_amax_over_6():
    rng = np.random.default_rng(2)
    x = (rng.normal(0, 1, (64, 512)) * np.exp2(rng.integers(-12, 8, (64, 1)))).astype(np.float32)
    xb = _bf16(x)
    rec = O.fp4_pack(xb)
    xv = _bf16_to_f64(xb).reshape(64, 32, 16).astype(np.float32)
    amax6 = (np.abs(xv).max(-1) / np.float32(6.0)).astype(np.float32)
    ref = torch.tensor(amax6).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(rec[:, 256:], ref)


def test_pack_roundtrip_on_grid():
    """Rows already on the grid, with each group's amax = 6S, come back exactly."""
    rng = np.random.default_rng(3)
    tab = _e2m1_table()
    scales = _e4m3_torch(rng.integers(0x08, 0x7F, (16, 32)))  # normal scales
    codes = rng.integers(0, 16, (16, 32, 16))
    codes[:, :, 0] = 7  # amax = 6S in every group
    vals = tab[codes] * scales[:, :, None]
    xb = _bf16(vals.reshape(16, 512))
    assert np.array_equal(_bf16_to_f64(xb), vals.reshape(16, 512))
    back = O.fp4_unpack(O.fp4_pack(xb))
    assert np.array_equal(back, vals.reshape(16, 512))


def test_pack_error_bound_and_independent_dequant():
    rng = np.random.default_rng(4)
    x = rng.normal(0, 1, (128, 512)) * np.exp2(rng.uniform(-10, 6.5, (128, 1)))
    x[0, :16] = np.linspace(-9000, 9000, 16)  # saturated group: scale 448, values clip to +-2688
    xb = _bf16(x)
    rec = O.fp4_pack(xb)
    xv = _bf16_to_f64(xb)
    back = O.fp4_unpack(rec)
    assert np.array_equal(back, _deq_independent(rec))
    assert rec[0, 256] == 0x7E and back[0, 0] == -2688.0 and back[0, 15] == 2688.0
    xv, back = xv[:, 16:], back[:, 16:]
    S = np.repeat(_e4m3_torch(rec[:, 256:].reshape(-1)).reshape(128, 32), 16, axis=1)[:, 16:]
    # nearest-grid error is at most one grid step S (largest half gap 1*S; the
    # saturated top value loses less than S when amax/6 rounds down)
    assert np.all(np.abs(xv - back) <= S + 6 * 2.0 ** -10)
    norm = S >= 2.0 ** -6
    assert np.all(np.abs(xv - back)[norm] <= S[norm])


def test_pack_signs_zero_and_tiny_groups():
    x = np.zeros((2, 512), np.float32)
    x[0, :16] = -0.0
    x[0, 16:32] = 1e-30  # amax/6 rounds to scale 0 -> all codes 0
    x[1, :16] = np.linspace(-6, 6, 16)
    rec = O.fp4_pack(_bf16(x))
    assert np.all(rec[0] == 0)
    assert rec[1, 256] == O.e4m3_encode(1.0)
    back = O.fp4_unpack(rec)[1, :16]
    assert np.all(np.sign(back) == np.sign(np.linspace(-6, 6, 16)) * (back != 0))


# ---------------------------------------------------------------- indexer

def _rand_bf16(rng, shape, scale=1.0):
    return _bf16(rng.normal(0, scale, shape))


def test_index_score_one_hot_w_is_relu_dot():
    rng = np.random.default_rng(5)
    nq, N = 3, 200
    q = _rand_bf16(rng, (nq, 32, 128))
    k = _rand_bf16(rng, (1, N, 128))
    for h in [0, 7, 31]:
        w = np.zeros((nq, 32), np.float32)
        w[:, h] = 1.0
        s = O.index_full(q, w, k, N, q_per_seq=nq)
        ref = np.maximum(_bf16_to_f64(q)[:, h, :] @ _bf16_to_f64(k)[0].T, 0.0)
        assert np.allclose(s, ref.astype(np.float32), rtol=1e-6, atol=1e-6)


def test_index_score_linear_in_w_and_homogeneous_in_k():
    rng = np.random.default_rng(6)
    q = _rand_bf16(rng, (2, 32, 128))
    k = _rand_bf16(rng, (2, 64, 128))
    w1 = rng.uniform(0, 1, (2, 32)).astype(np.float32)
    w2 = rng.uniform(0, 1, (2, 32)).astype(np.float32)
    s1 = O.index_full(q, w1, k, 64, 1).astype(np.float64)
    s2 = O.index_full(q, w2, k, 64, 1).astype(np.float64)
    s12 = O.index_full(q, (w1 + w2).astype(np.float32), k, 64, 1).astype(np.float64)
    w12 = (w1 + w2).astype(np.float32).astype(np.float64)
    # w1+w2 rounds in float32; compare against the same rounded weights via one-hot sums
    assert np.allclose(s12, s1 + s2, rtol=1e-5)
    k2 = _bf16(_bf16_to_f64(k) * 4.0)
    s4 = O.index_full(q, w1, k2, 64, 1)
    assert np.array_equal(s4, (s1 * 4).astype(np.float32))
    # heads whose dot is negative contribute nothing: negate q -> only the other sign survives
    qn = _bf16(-_bf16_to_f64(q))
    sn = O.index_full(qn, w1, k, 64, 1).astype(np.float64)
    qd, kd = _bf16_to_f64(q), _bf16_to_f64(k)
    d = np.einsum("qhc,qnc->qhn", qd, kd)
    assert np.allclose(s1 + sn, np.einsum("qh,qhn->qn", w1.astype(np.float64), np.abs(d)), rtol=1e-5)
    assert w12.shape == (2, 32)


def test_index_visibility_and_block_max():
    rng = np.random.default_rng(7)
    nq, N = 4, 77  # ragged tail: 77 = 9 * 8 + 5
    q = _rand_bf16(rng, (nq, 32, 128))
    w = rng.uniform(0, 1, (nq, 32)).astype(np.float32)
    k = _rand_bf16(rng, (1, N, 128))
    nv = np.array([77, 40, 1, 0], np.int32)
    s, b = O.index_full(q, w, k, N, q_per_seq=nq, n_visible=nv, block_size=8)
    full = O.index_full(q, w, k, N, q_per_seq=nq)
    for r in range(nq):
        assert np.all(np.isneginf(s[r, nv[r]:]))
        assert np.array_equal(s[r, :nv[r]], full[r, :nv[r]])
        pad = np.concatenate([s[r], np.full(80 - N, -np.inf, np.float32)])
        assert np.array_equal(b[r], pad.reshape(10, 8).max(1))
    assert np.all(np.isneginf(b[3]))


def test_reindex_scores_are_full_scores_on_pool():
    rng = np.random.default_rng(8)
    nq, N = 3, 256
    q = _rand_bf16(rng, (nq, 32, 128))
    w = rng.uniform(0, 1, (nq, 32)).astype(np.float32)
    k = _rand_bf16(rng, (nq, N, 128))
    full = O.index_full(q, w, k, N, 1)
    blocks = np.sort(rng.choice(N // 8, (nq, 10), replace=True), axis=1).astype(np.int32)
    blocks[0, -1] = -1
    pool = O.pool_ids(blocks, 8)
    assert pool.shape == (nq, 80)
    assert np.array_equal(pool[1, :8], blocks[1, 0] * 8 + np.arange(8))
    ps = O.index_reindex(q, w, k, N, 1, pool)
    for r in range(nq):
        for p in range(80):
            if pool[r, p] < 0:
                assert pool[r, p] == -1 and np.isneginf(ps[r, p])
            else:
                assert ps[r, p] == full[r, pool[r, p]]


# ---------------------------------------------------------------- Top-K

def _topk_def(s, k, row_len=None):
    """Textbook definition: sort positions by (-score, position), keep k."""
    n = len(s) if row_len is None else row_len
    cand = [i for i in range(n) if not (math.isnan(s[i]) or s[i] == -math.inf)]
    cand.sort(key=lambda i: (-float(s[i]), i))
    sel = sorted(cand[:k])
    return sel + [-1] * (k - len(sel))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_topk_matches_sorted_definition(seed):
    rng = np.random.default_rng(seed)
    rows, n, k = 5, 3000, 300
    s = rng.integers(-40, 40, (rows, n)).astype(np.float32) / 4  # many ties
    s[0, ::3] = -np.inf
    s[1, ::5] = np.nan
    s[2, :100] = -0.0
    s[2, 100:200] = 0.0
    s[3, :] = 1.0  # all tied -> first k positions
    row_len = np.array([n, n, 1500, n, 17], np.int32)
    got = O.topk(s, k, row_len=row_len)
    for r in range(rows):
        assert got[r].tolist() == _topk_def(s[r], k, row_len[r])
    assert got[3].tolist() == list(range(k))
    assert got[4].tolist()[:17] == list(range(17)) and got[4, 17:].tolist() == [-1] * (k - 17)


def test_topk_id_map_and_heapq_cross_check():
    import heapq
    rng = np.random.default_rng(9)
    s = rng.normal(0, 1, (2, 5000)).astype(np.float32)
    ids = np.sort(rng.choice(10 ** 6, (2, 5000), replace=False), axis=1).astype(np.int32)
    got = O.topk(s, 512, id_map=ids)
    for r in range(2):
        best = heapq.nlargest(512, range(5000), key=lambda i: (s[r, i], -i))
        assert got[r].tolist() == sorted(ids[r, best].tolist())


def test_topk_all_invisible_gives_padding():
    s = np.full((1, 100), -np.inf, np.float32)
    assert O.topk(s, 8).tolist() == [[-1] * 8]


# ---------------------------------------------------------------- hierarchical pool

def _hier(q, w, k, N, nb_keep, kk=512):
    s, b = O.index_full(q, w, k, N, 1, block_size=8)
    top = O.topk(s, kk)
    blocks = O.topk(b, nb_keep)
    pool = O.pool_ids(blocks, 8)
    return s, top, blocks, pool


def test_pool_contains_full_topk_and_reindex_reproduces_it():
    """Every block ranked above block b holds an entry ranked above all of b's
    entries, so a Full Top-K entry lives in one of the top-K blocks; scoring the
    pool with the Full layer's own (q, w) must return the Full Top-K."""
    rng = np.random.default_rng(10)
    nq, N = 2, 8192
    q = _rand_bf16(rng, (nq, 32, 128))
    w = rng.uniform(0, 1, (nq, 32)).astype(np.float32)
    k = _rand_bf16(rng, (nq, N, 128))
    s, top, blocks, pool = _hier(q, w, k, N, nb_keep=64, kk=64)
    for r in range(nq):
        assert set(top[r].tolist()) <= set(pool[r].tolist())
    ps = O.index_reindex(q, w, k, N, 1, pool)
    re = O.topk(ps, 64, id_map=pool)
    assert np.array_equal(re, top)


def test_pool_invariant_with_ties():
    rng = np.random.default_rng(11)
    N = 4096
    s = (rng.integers(0, 20, (3, N)) / 2).astype(np.float32)
    b = s.reshape(3, -1, 8).max(-1)
    top = O.topk(s, 100)
    blocks = O.topk(b, 100)
    pool = O.pool_ids(blocks, 8)
    for r in range(3):
        assert set(top[r].tolist()) <= set(pool[r].tolist())


# ---------------------------------------------------------------- attention

def _attn_inputs(rng, nq=2, N=300, k=40, T=128, slen=128):
    q = _rand_bf16(rng, (nq, 64, 512))
    kv = np.concatenate([rng.integers(0, 256, (nq * N, 256)),
                         torch.tensor(np.exp2(rng.uniform(-4, 0, (nq * N, 32))).astype(np.float32))
                         .to(torch.float8_e4m3fn).view(torch.uint8).numpy()], axis=1).astype(np.uint8)
    idx = np.sort(np.stack([rng.choice(N, k, replace=False) for _ in range(nq)]), axis=1).astype(np.int32)
    swa = _rand_bf16(rng, (nq, T, 512))
    st = np.zeros(nq, np.int32)
    sl = np.full(nq, slen, np.int32)
    return q, kv.reshape(nq, N, 288), idx, swa, st, sl


def _sdpa_ref(qv, keys, scale):
    """torch scaled_dot_product_attention in float64 on CPU (library routine)."""
    qt = torch.tensor(qv)[None]  # [1,64,512]
    kt = torch.tensor(keys)[None]  # [1,n,512]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=scale)
    l = torch.logsumexp(scale * (qt @ kt.transpose(-1, -2)), dim=-1)
    return o[0].numpy(), l[0].numpy()


def test_attention_matches_sdpa_on_gathered_keys():
    rng = np.random.default_rng(12)
    q, kv, idx, swa, st, sl = _attn_inputs(rng)
    idx[1, 5] = -1  # skipped slot
    sc = 1 / math.sqrt(512)
    out, lse = O.sparse_attn(q, kv, 300, 1, idx, swa, 128, st, sl, sc)
    for r in range(2):
        ids = [i for i in idx[r] if i >= 0]
        keys = np.concatenate([_deq_independent(kv[r, ids]), _bf16_to_f64(swa[r])], 0)
        ro, rl = _sdpa_ref(_bf16_to_f64(q[r]), keys, sc)
        assert np.allclose(out[r], ro, rtol=1e-9, atol=1e-12)
        assert np.allclose(lse[r], rl, rtol=1e-12)


def test_attention_swa_only_and_dense_masked_equivalence():
    rng = np.random.default_rng(13)
    q, kv, idx, swa, st, sl = _attn_inputs(rng, nq=1, N=64, k=16, T=160, slen=100)
    st[:] = 37
    sc = 1 / math.sqrt(512)
    none = np.full_like(idx, -1)
    out, lse = O.sparse_attn(q, kv, 64, 1, none, swa, 160, st, sl, sc)
    ro, rl = _sdpa_ref(_bf16_to_f64(q[0]), _bf16_to_f64(swa[0, 37:137]), sc)
    assert np.allclose(out[0], ro, rtol=1e-9, atol=1e-12) and np.allclose(lse[0], rl)
    # dense attention over all 64 entries + window with unselected entries masked
    out2, _ = O.sparse_attn(q, kv, 64, 1, idx, swa, 160, st, sl, sc)
    allk = np.concatenate([_deq_independent(kv[0]), _bf16_to_f64(swa[0, 37:137])], 0)
    mask = np.zeros(64 + 100, bool)
    mask[idx[0]] = True
    mask[64:] = True
    qt = torch.tensor(_bf16_to_f64(q[0]))[None]
    kt = torch.tensor(allk)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, attn_mask=torch.tensor(mask)[None, None],
                                                           scale=sc)[0].numpy()
    assert np.allclose(out2[0], ref, rtol=1e-9, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(14)
    q, kv, idx, swa, st, sl = _attn_inputs(rng, nq=1, N=50, k=10, slen=20)
    sc = 1 / math.sqrt(512)
    # Q = 0 -> plain mean of the 30 value rows
    qz = np.zeros_like(q)
    out, lse = O.sparse_attn(qz, kv, 50, 1, idx, swa, 128, st, sl, sc)
    keys = np.concatenate([_deq_independent(kv[0, idx[0]]), _bf16_to_f64(swa[0, :20])], 0)
    assert np.allclose(out[0], keys.mean(0)[None, :].repeat(64, 0), rtol=1e-12, atol=1e-14)
    assert np.allclose(lse[0], math.log(30))
    # permuting the index list leaves the output unchanged (up to rounding)
    out1, _ = O.sparse_attn(q, kv, 50, 1, idx, swa, 128, st, sl, sc)
    out2, _ = O.sparse_attn(q, kv, 50, 1, idx[:, ::-1].copy(), swa, 128, st, sl, sc)
    assert np.allclose(out1, out2, rtol=1e-10, atol=1e-13)
    # all keys identical -> output is that row
    kv_same = np.repeat(kv[:, :1], 50, axis=1)
    out3, _ = O.sparse_attn(q, kv_same, 50, 1, idx, swa, 128, st, np.zeros(1, np.int32), sc)
    row = _deq_independent(kv_same[0, 0])[0]
    assert np.allclose(out3[0], row[None].repeat(64, 0), rtol=1e-12, atol=1e-14)
    # no keys at all -> zeros and -inf
    out4, lse4 = O.sparse_attn(q, kv, 50, 1, np.full_like(idx, -1), swa, 128, st, np.zeros(1, np.int32), sc)
    assert np.all(out4 == 0) and np.all(np.isneginf(lse4))


# ---------------------------------------------------------------- planted structure

def test_planted_entries_are_recalled():
    from kv_cache_compression_csa2_amd.workloads import make_workload
    wl = make_workload("encoder64k", device="cpu", nq=4, N=4096)
    s = O.index_full(wl.q_idx[0].view(torch.int16).numpy().view(np.uint16), wl.w[0].numpy(),
                     wl.k_idx.view(torch.int16).numpy().view(np.uint16), wl.N, wl.q_per_seq)
    top = O.topk(s, 512)
    for r in range(4):
        assert set(wl.planted[r].tolist()) <= set(top[r].tolist())


# ------------------------------------------------------ FP4 indexer K (NEXT row)

def _mx_exp(amax, emax):
    """OCP MX shared exponent of a block: floor(log2 amax) - emax, emax being
    the exponent of the element type's largest power of two (2 for E2M1, 8 for
    E4M3), clamped to the E8M0 range; -127 for an all-zero block."""
    if amax == 0:
        return -127
    m, e = math.frexp(amax)  # amax = m * 2^e, 0.5 <= m < 1
    return min(max(e - 1 - emax, -127), 127)


def _kidx_deq_independent(rec):
    """Decode FP4 indexer-K entries (OCP MXFP4) with the OCP E2M1 table and
    the E8M0 scale 2^(b - 127) of each 32-channel block."""
    rec = np.asarray(rec, np.uint8).reshape(-1, 68)
    codes = rec[:, :64]
    nib = np.stack([codes & 15, codes >> 4], -1).reshape(rec.shape[0], 128)
    sb = rec[:, 64:68].astype(np.float64)
    sc = np.where(sb == 255, np.nan, np.exp2(sb - 127))
    return _e2m1_table()[nib] * np.repeat(sc, 32, axis=1)


def _nearest_grid_code(x, s):
    """Brute force over the 8 magnitudes: nearest v*s to |x| (exact in float64
    for a power-of-two s), ties to the even code, +0 for magnitude 0; past 6s
    the nearest is 6s, i.e. saturation."""
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64) * s
    d = np.abs(np.abs(x) - mags)
    best = 0
    for c in range(8):
        if d[c] < d[best] or (d[c] == d[best] and c % 2 == 0 and best % 2 == 1):
            best = c
    if best and x < 0:
        best |= 8
    return best


def _nibbles(rec_row):
    return np.stack([rec_row[:64] & 15, rec_row[:64] >> 4], -1).reshape(128)


def test_kidx_fp4_entry_layout_matches_68_byte_accounting():
    g = _golden("byte_accounting.txt")
    assert O.KIDX_RECORD_BYTES == int(g["indexer_key_bytes_read"]) == 128 // 2 + 128 // 32
    x = np.zeros((2, 128), np.float32)
    x[0, :6] = [6, -6, 3, 0.5, 0, -1.25]  # block 0: amax 6 -> X = 2^(2-2) = 1; -1.25 is a tie -> 1 (even code 2)
    x[0, 32:36] = [7, 5, 3.5, -0.25]      # block 1: amax 7 -> X = 1; 7 saturates to 6, ties 5 -> 4, 3.5 -> 4, -0.25 -> +0
    x[1, 127] = -0.75 * 2.0 ** -20        # block 3: X = 2^(-21-2); the value is -6 X
    rec = O.kidx_fp4_pack(_bf16(x))
    assert rec.shape == (2, 68)
    assert list(rec[0, :3]) == [0xF7, 0x15, 0xA0] and not rec[0, 3:16].any()
    assert list(rec[0, 16:18]) == [0x67, 0x06] and not rec[0, 18:64].any()
    assert list(rec[0, 64:]) == [127, 127, 0, 0]  # all-zero blocks take 2^-127
    assert rec[1, 63] == (0x8 | 7) << 4 and not rec[1, :63].any()
    assert list(rec[1, 64:]) == [0, 0, 0, 104]


def test_kidx_fp4_codes_brute_force_and_scale_rule():
    rng = np.random.default_rng(21)
    rows = np.concatenate([rng.normal(0, 1, (40, 128)), rng.normal(0, 1, (20, 128)) * np.exp2(
        rng.integers(-30, 30, (20, 1))), rng.uniform(-8, 8, (10, 128)),
        rng.normal(0, 1, (10, 128)) * np.exp2(rng.integers(-40, 40, (10, 128)))]).astype(np.float32)
    rows[-1, :32] = 0.0          # an all-zero block
    rows[-2, 32:64] = 1e-38      # a tiny block: the exponent clamps at -127
    xb = _bf16(rows)
    xf = _bf16_to_f64(xb)
    rec = O.kidx_fp4_pack(xb)
    for r in range(rows.shape[0]):
        nib = _nibbles(rec[r])
        for g in range(4):
            blk = xf[r, 32 * g:32 * g + 32]
            e = _mx_exp(np.abs(blk).max(), 2)
            assert rec[r, 64 + g] == e + 127, (r, g)
            want = [_nearest_grid_code(v, 2.0 ** e) for v in blk]
            assert list(nib[32 * g:32 * g + 32]) == want, (r, g)


def test_kidx_fp4_unpack_is_table_times_scale_and_ties_go_even():
    rng = np.random.default_rng(22)
    rec = rng.integers(0, 256, (40, 68)).astype(np.uint8)
    assert np.array_equal(O.kidx_fp4_unpack(rec), _kidx_deq_independent(rec), equal_nan=True)
    xb = _rand_bf16(rng, (64, 128), 3.0)
    rec = O.kidx_fp4_pack(xb)
    assert np.array_equal(O.kidx_fp4_unpack(rec), _kidx_deq_independent(rec))
    # every midpoint between neighbours of the grid, times scale 1 (block amax 6)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    even = np.array([0, 2, 2, 4, 4, 6, 6])  # the even neighbour's code
    x = np.zeros((1, 128), np.float32)
    x[0, 0] = 6.0
    x[0, 1:8] = mids
    x[0, 8:15] = -mids
    rec = O.kidx_fp4_pack(_bf16(x))
    nib = _nibbles(rec[0])
    assert list(nib[1:8]) == list(even)
    assert list(nib[8:15]) == [c | 8 if c else 0 for c in even]
    # an all-zero row: zero codes, every block scale 2^-127 (byte 0)
    assert not O.kidx_fp4_pack(np.zeros((1, 128), np.uint16)).any()


def test_kidx_fp4_round_trip_error_bound_and_saturation():
    rng = np.random.default_rng(25)
    xb = _rand_bf16(rng, (48, 128), 2.0)
    xf = _bf16_to_f64(xb)
    rt = O.kidx_fp4_unpack(O.kidx_fp4_pack(xb))
    for r in range(48):
        for g in range(4):
            blk, got = xf[r, 32 * g:32 * g + 32], rt[r, 32 * g:32 * g + 32]
            X = 2.0 ** _mx_exp(np.abs(blk).max(), 2)
            sat = np.abs(blk) > 6 * X
            assert np.all(got[sat] == np.sign(blk[sat]) * 6 * X)
            err = np.abs(got[~sat] - blk[~sat])
            # half the grid spacing: X/4 below 2X, |x|/4 above
            assert np.all(err <= np.maximum(np.abs(blk[~sat]) / 4, X / 4))


def test_kidx_fp4_pack_is_scale_equivariant():
    rng = np.random.default_rng(23)
    xb = _rand_bf16(rng, (32, 128))
    rec = O.kidx_fp4_pack(xb)
    for m in (-7, 5):
        rec2 = O.kidx_fp4_pack(_bf16(_bf16_to_f64(xb) * 2.0 ** m))
        assert np.array_equal(rec2[:, :64], rec[:, :64])
        assert np.array_equal(rec2[:, 64:].astype(int), rec[:, 64:].astype(int) + m)


def test_index_fp4k_is_the_score_formula_on_decoded_keys():
    rng = np.random.default_rng(24)
    nq, N = 3, 150
    q = _rand_bf16(rng, (nq, 32, 128))
    w = rng.uniform(0, 1, (nq, 32)).astype(np.float32)
    kf = O.kidx_fp4_pack(_rand_bf16(rng, (nq * N, 128))).reshape(nq, N, 68)
    nv = np.array([150, 61, 0], np.int32)
    s, b = O.index_full(q, w, None, N, 1, n_visible=nv, block_size=8, k_fp4=kf)
    kd = _kidx_deq_independent(kf.reshape(-1, 68)).reshape(nq, N, 128)
    d = np.einsum("qhc,qnc->qhn", _bf16_to_f64(q), kd)
    ref = np.einsum("qh,qhn->qn", w.astype(np.float64), np.maximum(d, 0.0))
    for r in range(nq):
        assert np.allclose(s[r, :nv[r]], ref[r, :nv[r]], rtol=1e-6, atol=1e-6)
        assert np.all(np.isneginf(s[r, nv[r]:]))
    pad = np.concatenate([s[0], np.full(152 - N, -np.inf, np.float32)])
    assert np.array_equal(b[0], pad.reshape(19, 8).max(1))
    # Reindex over a pool scores the same entries identically
    pool = np.stack([np.arange(0, 2048, 8) % N for _ in range(nq)]).astype(np.int32)
    pool[1, 5] = -1
    ps = O.index_reindex(q, w, None, N, 1, pool, n_visible=nv, k_fp4=kf)
    for r in range(nq):
        for j in range(pool.shape[1]):
            i = pool[r, j]
            exp = s[r, i] if i >= 0 else -np.inf
            assert ps[r, j] == exp or (np.isneginf(ps[r, j]) and np.isneginf(exp))


def test_index_fp4qk_is_the_score_formula_on_decoded_query_and_keys():
    """MXFP4 indexer Q and K (eogee.com report 3.4: the indexer Q/K ran in FP4):
    the score is the formula on the decoded values of both, each decoded here
    with the OCP table independently of the oracle."""
    rng = np.random.default_rng(25)
    nq, N = 4, 133
    qf = O.kidx_fp4_pack(_rand_bf16(rng, (nq * 32, 128))).reshape(nq, 32, 68)
    w = rng.uniform(0, 1, (nq, 32)).astype(np.float32)
    w[1, 3] = -0.5  # a negative weight: w * ReLU, not ReLU(w * .)
    kf = O.kidx_fp4_pack(_rand_bf16(rng, (2 * N, 128))).reshape(2, N, 68)
    nv = np.array([133, 70, 0, 9], np.int32)
    s, b = O.index_full(None, w, None, N, 2, n_visible=nv, block_size=8, k_fp4=kf, q_fp4=qf)
    qd = _kidx_deq_independent(qf.reshape(-1, 68)).reshape(nq, 32, 128)
    kd = _kidx_deq_independent(kf.reshape(-1, 68)).reshape(2, N, 128)
    d = np.einsum("qhc,qnc->qhn", qd, kd[np.arange(nq) // 2])  # query q reads sequence q // 2
    ref = np.einsum("qh,qhn->qn", w.astype(np.float64), np.maximum(d, 0.0))
    for r in range(nq):
        assert np.allclose(s[r, :nv[r]], ref[r, :nv[r]], rtol=1e-6, atol=1e-6)
        assert np.all(np.isneginf(s[r, nv[r]:]))
    pad = np.concatenate([s[0], np.full(136 - N, -np.inf, np.float32)])
    assert np.array_equal(b[0], pad.reshape(17, 8).max(1))
    # a query already on the MXFP4 grid packs losslessly, so its FP4 entries
    # score exactly like the bf16 query through the bf16-Q scorer
    qg = _bf16(qd.reshape(nq, 32, 128))
    assert np.array_equal(O.kidx_fp4_pack(qg.reshape(-1, 128)), qf.reshape(-1, 68))
    s_bf = O.index_full(qg, w, None, N, 2, n_visible=nv, k_fp4=kf)
    assert np.array_equal(O.index_full(None, w, None, N, 2, n_visible=nv, k_fp4=kf, q_fp4=qf), s_bf)
    # Reindex with the MXFP4 query: the independent numpy scores at the pool's
    # positions (-inf for padding and invisible ones), queries of sequence q // 2
    pool = np.stack([(np.arange(0, 160) * 7 + 3 * r) % N for r in range(nq)]).astype(np.int32)
    pool[2, 4] = -1
    ps = O.index_reindex(None, w, None, N, 2, pool, n_visible=nv, k_fp4=kf, q_fp4=qf)
    for r in range(nq):
        for j in range(pool.shape[1]):
            i = pool[r, j]
            if i < 0 or i >= nv[r]:
                assert np.isneginf(ps[r, j])
            else:
                assert abs(ps[r, j] - ref[r, i]) <= 1e-6 * max(1.0, abs(ref[r, i]))


# ------------------------------------------------------- FP8 window rows

def _ocp_mx_exp(amax):
    """OCP MX shared exponent for E4M3 elements (largest power of two 2^8)."""
    return _mx_exp(amax, 8)


def _swa_deq_independent(rec):
    """Dequantize FP8 window rows with torch's E4M3 decode times 2^(b - 127)."""
    rec = np.asarray(rec, np.uint8).reshape(-1, 528)
    el = _e4m3_torch(rec[:, :512].reshape(-1)).reshape(rec.shape[0], 512)
    sb = rec[:, 512:].astype(np.float64)
    sc = np.where(sb == 255, np.nan, np.exp2(sb - 127))
    return el * np.repeat(sc, 32, axis=1)


def test_swa_fp8_row_layout_and_ocp_scale_rule():
    x = np.zeros((1, 512), np.float32)
    x[0, 0:3] = [1.0, 0.5, -0.25]          # amax 1 -> X = 2^-8: codes of 256, 128, -64
    x[0, 32] = 3.90625                      # amax in [2, 4): X = 2^-7, 500 saturates to 448
    x[0, 96] = 2.0 ** -130                  # tiny amax: exponent clamps to -127, 2^-3 remains
    x[0, 128] = 2.0 ** 120                  # X = 2^112, element 256
    rec = O.swa_fp8_pack(_bf16(x))
    assert rec.shape == (1, 528) and O.SWA_RECORD_BYTES == 528 == 512 + 512 // 32
    assert list(rec[0, :3]) == [0x78, 0x70, 0xE8] and not rec[0, 3:32].any()
    assert rec[0, 32] == 0x7E
    assert rec[0, 96] == 0x20 and rec[0, 128] == 0x78
    assert list(rec[0, 512:517]) == [119, 120, 0, 0, 239]  # block 2 is all zero
    xf = _bf16_to_f64(_bf16(x))[0]
    for g in range(16):
        assert rec[0, 512 + g] == _ocp_mx_exp(np.abs(xf[32 * g:32 * g + 32]).max()) + 127


def test_swa_fp8_codes_match_torch_rne_and_saturate():
    rng = np.random.default_rng(31)
    rows = np.concatenate([rng.normal(0, 1, (24, 512)), rng.normal(0, 1, (16, 512)) * np.exp2(
        rng.integers(-40, 40, (16, 1))), rng.uniform(-1, 1, (8, 512)) * 3.99]).astype(np.float32)
    xb = _bf16(rows)
    xf = _bf16_to_f64(xb)
    rec = O.swa_fp8_pack(xb)
    for r in range(rows.shape[0]):
        for g in range(16):
            blk = xf[r, 32 * g:32 * g + 32]
            e = _ocp_mx_exp(np.abs(blk).max())
            assert rec[r, 512 + g] == e + 127
            v = blk * 2.0 ** -e
            codes = rec[r, 32 * g:32 * g + 32]
            fin = np.abs(v) <= 448.0
            # in range: torch's round-to-nearest-even cast (sign of a zero result is +)
            t = torch.tensor(np.abs(v[fin]).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            want = np.where((v[fin] < 0) & (t != 0), t | 0x80, t)
            assert np.array_equal(codes[fin], want), (r, g)
            # past 448: saturation to +-448
            assert np.all((codes[~fin] & 0x7F) == 0x7E)
            assert np.all((codes[~fin] >> 7) == (v[~fin] < 0))


def test_swa_fp8_unpack_is_table_times_scale_and_error_bound():
    rng = np.random.default_rng(32)
    rec = rng.integers(0, 256, (40, 528)).astype(np.uint8)
    assert np.array_equal(O.swa_fp8_unpack(rec), _swa_deq_independent(rec), equal_nan=True)
    # round trip: error <= 2^-4 |x| (normal elements) or half the subnormal step,
    # except saturated elements, which decode to +-448 X
    xb = _rand_bf16(rng, (32, 512), 2.0)
    xf = _bf16_to_f64(xb)
    rt = O.swa_fp8_unpack(O.swa_fp8_pack(xb))
    for r in range(32):
        for g in range(16):
            blk, got = xf[r, 32 * g:32 * g + 32], rt[r, 32 * g:32 * g + 32]
            X = 2.0 ** _ocp_mx_exp(np.abs(blk).max())
            sat = np.abs(blk) > 448 * X
            assert np.all(got[sat] == np.sign(blk[sat]) * 448 * X)
            err = np.abs(got[~sat] - blk[~sat])
            assert np.all(err <= np.maximum(np.abs(blk[~sat]) * 2.0 ** -4, X * 2.0 ** -10))


def test_attention_fp8_window_is_attention_on_the_decoded_rows():
    rng = np.random.default_rng(33)
    nq, N, k, T = 3, 200, 40, 140
    q = _rand_bf16(rng, (nq, 64, 512))
    kv = O.fp4_pack(_rand_bf16(rng, (nq * N, 512))).reshape(nq, N, 288)
    idx = np.sort(np.stack([rng.choice(N, k, replace=False) for _ in range(nq)]), 1).astype(np.int32)
    idx[1, -5:] = -1
    swa = _rand_bf16(rng, (nq, T, 512), 1.5)
    wrec = O.swa_fp8_pack(swa.reshape(-1, 512)).reshape(nq, T, 528)
    st = np.array([0, 3, 12], np.int32)
    sl = np.array([128, 0, 100], np.int32)
    o8, l8 = O.sparse_attn(q, kv, N, 1, idx, None, T, st, sl, swa_fp8=wrec)
    # the decoded rows are bf16 values (4 significant bits times a power of two)
    dec = O.swa_fp8_unpack(wrec.reshape(-1, 528)).reshape(nq, T, 512)
    db = _bf16(dec)
    assert np.array_equal(_bf16_to_f64(db), dec)
    ob, lb = O.sparse_attn(q, kv, N, 1, idx, db, T, st, sl)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)
