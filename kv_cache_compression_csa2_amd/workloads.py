"""Seeded synthetic inputs for the CSA2 hot path.

This module only draws random tensors of the shapes and distributions of the
five workloads below; it does none of the path's arithmetic (no scoring, no
selection, no packing, no attention). The GPU library and the CPU oracle both
read what it produces. Main-KV entries that must hold a chosen value (the
planted entries of the 64K workload, every entry of the 1M workload) are
produced as bf16 rows *before* packing; each side packs them with its own
packer.

Workloads (sizes from the pages: 32-head x 128-dim indexer, Top-512, 2048 x 8
candidate pool, 64-head x 512-dim MQA, 128-token sliding window, m=2 encoder /
m=1 decoder compression -- eogee.com report 3.2-3.4, nxbn.cn walkthrough 3.3):

  tiny         1 query, 1024 entries, Full mode.
  encoder64k   64 queries, 64K tokens at m=2 -> 32768 entries per sequence,
               Full mode, 8 planted high-similarity entries per query.
  decoder256k  32 queries, 262144 entries (m=1); Full + 3 Reindex + 1 Reuse.
  prefill128k  4096 queries on one sequence (the last 4096 positions of a
               131072-token context), 65536 entries at m=2, causal visibility.
  decode1m     8 queries, 1048576 entries (m=1), clustered keys (16 centroids,
               sigma 0.3); Full + 3 Reindex + 1 Reuse.

With the pages' storage precision for the indexer K (FP4, 68 B per entry),
packed from the same bf16 keys on the GPU before timing:

  encoder64k_fp4k    the 64K shapes.
  decode1m_fp4k      the 1M shapes, Full + 3 Reindex + 1 Reuse.

With both of the pages' cache precisions (FP4 indexer K and FP8 window KV,
528 B per row, packed from the same kind of bf16 rows on the GPU before
timing):

  encoder64k_fp4k_fp8w, decode1m_fp4k_fp8w.

The prefill chunk with the indexer K in FP4 (prefill128k_fp4k), and with the
indexer Q in FP4 as well (prefill128k_fp4qk; eogee.com report 3.4: the
predecessor already trained the indexer Q/K in FP4): the step itself packs
the Full layer's bf16 query into one MXFP4 entry per head before scoring.
The 64K and 1M decode steps at all of these precisions (MXFP4 indexer Q and K,
FP8 window KV; each scoring layer's query packed inside the step):

  encoder64k_fp4qk_fp8w, decode1m_fp4qk_fp8w.

Layer groups that share one cache (eogee.com report 3.2: an encoder cache
serves a Full layer and the Reuse layers after it; a decoder cache serves a
Reindex layer and Reuse layers), timed as layer sequences:

  encoder_group64k   the 64K shapes; Full + 5 Reuse (6 attention layers on
                     one Top-512).
  decoder_group256k  the 256K shapes; a Full layer builds the 2048-block pool
                     once (set-up, untimed), then Reindex + 3 Reuse (4
                     attention layers on the Reindex layer's Top-512).
"""
import math
from dataclasses import dataclass, field

import torch

IDX_HEADS, IDX_DIM, HEADS, DIM, RECORD = 32, 128, 64, 512, 288
TOPK, POOL_BLOCKS, BLOCK = 512, 2048, 8
WINDOW = 128

CONFIGS = {
    "tiny": dict(nq=1, N=1024, q_per_seq=1, hier=False, seed=0, kv="random", kidx="normal", planted=0,
                 prefill=False),
    "encoder64k": dict(nq=64, N=32768, q_per_seq=1, hier=False, seed=1, kv="random", kidx="normal", planted=8,
                       prefill=False),
    "decoder256k": dict(nq=32, N=262144, q_per_seq=1, hier=True, seed=2, kv="random", kidx="normal", planted=0,
                        prefill=False),
    "prefill128k": dict(nq=4096, N=65536, q_per_seq=4096, hier=False, seed=3, kv="random", kidx="normal",
                        planted=0, prefill=True),
    "decode1m": dict(nq=8, N=1048576, q_per_seq=1, hier=True, seed=4, kv="clustered", kidx="clustered", planted=0,
                     prefill=False),
    "encoder_group64k": dict(nq=64, N=32768, q_per_seq=1, hier=False, seed=5, kv="random", kidx="normal",
                             planted=8, prefill=False, group="encoder"),
    "decoder_group256k": dict(nq=32, N=262144, q_per_seq=1, hier=True, seed=6, kv="random", kidx="normal",
                              planted=0, prefill=False, group="decoder"),
    "encoder64k_fp4k": dict(nq=64, N=32768, q_per_seq=1, hier=False, seed=7, kv="random", kidx="normal",
                            planted=8, prefill=False, kfmt="fp4"),
    "decode1m_fp4k": dict(nq=8, N=1048576, q_per_seq=1, hier=True, seed=8, kv="clustered", kidx="clustered",
                          planted=0, prefill=False, kfmt="fp4"),
    "encoder64k_fp4k_fp8w": dict(nq=64, N=32768, q_per_seq=1, hier=False, seed=9, kv="random", kidx="normal",
                                 planted=8, prefill=False, kfmt="fp4", swa_fmt="fp8"),
    "decode1m_fp4k_fp8w": dict(nq=8, N=1048576, q_per_seq=1, hier=True, seed=10, kv="clustered", kidx="clustered",
                               planted=0, prefill=False, kfmt="fp4", swa_fmt="fp8"),
    "encoder64k_fp4qk_fp8w": dict(nq=64, N=32768, q_per_seq=1, hier=False, seed=13, kv="random", kidx="normal",
                                  planted=8, prefill=False, kfmt="fp4", swa_fmt="fp8", qfmt="fp4"),
    "decode1m_fp4qk_fp8w": dict(nq=8, N=1048576, q_per_seq=1, hier=True, seed=14, kv="clustered", kidx="clustered",
                                planted=0, prefill=False, kfmt="fp4", swa_fmt="fp8", qfmt="fp4"),
    "prefill128k_fp4k": dict(nq=4096, N=65536, q_per_seq=4096, hier=False, seed=11, kv="random", kidx="normal",
                             planted=0, prefill=True, kfmt="fp4"),
    "prefill128k_fp4qk": dict(nq=4096, N=65536, q_per_seq=4096, hier=False, seed=12, kv="random", kidx="normal",
                              planted=0, prefill=True, kfmt="fp4", qfmt="fp4"),
}

# Norm given to a planted main-KV row before packing: about twice the RMS norm
# of a random entry (uniform E2M1 codes times scales 2^U[-4,0] over 512 channels).
PLANT_V_NORM = 56.0
PLANT_K_GAIN = 4.0  # planted indexer key = 4 * sqrt(128) * unit direction + 0.1 noise
CLUSTERS, CLUSTER_SIGMA = 16, 0.3
PREFILL_CONTEXT, PREFILL_M = 131072, 2


def generator(device, seed, stream):
    """Independent reproducible stream `stream` of workload seed `seed`."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + int(stream))
    return g


def bf16_normal(shape, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def random_scale_bytes(shape, g, device):
    """E4M3 scale bytes of 2^u, u ~ U[-4, 0] (torch's float8_e4m3fn cast rounds)."""
    u = torch.rand(shape, generator=g, device=device, dtype=torch.float32) * -4.0
    return torch.exp2(u).to(torch.float8_e4m3fn).view(torch.uint8)


def random_records(n_rows, g, device):
    """Main-KV records with uniformly random E2M1 codes and random scales."""
    codes = torch.randint(0, 256, (n_rows, DIM // 2), generator=g, device=device, dtype=torch.uint8)
    scales = random_scale_bytes((n_rows, DIM // 16), g, device)
    return torch.cat([codes, scales], dim=1).contiguous()


@dataclass
class Workload:
    name: str
    nq: int
    N: int
    q_per_seq: int
    nseq: int
    hier: bool
    swa_T: int
    group: str = None  # None, "encoder" (Full + 5 Reuse) or "decoder" (Reindex + 3 Reuse)
    kfmt: str = "bf16"  # indexer-K cache precision the step reads: "bf16" or "fp4" (68 B entries)
    swa_fmt: str = "bf16"  # window-KV precision the step reads: "bf16" or "fp8" (528 B rows)
    qfmt: str = "bf16"  # indexer-Q precision: "bf16", or "fp4" (the step packs each layer's MXFP4 entries per head)
    q_idx: list = field(default_factory=list)  # per indexer layer: bf16 [nq,32,128]
    w: list = field(default_factory=list)  # per indexer layer: f32 [nq,32]
    k_idx: torch.Tensor = None  # bf16 [nseq,N,128]
    kv: torch.Tensor = None  # u8 [nseq,N,288]; None where every row comes from kv_prepack
    kv_prepack_rows: torch.Tensor = None  # i64 [P] flat row ids (seq*N + i) to overwrite after packing
    kv_prepack: torch.Tensor = None  # bf16 [P,512] rows to pack into those ids
    q: list = field(default_factory=list)  # per attention layer: bf16 [nq,64,512]
    swa: list = field(default_factory=list)  # per attention layer: bf16 [nseq,T,512]
    swa_start: torch.Tensor = None  # i32 [nq]
    swa_len: torch.Tensor = None  # i32 [nq]
    n_visible: torch.Tensor = None  # i32 [nq] or None (= N)
    planted: torch.Tensor = None  # i64 [nq, P] planted entry positions or None
    clustered_seed: int = None  # decode1m: main KV rows come from clustered_kv_rows()

    @property
    def n_index_layers(self):
        """Scoring layers: the Full layer, then Reindex layers."""
        if self.group == "decoder":
            return 2
        return 4 if self.hier else 1

    @property
    def reindex_layers(self):
        return list(range(1, self.n_index_layers))

    @property
    def attn_src(self):
        """For each attention layer, the scoring layer whose Top-512 it uses
        (a Reuse layer repeats the previous layer's)."""
        if self.group == "encoder":
            return [0] * 6
        if self.group == "decoder":
            return [1] * 4
        return [0, 1, 2, 3, 3] if self.hier else [0]

    @property
    def n_attn_layers(self):
        return len(self.attn_src)


def clustered_kv_rows(seed, seq, N, device, row0=0, nrows=None):
    """bf16 pre-pack main-KV rows [nrows,512] of one clustered sequence.

    Row i belongs to cluster z_i (shared with the indexer keys) and equals
    c_z + 0.3 * noise. Rows are produced in slabs of 65536 so any sub-range can
    be regenerated on its own.
    """
    nrows = N - row0 if nrows is None else nrows
    cent = bf16_normal((CLUSTERS, DIM), generator(device, seed, 9000), device).float()
    z = torch.randint(0, CLUSTERS, (N,), generator=generator(device, seed, 8000 + seq), device=device)
    out = []
    SLAB = 65536
    for s0 in range((row0 // SLAB) * SLAB, row0 + nrows, SLAB):
        s1 = min(s0 + SLAB, N)
        noise = torch.randn((s1 - s0, DIM), generator=generator(device, seed, 100000 + seq * 1024 + s0 // SLAB),
                            device=device)
        rows = (cent[z[s0:s1]] + CLUSTER_SIGMA * noise).to(torch.bfloat16)
        a, b = max(row0, s0), min(row0 + nrows, s1)
        out.append(rows[a - s0:b - s0])
    return torch.cat(out, 0)


def make_workload(name, device="cpu", seed=None, nq=None, N=None):
    """Draw all inputs of workload `name` on `device` (optionally resized)."""
    c = dict(CONFIGS[name])
    seed = c["seed"] if seed is None else seed
    nq = c["nq"] if nq is None else nq
    N = c["N"] if N is None else N
    q_per_seq = nq if c["prefill"] else c["q_per_seq"]
    nseq = nq // q_per_seq
    swa_T = (nq + WINDOW - 1) if c["prefill"] else WINDOW
    wl = Workload(name, nq, N, q_per_seq, nseq, c["hier"], swa_T, c.get("group"), c.get("kfmt", "bf16"),
                  c.get("swa_fmt", "bf16"), c.get("qfmt", "bf16"))
    s = 0

    def nxt():
        nonlocal s
        s += 1
        return generator(device, seed, s)

    for _ in range(wl.n_index_layers):
        wl.q_idx.append(bf16_normal((nq, IDX_HEADS, IDX_DIM), nxt(), device))
        wl.w.append(torch.rand((nq, IDX_HEADS), generator=nxt(), device=device, dtype=torch.float32))
    for _ in range(wl.n_attn_layers):
        wl.q.append(bf16_normal((nq, HEADS, DIM), nxt(), device))
        wl.swa.append(bf16_normal((nseq, swa_T, DIM), nxt(), device))

    if c["kidx"] == "clustered":
        cent = bf16_normal((CLUSTERS, IDX_DIM), generator(device, seed, 9001), device).float()
        k = torch.empty((nseq, N, IDX_DIM), dtype=torch.bfloat16, device=device)
        for sq in range(nseq):
            z = torch.randint(0, CLUSTERS, (N,), generator=generator(device, seed, 8000 + sq), device=device)
            noise = torch.randn((N, IDX_DIM), generator=generator(device, seed, 7000 + sq), device=device)
            k[sq] = (cent[z] + CLUSTER_SIGMA * noise).to(torch.bfloat16)
        wl.k_idx = k
        wl.clustered_seed = seed
    else:
        wl.k_idx = bf16_normal((nseq, N, IDX_DIM), nxt(), device)

    if c["kv"] == "random":
        wl.kv = random_records(nseq * N, nxt(), device).view(nseq, N, RECORD)

    if c["planted"]:
        P = c["planted"]
        g = nxt()
        pos = torch.stack([torch.randperm(N, generator=g, device=device)[:P] for _ in range(nq)])
        qi = wl.q_idx[0].float()
        u = (wl.w[0].unsqueeze(-1) * qi).sum(1)
        u = u / u.norm(dim=-1, keepdim=True)
        eps = torch.randn((nq, P, IDX_DIM), generator=nxt(), device=device)
        kp = PLANT_K_GAIN * math.sqrt(IDX_DIM) * u.unsqueeze(1) + 0.1 * eps
        seqs = torch.arange(nq, device=device) // q_per_seq
        wl.k_idx[seqs.unsqueeze(1).expand(-1, P), pos] = kp.to(torch.bfloat16)
        v = wl.q[0].float().sum(1)
        v = v / v.norm(dim=-1, keepdim=True)
        rows = (PLANT_V_NORM * v).unsqueeze(1).expand(-1, P, -1).reshape(-1, DIM).to(torch.bfloat16)
        wl.kv_prepack_rows = (seqs.unsqueeze(1) * N + pos).reshape(-1)
        wl.kv_prepack = rows.contiguous()
        wl.planted = pos

    if c["prefill"]:
        pos = (PREFILL_CONTEXT - nq) + torch.arange(nq, device=device, dtype=torch.int64)
        nv = torch.clamp((pos + 1) // PREFILL_M, max=N)
        wl.n_visible = nv.to(torch.int32)
        # One token-level window buffer of nq + 127 rows: query j sees rows [j, j+128).
        wl.swa_start = torch.arange(nq, device=device, dtype=torch.int32)
        wl.swa_len = torch.full((nq,), WINDOW, device=device, dtype=torch.int32)
    else:
        wl.swa_start = torch.zeros((nq,), device=device, dtype=torch.int32)
        wl.swa_len = torch.full((nq,), WINDOW, device=device, dtype=torch.int32)
    return wl
