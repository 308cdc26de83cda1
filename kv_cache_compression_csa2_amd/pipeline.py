"""One step of the CSA2 hot path, composed from the C-ABI calls.

Layer modes (titansim blog, CSA2 paragraph; eogee.com report 3.2 and 3.3):
  Full     score every visible entry, keep its own Top-512 (and, in the
           hierarchical decoder, the 2048 best 8-position blocks as the pool);
  Reindex  the layer's own indexer Q over the shared indexer K, inside the pool,
           keeps its own Top-512;
  Reuse    attends with the indices of the previous layer, no scoring.
Every layer attends with its own Q and its own window KV.

Decode workloads (one query per sequence) run the Full layer's scoring and
Top-512 fused (csa2_index_topk: no score row is written; its two launches are
timed separately; the hierarchical layer completes the Top-512 and selects
its 2048-block pool together, csa2_index_topk_merge_pool); so does the
prefill chunk (csa2_index_prefill_topk, one
launch when each row is one chunk). Reindex layers score the pool and select in one call
(csa2_index_reindex_topk); `fused_reindex = False` switches them to
csa2_index_reindex + csa2_topk. `debug_scores` makes the fused calls also
write the score rows (parity checks).

Buffers are allocated once per Step object, so a timed loop allocates nothing.
"""
import torch

from . import _lib as L
from .workloads import BLOCK, POOL_BLOCKS, TOPK


class Step:
    """Pre-allocated outputs for one workload; call run(...) per step."""

    def __init__(self, wl, device):
        self.wl = wl
        nq, N = wl.nq, wl.N
        f32, i32, bf16 = torch.float32, torch.int32, torch.bfloat16
        self.scores = torch.empty((nq, N), dtype=f32, device=device)
        self.blocks = torch.empty((nq, (N + 7) // 8), dtype=f32, device=device) if wl.hier else None
        self.top = [torch.empty((nq, TOPK), dtype=i32, device=device) for _ in range(wl.n_index_layers)]
        self.cand = torch.empty((nq, POOL_BLOCKS), dtype=i32, device=device) if wl.hier else None
        pool = POOL_BLOCKS * BLOCK
        self.pool_scores = torch.empty((nq, pool), dtype=f32, device=device) if wl.hier else None
        self.pool_ids = torch.empty((nq, pool), dtype=i32, device=device) if wl.hier else None
        self.out = [torch.empty((nq, L.HEADS, L.DIM), dtype=bf16, device=device) for _ in range(wl.n_attn_layers)]
        self.lse = [torch.empty((nq, L.HEADS), dtype=f32, device=device) for _ in range(wl.n_attn_layers)]

        def ws(nbytes):
            return torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=device)

        self.ws_topk = ws(max(L.csa2_topk_workspace_bytes(nq, N, TOPK),
                              L.csa2_topk_workspace_bytes(nq, (N + 7) // 8, POOL_BLOCKS) if wl.hier else 0,
                              L.csa2_topk_workspace_bytes(nq, pool, TOPK) if wl.hier else 0))
        self.ws_attn = ws(L.csa2_sparse_attn_workspace_bytes(nq, TOPK))
        self.fused = wl.q_per_seq == 1
        self.ws_ft = None
        if self.fused:
            # the hierarchical layer's pool selection runs beside the merge (csa2_index_topk_merge_pool)
            self.ws_ft = ws(L.csa2_index_topk_pool_workspace_bytes(nq, N, TOPK, POOL_BLOCKS) if wl.hier
                            else L.csa2_index_topk_workspace_bytes(nq, N, TOPK))
        # prefill chunk: scoring fused with the Top-512 (8 queries of a sequence per workgroup)
        self.prefill_fused = not self.fused and wl.q_per_seq % 8 == 0 and not wl.hier
        self.ws_pf = ws(L.csa2_index_prefill_topk_workspace_bytes(nq, N, TOPK)) if self.prefill_fused else None
        # MXFP4 indexer Q of every scoring layer (with FP4 K): packed inside the step from the bf16 query
        self.qfl = None
        if wl.qfmt == "fp4":
            if wl.kfmt != "fp4":
                raise ValueError("an MXFP4 indexer Q is scored against FP4 K entries")
            self.qfl = [torch.empty((nq, L.IDX_HEADS, L.KIDX_RECORD), dtype=torch.uint8, device=device)
                        for _ in range(wl.n_index_layers)]
        self.qf = self.qfl[0] if self.qfl else None
        self.debug_scores = False
        self.fused_reindex = True
        self.ws_rt = ws(L.csa2_index_reindex_topk_workspace_bytes(nq, POOL_BLOCKS, TOPK)) if wl.hier else None
        # FP8 window rows (the cache format; packed once, outside any timed step)
        self.swa8 = None
        if wl.swa_fmt == "fp8":
            self.swa8 = [L.swa_fp8_pack(s.reshape(-1, L.DIM)).view(s.shape[0], s.shape[1], L.SWA_RECORD)
                         for s in wl.swa]

    @staticmethod
    def _k(k):
        """(k_idx, k_fp4) keyword pair for an indexer-K operand: bf16 keys or
        FP4 entries (uint8 [.., 68])."""
        return (None, k) if k.dtype == torch.uint8 else (k, None)

    def index_full(self, k):
        wl = self.wl
        kb, kf = self._k(k)
        if wl.hier:
            L.csa2_index_full(wl.q_idx[0], wl.w[0], kb, wl.N, wl.q_per_seq, wl.n_visible, 8, self.scores,
                              self.blocks, k_fp4=kf)
        else:
            L.csa2_index_full(wl.q_idx[0], wl.w[0], kb, wl.N, wl.q_per_seq, wl.n_visible, 0, self.scores, k_fp4=kf)

    def _q(self, layer):
        """(q_idx, q_fp4) keyword pair of a scoring layer's indexer query."""
        return (None, self.qfl[layer]) if self.qfl else (self.wl.q_idx[layer], None)

    def index_topk(self, k, stage):
        wl = self.wl
        kb, kf = self._k(k)
        qb, qf = self._q(0)
        L.csa2_index_topk(qb, wl.w[0], kb, wl.N, TOPK, n_visible=wl.n_visible, block_size=8 if wl.hier else 0,
                          top=self.top[0], block_scores=self.blocks, scores=self.scores if self.debug_scores else None,
                          workspace=self.ws_ft, k_fp4=kf, stage=stage, q_fp4=qf)

    def index_prefill_topk(self, k):
        wl = self.wl
        kb, kf = self._k(k)
        qb, qf = self._q(0)
        L.csa2_index_prefill_topk(qb, wl.w[0], kb, wl.N, wl.q_per_seq, TOPK, n_visible=wl.n_visible,
                                  top=self.top[0], scores=self.scores if self.debug_scores else None,
                                  workspace=self.ws_pf, k_fp4=kf, q_fp4=qf)

    def pack_query(self, layer=0):
        """A scoring layer's bf16 indexer query -> one MXFP4 entry per head."""
        L.kidx_fp4_pack(self.wl.q_idx[layer].reshape(-1, L.IDX_DIM), out=self.qfl[layer].view(-1, L.KIDX_RECORD))

    def full_layer(self, k, sp):
        """The Full layer's scoring and Top-512 (+ the 2048-block pool)."""
        if self.qfl is not None:
            with sp("q_pack"):
                self.pack_query(0)
        if self.fused:
            with sp("index_topk"):
                self.index_topk(k, "select")
            if self.wl.hier:
                # Top-512 merge and the 2048-block pool, sharing launches
                with sp("topk_merge+pool"):
                    L.csa2_index_topk_merge_pool(self.wl.N, TOPK, self.top[0], self.blocks, POOL_BLOCKS,
                                                 cand_blocks=self.cand, workspace=self.ws_ft)
            else:
                with sp("topk_merge"):
                    self.index_topk(k, "merge")
        elif self.prefill_fused:
            with sp("index_topk"):
                self.index_prefill_topk(k)
        else:
            if self.qfl is not None:
                raise ValueError("the MXFP4-Q steps score with the fused calls")
            with sp("index_full"):
                self.index_full(k)
            with sp("topk_full"):
                self.topk_full()

    def topk_full(self):
        wl = self.wl
        L.csa2_topk(self.scores, TOPK, row_len=wl.n_visible, out=self.top[0], workspace=self.ws_topk)
        if wl.hier:
            L.csa2_topk(self.blocks, POOL_BLOCKS, out=self.cand, workspace=self.ws_topk)

    def reindex(self, layer, k):
        wl = self.wl
        kb, kf = self._k(k)
        qb, qf = self._q(layer)
        if self.fused_reindex:
            L.csa2_index_reindex_topk(qb, wl.w[layer], kb, wl.N, wl.q_per_seq, self.cand, TOPK,
                                      n_visible=wl.n_visible, top=self.top[layer],
                                      pool_scores=self.pool_scores if self.debug_scores else None,
                                      workspace=self.ws_rt, k_fp4=kf, q_fp4=qf)
            return
        L.csa2_index_reindex(qb, wl.w[layer], kb, wl.N, wl.q_per_seq, self.cand, wl.n_visible,
                             pool_scores=self.pool_scores, pool_ids=self.pool_ids, k_fp4=kf, q_fp4=qf)
        L.csa2_topk(self.pool_scores, TOPK, id_map=self.pool_ids, out=self.top[layer], workspace=self.ws_topk)

    def attend(self, layer, kv, idx):
        wl = self.wl
        if self.swa8 is not None:
            L.csa2_sparse_attn(wl.q[layer], kv, wl.N, wl.q_per_seq, idx, None, wl.swa_start, wl.swa_len,
                               out=self.out[layer], lse=self.lse[layer], workspace=self.ws_attn,
                               swa_fp8=self.swa8[layer])
        else:
            L.csa2_sparse_attn(wl.q[layer], kv, wl.N, wl.q_per_seq, idx, wl.swa[layer], wl.swa_start, wl.swa_len,
                               out=self.out[layer], lse=self.lse[layer], workspace=self.ws_attn)

    def prepare(self, k_idx):
        """Set-up outside a timed step: the decoder group's pool comes from a
        Full layer of another group."""
        if self.wl.group == "decoder":
            import contextlib
            self.full_layer(k_idx, lambda n: contextlib.nullcontext())

    def run(self, k_idx, kv, span=None):
        """The whole hot path once, layer by layer: the Full layer (not for the
        decoder group, whose pool prepare() built), each Reindex layer, and
        every attention layer on the Top-512 it inherits. `span(name)` gives
        an optional timing context per call."""
        import contextlib
        sp = span or (lambda n: contextlib.nullcontext())
        wl = self.wl
        if wl.group != "decoder":
            self.full_layer(k_idx, sp)
        done = {0} if wl.group != "decoder" else set()
        for layer, src in enumerate(wl.attn_src):
            if src not in done:
                if self.qfl is not None:
                    with sp("q_pack"):
                        self.pack_query(src)
                with sp("reindex+topk"):
                    self.reindex(src, k_idx)
                done.add(src)
            with sp("attn"):
                self.attend(layer, kv, self.top[src])
        return self.out


def workload_kidx(wl):
    """The indexer-K operand a workload's step reads: the bf16 keys, or their
    FP4 entries packed on the GPU (kidx_fp4_pack) for kfmt == "fp4"."""
    if wl.kfmt != "fp4":
        return wl.k_idx
    return L.kidx_fp4_pack(wl.k_idx.reshape(-1, L.IDX_DIM)).view(wl.nseq, wl.N, L.KIDX_RECORD)


def pack_workload_kv(wl, device):
    """Main-KV cache of a workload, packed on the GPU where rows come as bf16."""
    from .workloads import RECORD, clustered_kv_rows
    if wl.kv is None:
        kv = torch.empty((wl.nseq, wl.N, RECORD), dtype=torch.uint8, device=device)
        for s in range(wl.nseq):
            for r0 in range(0, wl.N, 262144):
                n = min(262144, wl.N - r0)
                rows = clustered_kv_rows(wl.clustered_seed, s, wl.N, device, r0, n)
                L.fp4_kv_pack(rows.contiguous(), out=kv[s, r0:r0 + n])
    else:
        kv = wl.kv.clone()
    if wl.kv_prepack is not None:
        packed = L.fp4_kv_pack(wl.kv_prepack)
        kv.view(-1, RECORD)[wl.kv_prepack_rows] = packed
    return kv
