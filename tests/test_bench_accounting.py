"""Host-side byte and flop accounting of bench.py against the figures derived
from the pages' shapes (per query-layer attention bytes and flops, the
decode steps' algorithmic bytes, the headline kernel's bytes per launch), and
the machine-read lines of the committed counter summaries."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


class _Wl:
    """The shape fields bench's accounting reads from a workload."""

    def __init__(self, nq, N, hier, n_index_layers, n_attn_layers, kfmt="bf16", q_per_seq=1, qfmt="bf16"):
        self.nq, self.N, self.hier, self.kfmt, self.q_per_seq, self.qfmt = nq, N, hier, kfmt, q_per_seq, qfmt
        self.nseq = nq // q_per_seq
        self.n_visible = None
        self.n_index_layers, self.n_attn_layers = n_index_layers, n_attn_layers


def test_attention_bytes_and_flops_per_query_layer():
    # 512 x 288 B records + 128 x 1 KiB window rows + 64 KiB Q + 64 KiB out + 512 x 4 B ids
    assert bench.alg_bytes_attn(1) == 411648
    # 2 products x 64 heads x 640 keys x 512 dims x 2 flop
    assert bench.alg_flops_attn(1) == 83886080
    assert bench.alg_bytes_attn(1024) == 1024 * 411648
    # FP8 window rows: 128 x 528 B
    assert bench.alg_bytes_attn(1, window_row=528) == 512 * 288 + 128 * 528 + 2 * 65536 + 2048


def test_prefill_fused_scoring_bytes_with_mxfp4_query():
    # one sequence of 65536 FP4 key entries read once, 4096 x 512 ids written,
    # per query 32 MXFP4 entries (68 B) of indexer Q and 32 fp32 weights
    wl = _Wl(4096, 65536, False, 1, 1, kfmt="fp4", q_per_seq=4096, qfmt="fp4")
    assert bench.alg_bytes_index_topk(wl) == 65536 * 68 + 4096 * 512 * 4 + 4096 * (32 * 68 + 128)
    wl.qfmt = "bf16"
    assert bench.alg_bytes_index_topk(wl) == 65536 * 68 + 4096 * 512 * 4 + 4096 * (8192 + 128)


def test_headline_fused_scoring_bytes_per_launch():
    wl = _Wl(64, 32768, False, 1, 1)
    # keys + 8 chunks x 512 candidates x 8 B + query and weights
    assert bench.alg_bytes_index_topk(wl) == 64 * 32768 * 256 + 64 * 8 * 512 * 8 + 64 * (8192 + 128) == 539500544


@pytest.mark.parametrize("nq,N,mib", [(8, 1 << 20, 2235.1), (32, 262144, 2580.6), (64, 32768, 553.6)])
def test_step_bytes_match_the_derived_step_totals(nq, N, mib):
    hier = N > 100000
    wl = _Wl(nq, N, hier, 4 if hier else 1, 5 if hier else 1)
    got = bench.alg_bytes_step_unfused(wl) / 2 ** 20
    # the derived totals round each call's MiB; agreement to 0.1 %
    assert abs(got - mib) <= 1e-3 * mib, (got, mib)


def test_committed_counter_summaries_are_machine_readable():
    for name, key in [("index_topk_encoder64k_traffic.md", "hbm_bytes_per_launch"),
                      ("sparse_attn_gather_traffic.md", "hbm_bytes_per_launch_1024q"),
                      ("index_prefill_prefill128k_mfma.md", "mfma_busy_scoring_only")]:
        text = open(os.path.join(ROOT, "profiles", name)).read()
        fields = dict(l.split(":", 1) for l in text.splitlines()
                      if ":" in l and not l.startswith(("|", "#", "`", "rocprof")))
        fields = {k.strip(): v.strip() for k, v in fields.items()}
        assert len(fields.get("kernel_source_sha256_16", "")) == 16, name
        float(fields[key])


def test_bench_refuses_more_than_one_gpu():
    """The benchmark measures one GPU; asking for more ends with a message and
    a non-zero status before any GPU work."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
