"""Host-side pieces of bench.py, on the CPU: the visible-token count that the
roofline's algorithmic work is built from (checked by brute force), the
kernel-name parsing behind the traffic table, the traffic lookup's refusal of
counters taken on other sources, and the one-GPU refusal of --gpus N > 1."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def brute_visible(ids, cu_q, cu_k, B):
    """Visible selected tokens per (row, group) by walking every token of every selected block."""
    total_q, h, k = ids.shape
    out = np.zeros((total_q, h), np.int64)
    for s in range(len(cu_q) - 1):
        lq, lk = cu_q[s + 1] - cu_q[s], cu_k[s + 1] - cu_k[s]
        for r in range(lq):
            p = lk - lq + r
            for g in range(h):
                for j in ids[cu_q[s] + r, g]:
                    if j < 0:
                        continue
                    out[cu_q[s] + r, g] += sum(1 for t in range(j * B, min((j + 1) * B, lk)) if t <= p)
    return out


@pytest.mark.parametrize("B", [4, 8])
def test_visible_tokens_brute_force(B):
    rng = np.random.default_rng(5)
    lens_q = [5, 1, 0, 9]
    lens_k = [13, 7, 3, 9]     # bottom-right aligned; a partial last block in most sequences
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    h, k = 3, 3
    ids = np.full((cu_q[-1], h, k), -1, np.int32)
    for s in range(len(lens_q)):
        for r in range(lens_q[s]):
            p = lens_k[s] - lens_q[s] + r
            E = p // B + 1
            for g in range(h):
                pick = np.sort(rng.choice(E, size=min(k, E), replace=False))
                ids[cu_q[s] + r, g, :len(pick)] = pick
    got = bench.visible_tokens(torch.from_numpy(ids), torch.from_numpy(cu_q), torch.from_numpy(cu_k), B)
    np.testing.assert_array_equal(got.numpy(), brute_visible(ids, cu_q, cu_k, B))


def test_kernel_symbol_parsing():
    assert bench._kernel_symbol("void msa::(anonymous namespace)::attn_prefill_tile<128, 16>(unsigned short const*, int)") \
        == ("attn_prefill_tile", "attn_prefill_tile<128, 16>")
    assert bench._kernel_symbol("msa::(anonymous namespace)::lists_count_lds(int const*, long)") \
        == ("lists_count_lds", "lists_count_lds")
    assert bench._kernel_symbol("void msa::(anonymous namespace)::fwd_block<128, 64>(msa::FastDiv, float)") \
        == ("fwd_block", "fwd_block<128, 64>")


def test_traffic_lookup_matches_sources_only(tmp_path, monkeypatch):
    table = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic.json")))
    entries = [e for e in table["kernels"] if e["workload"] == "prefill_32k" and e["symbol"] == "fwd_merge"]
    assert entries, "the committed table has the 32K merge"
    kernels = [("attn_block_fwd.hip", "fwd_merge")]
    assert bench.measured_traffic(kernels, "prefill_32k") == pytest.approx(entries[0]["bytes_per_dispatch"])
    # a workload the counters were not taken on, or a kernel the table does not hold: no figure
    assert bench.measured_traffic(kernels, "no_such_workload") is None
    assert bench.measured_traffic([("attn_block_fwd.hip", "no_such_kernel")], "prefill_32k") is None
    # counters taken on another version of the source: no figure
    fake_root = tmp_path / "repo"
    (fake_root / "profiles").mkdir(parents=True)
    (fake_root / "block_sparse_gqa_amd" / "csrc").mkdir(parents=True)
    (fake_root / "profiles" / "hbm_traffic.json").write_text(json.dumps(table))
    (fake_root / "block_sparse_gqa_amd" / "csrc" / "attn_block_fwd.hip").write_text("// another version\n")
    monkeypatch.setattr(bench, "ROOT", str(fake_root))
    assert bench.measured_traffic(kernels, "prefill_32k") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
