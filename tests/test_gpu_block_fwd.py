"""GPU parity of the block-centric prefill schedule
(msa_sparse_attn_prefill_blocks): per-(group, block) lists of selecting
queries, per-block partial outputs, log-sum-exp merge.

* against the oracle on the GPU's own ids: O within atol 2e-3 / rtol 1e-2 and
  LSE likewise, over ragged packing, partial final blocks, chunked prefill
  (len_q < len_k), G = 1, 3, 4, 6 and 16, d = 64 and 128, B = 64 and 128,
  k = 1, k covering every block (dense causal attention), and more
  (group, block) keys than the LDS count of the list pass holds;
* V scaled by 2^20 and by 2^-20, so each block's power-of-two scaling of V
  into fp16 is exercised (compared after undoing the scale);
* the query-tile kernel on the same ids agrees with it within the same
  tolerance, and two calls give identical bits;
* the 32K-token prefill workload at full size, sampled rows.
"""
import sys
import zlib

import numpy as np
import pytest

import oracle
from block_sparse_gqa_amd import synth
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run(inp):
    from block_sparse_gqa_amd import device
    dp = device.upload(inp)
    ids = device.index_topk(dp)
    out_b, lse_b = device.sparse_attention_blocks(dp, ids)
    out_q, lse_q = device.sparse_attention_tiles(dp, ids)
    torch.cuda.synchronize()
    res = dict(ids=ids.cpu().numpy(), out_b=out_b.float().cpu().numpy(), lse_b=lse_b.cpu().numpy(),
               out_q=out_q.float().cpu().numpy(), lse_q=lse_q.cpu().numpy())
    del dp
    return res


def check(inp, rows, label, scale=1.0):
    r = run(inp)
    ref_out, ref_lse = oracle.sparse_attention(inp, r["ids"][rows], rows)
    e1 = parity.assert_close(r["out_b"][rows] / scale, ref_out / scale, f"{label} block-centric O")
    e2 = parity.assert_close(r["lse_b"][rows], ref_lse, f"{label} block-centric LSE")
    e3 = parity.assert_close(r["out_b"] / scale, r["out_q"] / scale, f"{label} block-centric vs query-tile O")
    say(f"[{label}] max err: O {e1:.3g}, LSE {e2:.3g}; vs query-tile {e3:.3g}")


CASES = [
    # name, seqlens_q, seqlens_k, H, h, d, d_idx, B, k, clustered
    ("blk_d128_B64_G4", (700, 129), (700, 129), 16, 4, 128, 64, 64, 4, True),
    ("blk_d64_B128_G3", (900,), (900,), 6, 2, 64, 32, 128, 3, False),
    ("blk_G6_ragged", (300, 77, 257), (300, 77, 257), 48, 8, 128, 64, 128, 2, True),
    ("blk_G1", (400,), (400,), 4, 4, 64, 32, 64, 3, False),
    ("blk_G16", (333,), (333,), 16, 1, 128, 64, 64, 2, False),
    ("blk_dense", (257,), (257,), 8, 2, 128, 64, 64, 8, False),
    ("blk_k1", (600,), (600,), 12, 4, 128, 32, 64, 1, False),
    ("blk_chunked", (100, 37), (300, 400), 8, 4, 128, 64, 64, 3, False),
    ("blk_many_keys", (64, 64), (40000, 30000), 16, 16, 64, 32, 64, 3, False),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_block_centric_matches_oracle(case):
    name, sq, sk, H, h, d, di, B, k, cl = case
    inp = synth.custom(sq, sk, H, h, d, di, B, k, clustered=cl, seed=zlib.crc32(name.encode()) % 1000, name=name)
    say(f"[{name}] gpu run")
    check(inp, np.arange(inp.wl.total_q, dtype=np.int64), name)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("log2_scale", [20, -20])
def test_block_centric_v_scaling(log2_scale):
    name = f"blk_vscale_{log2_scale}"
    inp = synth.custom((500,), (500,), 8, 2, 128, 64, 64, 4, seed=11, name=name)
    scale = 2.0 ** log2_scale
    inp.v = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(inp.v) * np.float32(scale))
    say(f"[{name}] gpu run")
    check(inp, np.arange(inp.wl.total_q, dtype=np.int64), name, scale=scale)


@pytest.mark.timeout(300)
def test_block_centric_repeatable():
    from block_sparse_gqa_amd import device
    inp = synth.custom((777,), (777,), 16, 4, 128, 64, 64, 5, seed=5, name="blk_repeat")
    dp = device.upload(inp)
    ids = device.index_topk(dp)
    a, la = device.sparse_attention_blocks(dp, ids)
    b, lb = device.sparse_attention_blocks(dp, ids)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(la.view(torch.int32), lb.view(torch.int32))


@pytest.mark.timeout(900)
def test_block_centric_prefill_32k():
    say("[prefill_32k] generating inputs")
    inp = synth.make_inputs("prefill_32k")
    rows = synth.sample_rows(inp.wl, n_per_seq=160)
    say(f"[prefill_32k] gpu run, {len(rows)} sampled rows")
    check(inp, rows, "prefill_32k")
