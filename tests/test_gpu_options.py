"""GPU parity of the selection options: forced attention-sink and local
blocks (msa_index_topk_ex) against the oracle's forced TopK, on the one-wave
select path (prefill rows), the workgroup select path (decode over more than
2048 blocks) and a paged cache; attention then runs on the GPU's own ids and
is checked against the oracle on those ids."""
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


CASES = [
    # name, seqlens_q, seqlens_k, H, h, d, d_idx, B, k, sink, local
    ("prefill_s1_l1", (700, 129), (700, 129), 16, 4, 128, 64, 64, 4, 1, 1),
    ("prefill_s2_l3_B128", (900,), (900,), 12, 2, 64, 32, 128, 5, 2, 3),
    ("prefill_forced_is_k", (600,), (600,), 8, 2, 128, 64, 64, 3, 1, 2),
    ("decode_block_path", (1, 1), (140_000, 2_000), 8, 2, 128, 64, 64, 16, 1, 2),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_forced_blocks(case):
    from block_sparse_gqa_amd import device
    name, sq, sk, H, h, d, di, B, k, sink, local = case
    inp = synth.custom(sq, sk, H, h, d, di, B, k, seed=zlib.crc32(name.encode()) % 1000, name=name)
    dp = device.upload(inp)
    ids = device.index_topk_forced(dp, sink, local)
    out, lse = device.sparse_attention(dp, ids)
    torch.cuda.synchronize()
    gids = ids.cpu().numpy()
    rows = np.arange(inp.wl.total_q, dtype=np.int64)
    ref_ids, kth, tie = oracle.index_topk(inp, rows, sink=sink, local=local)
    rep = parity.compare_ids(oracle, inp, rows, gids, ref_ids, kth, tie)
    ref_out, ref_lse = oracle.sparse_attention(inp, gids, rows)
    e1 = parity.assert_close(out.float().cpu().numpy(), ref_out, f"{name} attention")
    parity.assert_close(lse.cpu().numpy(), ref_lse, f"{name} lse")
    say(f"[{name}] selection {rep}; attention max err {e1:.3g}")


@pytest.mark.timeout(300)
def test_forced_blocks_paged():
    from block_sparse_gqa_amd import device
    inp = synth.custom((1, 1, 1), (3000, 70, 900), 16, 4, 128, 64, 64, 8, seed=31, name="paged_forced")
    wl = inp.wl
    dp = device.upload(inp)
    blocks = sum((n + 63) // 64 for n in wl.seqlens_k)
    table = device.random_page_table(wl.seqlens_k, 64, blocks + 9, seed=4)
    pc = device.alloc_paged(wl, table, blocks + 9)
    device.page_in(dp, pc, table)
    ids_p = device.index_topk_forced(dp, 2, 1, pc=pc)
    ids_c = device.index_topk_forced(dp, 2, 1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids_p.cpu().numpy(), ids_c.cpu().numpy())
    rows = np.arange(wl.total_q, dtype=np.int64)
    ref_ids, kth, tie = oracle.index_topk(inp, rows, sink=2, local=1)
    rep = parity.compare_ids(oracle, inp, rows, ids_p.cpu().numpy(), ref_ids, kth, tie)
    say(f"[paged_forced] selection {rep}")


# Decode rows whose eligible-block counts sit on every key-width boundary of the
# one-wave select (1, 2, 4, 8, 16 and 32 keys per lane: 64, 128, ..., 2048
# blocks): one launch holds them all, and each row takes the narrowest width
# that holds it.
WIDTH_EDGES = (33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 512, 513, 1023, 1024, 1025, 2047, 2048)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("sink,local", [(0, 0), (1, 2)])
def test_select_width_boundaries(sink, local):
    from block_sparse_gqa_amd import device
    rng = np.random.default_rng(5)
    B, k = 64, 32
    lens_k = tuple(int((e - 1) * B + 1 + rng.integers(0, B)) for e in WIDTH_EDGES)   # row position p gives E = p / B + 1
    inp = synth.custom((1,) * len(lens_k), lens_k, 8, 2, 128, 64, B, k, seed=19, name="width_edges")
    dp = device.upload(inp)
    ids = device.index_topk_forced(dp, sink, local) if (sink or local) else device.index_topk(dp)
    out, lse = device.sparse_attention(dp, ids)
    torch.cuda.synchronize()
    gids = ids.cpu().numpy()
    rows = np.arange(inp.wl.total_q, dtype=np.int64)
    ref_ids, kth, tie = oracle.index_topk(inp, rows, sink=sink, local=local)
    rep = parity.compare_ids(oracle, inp, rows, gids, ref_ids, kth, tie)
    ref_out, ref_lse = oracle.sparse_attention(inp, gids, rows)
    parity.assert_close(out.float().cpu().numpy(), ref_out, "width edges attention")
    parity.assert_close(lse.cpu().numpy(), ref_lse, "width edges lse")
    say(f"[width_edges sink={sink} local={local}] selection {rep}")
