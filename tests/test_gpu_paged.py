"""GPU parity of the paged KV cache (decode): append, index branch and sparse
branch over pools of pages addressed through a block table.

* append: the pools after msa_kv_append_paged equal a host scatter of the
  same rows, bit for bit; padding slots (-1) and slots past the pool are
  skipped;
* paged decode equals contiguous decode bit for bit on the same logical cache
  (ids, O and LSE), with pages scattered at random through a larger pool of
  noise, and also meets the oracle (ids exact off near ties, O within
  atol 2e-3 / rtol 1e-2);
* shared pages: two sequences whose first blocks map to one page;
* the headline decode workload (4 x 1M context) at full size, paged in with
  the append kernel.
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


def bits(t):
    """Raw 16-bit patterns of a bf16 tensor (exact comparison)."""
    return t.view(torch.int16).cpu().numpy()


def run_both(inp, extra_pages=37, seed=0, table=None):
    """Contiguous and paged decode on the same inputs; returns both results."""
    from block_sparse_gqa_amd import device
    wl = inp.wl
    dp = device.upload(inp)
    ids_c, out_c, lse_c = device.forward(dp)
    blocks = sum((n + wl.block_size - 1) // wl.block_size for n in wl.seqlens_k)
    num_pages = blocks + extra_pages
    if table is None:
        table = device.random_page_table(wl.seqlens_k, wl.block_size, num_pages, seed)
    else:
        num_pages = max(num_pages, int(table.max()) + 1)
    pc = device.alloc_paged(wl, table, num_pages)
    device.page_in(dp, pc, table)
    ids_p = device.index_topk_paged(dp, pc)
    out_p, lse_p = device.sparse_attention_paged(dp, pc, ids_p)
    torch.cuda.synchronize()
    res = dict(ids_c=ids_c.cpu().numpy(), ids_p=ids_p.cpu().numpy(), out_c=bits(out_c), out_p=bits(out_p),
               lse_c=lse_c.cpu().numpy(), lse_p=lse_p.cpu().numpy(), out_p_f=out_p.float().cpu().numpy())
    del dp, pc
    return res


def assert_same(r, label):
    np.testing.assert_array_equal(r["ids_p"], r["ids_c"], err_msg=f"{label}: paged ids")
    np.testing.assert_array_equal(r["out_p"], r["out_c"], err_msg=f"{label}: paged O bits")
    np.testing.assert_array_equal(r["lse_p"].view(np.int32), r["lse_c"].view(np.int32), err_msg=f"{label}: paged LSE")


CASES = [
    # name, seqlens_k, H, h, d, d_idx, B, k
    ("paged_B64", (1000, 64, 1, 4097), 32, 8, 128, 64, 64, 8),
    ("paged_B128_d64", (5000, 129, 128), 16, 16, 64, 32, 128, 5),
    ("paged_k_over_E", (200, 3000), 16, 4, 128, 64, 64, 64),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_equals_contiguous_and_oracle(case):
    name, sk, H, h, d, di, B, k = case
    inp = synth.custom((1,) * len(sk), sk, H, h, d, di, B, k, seed=zlib.crc32(name.encode()) % 1000, name=name)
    say(f"[{name}] contiguous and paged decode")
    r = run_both(inp, seed=zlib.crc32(name.encode()) % 97)
    assert_same(r, name)
    rows = np.arange(inp.wl.total_q, dtype=np.int64)
    ref_ids, kth, tie = oracle.index_topk(inp, rows)
    rep = parity.compare_ids(oracle, inp, rows, r["ids_p"], ref_ids, kth, tie)
    ref_out, _ = oracle.sparse_attention(inp, r["ids_p"], rows)
    err = parity.assert_close(r["out_p_f"], ref_out, f"{name} paged attention (own ids)")
    say(f"[{name}] paged == contiguous bit for bit; selection {rep}; max err {err:.3g}")


@pytest.mark.timeout(300)
def test_shared_prefix_page():
    """Two sequences whose block 0 is one shared page (their first 64 tokens
    are made identical), the rest on private pages."""
    from block_sparse_gqa_amd import device
    inp = synth.custom((1, 1), (700, 300), 16, 4, 128, 64, 64, 6, seed=21, name="shared_prefix")
    B = 64
    c0, c1 = inp.cu_seqlens_k[0], inp.cu_seqlens_k[1]
    for arr in (inp.k, inp.v, inp.k_idx):
        arr[c1:c1 + B] = arr[c0:c0 + B]
    wl = inp.wl
    table = device.random_page_table(wl.seqlens_k, B, 40, seed=3)
    table[1, 0] = table[0, 0]
    r = run_both(inp, table=table)
    assert_same(r, "shared_prefix")


@pytest.mark.timeout(300)
def test_append_scatter_exact():
    """Prefill-sized appends, then one decode token per sequence, then a
    batch with padding and out-of-pool slots: pools must equal a host scatter
    of the same rows, and untouched rows must keep their old contents."""
    from block_sparse_gqa_amd import device
    rng = np.random.Generator(np.random.PCG64(5))
    h, d, di, B = 8, 128, 64, 64
    wl = synth.custom((1, 1, 1), (300, 65, 128), 8, h, d, di, B, 4, seed=2).wl
    num_pages = 24
    table = device.random_page_table((301, 66, 129), B, num_pages, seed=9)
    pc = device.alloc_paged(wl, table, num_pages)
    host_k = bits(pc.k_pool).copy()
    host_v = bits(pc.v_pool).copy()
    host_ki = bits(pc.k_idx_pool).copy()

    def push(seq, pos, slots_override=None):
        n = len(seq)
        k = rng.standard_normal((n, h, d), np.float32)
        v = rng.standard_normal((n, h, d), np.float32)
        ki = rng.standard_normal((n, di), np.float32)
        kb, vb, kib = synth.f32_to_bf16_bits(k), synth.f32_to_bf16_bits(v), synth.f32_to_bf16_bits(ki)
        slots = device.slot_mapping(table, seq, pos, B) if slots_override is None else slots_override
        device.append(pc, torch.from_numpy(slots).cuda(), device.to_device_bf16(kb), device.to_device_bf16(vb),
                      device.to_device_bf16(kib))
        for i, sl in enumerate(slots):
            if 0 <= sl < num_pages * B:
                host_k[sl], host_v[sl], host_ki[sl] = kb[i].view(np.int16), vb[i].view(np.int16), kib[i].view(np.int16)

    lens = (300, 65, 128)
    seq = np.repeat(np.arange(3), lens)
    pos = np.concatenate([np.arange(n) for n in lens])
    push(seq, pos)                                           # the prompts
    push(np.arange(3), np.array(lens))                       # one decode token each
    seq2, pos2 = np.array([0, 1, 2, 0]), np.array([0, 1, 2, 3])
    slots = device.slot_mapping(table, seq2, pos2, B)
    slots[1] = -1                                            # padding
    slots[2] = num_pages * B + 5                             # outside the pools
    push(seq2, pos2, slots)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(pc.k_pool), host_k)
    np.testing.assert_array_equal(bits(pc.v_pool), host_v)
    np.testing.assert_array_equal(bits(pc.k_idx_pool), host_ki)


@pytest.mark.timeout(900)
def test_decode_1m_paged_full_size():
    """The 4 x 1M-context decode workload, paged in with the append kernel
    over a pool with spare pages: paged decode must equal contiguous decode
    bit for bit (the contiguous path is checked against the oracle at this
    size by the full-size parity test)."""
    say("[decode_1m_paged] generating inputs")
    inp = synth.make_inputs("decode_1m")
    r = run_both(inp, extra_pages=4096, seed=17)
    assert_same(r, "decode_1m_paged")
    say("[decode_1m_paged] paged == contiguous bit for bit")
