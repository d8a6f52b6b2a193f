"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

* selection: bit-exact top-k ids, near ties judged by the band rule;
* attention: atol 2e-3 / rtol 1e-2, run with the oracle's ids (so selection and
  attention are pinned separately), and end to end with the GPU's own ids on
  every row where those equal the oracle's;
* edge cases: ragged packing, empty sequences inside a batch, partial final blocks, rows with fewer eligible
  blocks than k, k covering every block, G = 1 and G = 16, decode contexts
  shorter than one block, planted and all-tie closed forms, determinism.
The five named workloads run at full size with the launch configuration the
benchmark times; prefill rows are sampled (block edges, sequence ends and
seeded random rows).
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


def run_gpu(inp, ids_override=None):
    from block_sparse_gqa_amd import device
    dp = device.upload(inp)
    ids = device.index_topk(dp)
    out, lse = device.sparse_attention(dp, ids)
    res = dict(ids=ids.cpu().numpy(), out=out.float().cpu().numpy(), lse=lse.cpu().numpy())
    if ids_override is not None:
        ids2 = torch.from_numpy(ids_override).to(ids.device)
        out2, lse2 = device.sparse_attention(dp, ids2)
        res["out_given"] = out2.float().cpu().numpy()
        res["lse_given"] = lse2.cpu().numpy()
        if not inp.wl.is_decode:
            # both prefill schedules explicitly, whichever the call above chose
            from block_sparse_gqa_amd import msa
            for name, fn, op in (("tiles", device.sparse_attention_tiles, msa.MSA_OP_SPARSE_ATTN_PREFILL_TILES),
                                 ("blocks", device.sparse_attention_blocks, msa.MSA_OP_SPARSE_ATTN_PREFILL_BLOCKS)):
                ws = device.workspace(dp, op)
                o3, l3 = fn(dp, ids2, ws=ws)
                torch.cuda.synchronize()
                if name == "tiles":
                    # every hand-off wait between the waves ended before its bound
                    assert device.wait_word(dp, op, ws) == 0
                res[f"out_{name}"] = o3.float().cpu().numpy()
                res[f"lse_{name}"] = l3.cpu().numpy()
                del o3, l3, ws
                torch.cuda.empty_cache()
    torch.cuda.synchronize()
    del dp
    return res


def check_case(inp, rows=None, label=""):
    """Full comparison of one input set; returns the selection report."""
    wl = inp.wl
    all_rows = np.arange(wl.total_q, dtype=np.int64)
    rows = all_rows if rows is None else rows
    ref_ids, kth, tie = oracle.index_topk(inp, rows)
    # GPU attention runs once with the oracle's ids on the checked rows (GPU's
    # own ids elsewhere are not needed: fill the rest with the first eligible block).
    given = np.full((wl.total_q, wl.num_kv_heads, wl.top_k), -1, np.int32)
    given[:, :, 0] = 0
    given[rows] = ref_ids
    say(f"[{label}] gpu run: {wl.name} rows={len(rows)}")
    g = run_gpu(inp, ids_override=given)
    rep = parity.compare_ids(oracle, inp, rows, g["ids"][rows], ref_ids, kth, tie)
    say(f"[{label}] selection: {rep}")
    ref_out, ref_lse = oracle.sparse_attention(inp, ref_ids, rows)
    e1 = parity.assert_close(g["out_given"][rows], ref_out, f"{label} attention (oracle ids)")
    e2 = parity.assert_close(g["lse_given"][rows], ref_lse, f"{label} lse (oracle ids)")
    for name in ("tiles", "blocks"):
        if f"out_{name}" in g:
            parity.assert_close(g[f"out_{name}"][rows], ref_out, f"{label} attention, {name} schedule (oracle ids)")
            parity.assert_close(g[f"lse_{name}"][rows], ref_lse, f"{label} lse, {name} schedule (oracle ids)")
    same = np.array([np.array_equal(g["ids"][r], ref_ids[i]) for i, r in enumerate(rows)])
    e3 = parity.assert_close(g["out"][rows[same]], ref_out[same], f"{label} end-to-end attention")
    say(f"[{label}] attention max err: oracle-ids {e1:.3g}, lse {e2:.3g}, end-to-end {e3:.3g} "
        f"({int(same.sum())}/{len(rows)} rows with identical ids)")
    return rep, g


SMALL = [
    # name, seqlens_q, seqlens_k, H, h, d, d_idx, B, k, clustered
    ("prefill_d64_B64", (1024,), (1024,), 6, 2, 64, 32, 64, 4, False),
    ("ragged_partial", (300, 77, 129, 64), (300, 77, 129, 64), 8, 2, 128, 64, 64, 3, True),
    ("ragged_B128_G6", (700, 257, 131), (700, 257, 131), 48, 8, 128, 64, 128, 4, True),
    ("k_covers_all", (513,), (513,), 4, 2, 64, 32, 64, 16, False),
    ("G1_h8", (400,), (400,), 8, 8, 128, 64, 64, 2, False),
    ("G16_h1", (333,), (333,), 16, 1, 64, 64, 128, 2, False),
    ("k1", (600,), (600,), 12, 4, 128, 32, 64, 1, False),
    ("decode_short", (1, 1, 1, 1), (1, 63, 64, 1000), 32, 8, 128, 64, 64, 8, False),
    ("decode_B128_d64", (1, 1, 1), (5000, 129, 128), 16, 16, 64, 32, 128, 5, False),
    ("decode_k_over_E", (1, 1), (200, 3000), 16, 4, 128, 64, 64, 64, False),
    ("chunked_prefill", (100, 37), (300, 400), 8, 4, 128, 64, 64, 3, False),
    ("empty_sequences", (0, 300, 0, 129), (0, 300, 0, 129), 8, 2, 128, 64, 64, 3, True),
    # long enough for the automatic prefill to split its rows: query tiles for positions below 1600
    # (R = 64 * 4 / E >= 10), the block-centric schedule after, across two sequences
    ("hybrid_split", (6000, 2500), (6000, 2500), 16, 4, 128, 64, 64, 4, True),
    # the same split inside chunked prefills (queries at positions 1000..2999 and 1500..2199 of their sequences)
    ("hybrid_split_chunked", (2000, 700), (3000, 2200), 16, 4, 128, 64, 64, 4, True),
    # one query per non-empty sequence, with empty ones before and between: not the decode shape
    # (total_q != num_seqs), so the index call takes the prefill kernel, which skips them
    ("decode_like_empty_seqs", (0, 1, 0, 1), (50, 700, 300, 1500), 32, 8, 128, 64, 64, 8, False),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_cases(case):
    name, sq, sk, H, h, d, di, B, k, cl = case
    inp = synth.custom(sq, sk, H, h, d, di, B, k, clustered=cl, seed=zlib.crc32(name.encode()) % 1000, name=name)
    check_case(inp, label=name)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("log2_scale", [24, -24])
def test_value_magnitude(log2_scale):
    """V scaled by 2^24 and 2^-24 (exactly, in bf16): O scales by the same
    power of two, so O / 2^s must meet the tolerance against the oracle's
    O / 2^s (the tolerance is stated for unit-scale values).  The prefill
    path's fp16 copy of V is rescaled by a power of two internally, which must
    be invisible."""
    from block_sparse_gqa_amd import device
    inp = synth.custom((600, 129), (600, 129), 8, 2, 128, 64, 64, 4, seed=11, name=f"v_2^{log2_scale}")
    f = np.float32(2.0 ** log2_scale)
    inp.v[...] = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(inp.v) * f)
    rows = np.arange(inp.wl.total_q, dtype=np.int64)
    ref_ids, _, _ = oracle.index_topk(inp, rows)
    ref_out, ref_lse = oracle.sparse_attention(inp, ref_ids, rows)
    dp = device.upload(inp)
    out, lse = device.sparse_attention(dp, torch.from_numpy(ref_ids).to(dp.q.device))
    torch.cuda.synchronize()
    err = parity.assert_close(out.float().cpu().numpy() / f, ref_out / f, f"{inp.wl.name} attention / 2^s")
    parity.assert_close(lse.cpu().numpy(), ref_lse, f"{inp.wl.name} lse")
    say(f"[{inp.wl.name}] max err of O / 2^s: {err:.3g}")


@pytest.mark.timeout(300)
def test_value_magnitude_per_head():
    """V of different (sequence, KV head) pairs scaled by very different powers
    of two (2^20 down to 2^-28, exact in bf16).  Each group's O / 2^s must meet
    the tolerance against the oracle's O / 2^s on all three prefill calls: the
    query-tile schedule scales its fp16 copy of V per (sequence, head), so a
    head far below another keeps its relative precision (one scale for the
    whole tensor would flush it to zero), and the block-centric schedule
    scales per block."""
    from block_sparse_gqa_amd import device
    H, h = 8, 4
    inp = synth.custom((500, 300), (500, 300), H, h, 128, 64, 64, 4, seed=23, name="v_per_head_scales")
    log2 = np.array([[20, -28, 0, 9], [-12, 3, -28, 20]])   # [sequence, KV head]
    cu = inp.cu_seqlens_k
    vf = synth.bf16_bits_to_f32(inp.v)
    for s in range(2):
        for g in range(h):
            vf[cu[s]:cu[s + 1], g] *= np.float32(2.0 ** log2[s, g])
    inp.v[...] = synth.f32_to_bf16_bits(vf)
    rows = np.arange(inp.wl.total_q, dtype=np.int64)
    ref_ids, _, _ = oracle.index_topk(inp, rows)
    ref_out, ref_lse = oracle.sparse_attention(inp, ref_ids, rows)
    seq = np.searchsorted(inp.cu_seqlens_q, rows, side="right") - 1
    f = (2.0 ** log2[seq][:, np.arange(H) // (H // h)]).astype(np.float32)[:, :, None]
    dp = device.upload(inp)
    ids = torch.from_numpy(ref_ids).to(dp.q.device)
    for name, fn in (("auto", device.sparse_attention), ("tiles", device.sparse_attention_tiles),
                     ("blocks", device.sparse_attention_blocks)):
        out, lse = fn(dp, ids)
        torch.cuda.synchronize()
        err = parity.assert_close(out.float().cpu().numpy() / f, ref_out / f, f"{name}: attention / 2^s")
        parity.assert_close(lse.cpu().numpy(), ref_lse, f"{name}: lse")
        say(f"[v_per_head_scales] {name}: max err of O / 2^s {err:.3g}")


@pytest.mark.timeout(300)
def test_split_prefill_ignores_stale_workspace():
    """The automatic prefill splits this call's rows between the schedules, and
    the query tiles' fp16 copy of V then covers only the key blocks they can
    stage.  With the workspace filled with NaN bit patterns before the call, no
    stale value may reach the output (a masked key still enters the P.V
    product with weight 0, and 0 * NaN is NaN)."""
    from block_sparse_gqa_amd import device
    inp = synth.custom((6000, 2500), (6000, 2500), 16, 4, 128, 64, 64, 4, clustered=True, seed=7,
                       name="stale_workspace")
    rows = np.unique(np.concatenate([np.arange(0, 8500, 37), np.arange(2200, 2400), np.arange(6000, 6100)]))
    ref_ids, _, _ = oracle.index_topk(inp, rows)
    ref_out, ref_lse = oracle.sparse_attention(inp, ref_ids, rows)
    given = np.zeros((inp.wl.total_q, 4, 4), np.int32)
    given[:, :, 1:] = -1
    given[rows] = ref_ids
    dp = device.upload(inp)
    dp.ws_attn.fill_(0xFF)   # fp16 0xFFFF is NaN
    out, lse = device.sparse_attention(dp, torch.from_numpy(given).to(dp.q.device))
    torch.cuda.synchronize()
    err = parity.assert_close(out.float().cpu().numpy()[rows], ref_out, "attention after a NaN-filled workspace")
    parity.assert_close(lse.cpu().numpy()[rows], ref_lse, "lse after a NaN-filled workspace")
    say(f"[stale_workspace] max err {err:.3g} over {len(rows)} rows")


def test_dense_equivalence_through_gpu():
    """k >= #blocks: the GPU output equals dense causal attention; here the
    oracle (itself pinned to float64 dense attention) is the reference and the
    GPU ids must be every block."""
    inp = synth.custom((257, 190), (257, 190), 8, 2, 128, 64, 64, 8, seed=3)
    rep, g = check_case(inp, label="dense")
    for row in range(inp.wl.total_q):
        s = 0 if row < 257 else 1
        p = row - inp.cu_seqlens_q[s]
        E = p // 64 + 1
        assert list(g["ids"][row, 0, :E]) == list(range(E))


def test_planted_and_all_ties_closed_forms():
    n, h, B, K, di = 1024, 2, 64, 3, 32
    q_idx = np.zeros((n, h, di), np.float32)
    q_idx[:, 0, 0] = 1.0
    q_idx[:, 1, 1] = 1.0
    k_idx = np.zeros((n, di), np.float32)
    planted = {0: [2, 5, 9, 14], 1: [1, 3, 4, 15]}
    for g, blocks in planted.items():
        for rank, j in enumerate(blocks):
            k_idx[j * B + 10, g] = 100.0 - 10.0 * rank
    inp = synth.custom((n,), (n,), 4, h, 64, di, B, K, seed=1)
    inp.q_idx = synth.f32_to_bf16_bits(q_idx)
    inp.k_idx = synth.f32_to_bf16_bits(k_idx)
    g = run_gpu(inp)
    last = g["ids"][n - 1]
    assert list(last[0]) == sorted(planted[0][:3])
    assert list(last[1]) == sorted(planted[1][:3])
    # all ties: every block score equal -> ids 0..m-1
    inp.k_idx = synth.f32_to_bf16_bits(np.full((n, di), 0.25, np.float32))
    g = run_gpu(inp)
    for row in range(0, n, 37):
        E = row // B + 1
        m = min(K, E)
        assert list(g["ids"][row, 0]) == list(range(m)) + [-1] * (K - m)


# name, context length, block size, top_k, period of the block-score levels:
# decode rows long enough for the workgroup-level select, with many exactly
# equal block scores.
LONG_TIES = [
    ("e4096_k1024_all_equal", 4096 * 64, 64, 1024, 1),
    ("e4096_k2048_three_levels", 4096 * 64, 64, 2048, 3),
    ("e40000_k4096_seven_levels", 40000 * 64, 64, 4096, 7),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("case", LONG_TIES, ids=[c[0] for c in LONG_TIES])
def test_long_row_ties_closed_forms(case):
    """Block j's score is exactly 1 + (j mod period): the selection is every
    block of the top level from the lowest id on, then the next level's
    lowest ids, i.e. the first k blocks in (score desc, id asc) order."""
    name, L, B, K, period = case
    say(f"[{name}] decode at context {L}")
    inp = synth.custom((1,), (L,), 2, 1, 64, 32, B, K, seed=3, name=name)
    q_idx = np.zeros((1, 1, 32), np.float32)
    q_idx[0, 0, 0] = 1.0
    k_idx = np.zeros((L, 32), np.float32)
    k_idx[:, 0] = 1.0 + (np.arange(L) // B) % period
    inp.q_idx = synth.f32_to_bf16_bits(q_idx)
    inp.k_idx = synth.f32_to_bf16_bits(k_idx)
    g = run_gpu(inp)
    E = L // B
    level = 1 + np.arange(E) % period
    first_k = np.lexsort((np.arange(E), -level))[:K]
    assert list(g["ids"][0, 0]) == sorted(int(x) for x in first_k)


def test_determinism():
    inp = synth.custom((777,), (777,), 16, 4, 128, 64, 64, 5, seed=5)
    a = run_gpu(inp)
    b = run_gpu(inp)
    np.testing.assert_array_equal(a["ids"], b["ids"])
    np.testing.assert_array_equal(a["out"], b["out"])


# name, seqlens_q, seqlens_k, H, h, d, d_idx, B, k: selection paths the headline
# workloads do not reach.
LONG = [
    # 32768 blocks: workgroup select with 32 keys per thread; top_k at its maximum
    ("decode_e32k_k4096", (1, 1), (2_097_152, 1_500_000), 4, 1, 64, 32, 64, 4096),
    # 62500 blocks: 64 keys per thread
    ("decode_e62k", (1,), (4_000_000,), 2, 1, 64, 32, 64, 64),
    # 1250 blocks: one wave per row with 32 keys per lane
    ("prefill_e1250", (80_000,), (80_000,), 4, 2, 64, 32, 64, 8),
    # index keys above the 192 MiB line (non-temporal scan) with short sequences beside the long one: their waves
    # score at most one block, so every prefetch past it reads the L2-resident query row; one cache is a single
    # partial block
    ("decode_mixed_streamed", (1, 1, 1, 1), (3_300_000, 100, 5000, 40), 4, 2, 64, 32, 64, 16),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", LONG, ids=[c[0] for c in LONG])
def test_long_rows(case):
    name, sq, sk, H, h, d, di, B, k = case
    inp = synth.custom(sq, sk, H, h, d, di, B, k, seed=zlib.crc32(name.encode()) % 1000, name=name)
    rows = None if inp.wl.is_decode else synth.sample_rows(inp.wl, n_per_seq=96)
    rep, _ = check_case(inp, rows=rows, label=name)
    say(f"[{name}] near-tie pairs {rep['near_tie']} of {rep['pairs']}, in-band flips {rep['band_flips']}")


_CACHE = {}


def _inputs(name):
    if name not in _CACHE:
        _CACHE.clear()
        say(f"[{name}] generating inputs")
        _CACHE[name] = synth.make_inputs(name)
    return _CACHE[name]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny_prefill", "decode_64k", "prefill_32k", "ragged_prefill", "decode_1m"])
def test_full_workload(name):
    inp = _inputs(name)
    wl = inp.wl
    rows = None
    if not wl.is_decode and wl.total_q > 4096:
        rows = synth.sample_rows(wl, n_per_seq=160)
    rep, _ = check_case(inp, rows=rows, label=name)
    say(f"[{name}] near-tie pairs {rep['near_tie']} of {rep['pairs']}, in-band flips {rep['band_flips']}")
