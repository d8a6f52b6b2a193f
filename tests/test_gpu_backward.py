"""GPU parity of the sparse-branch backward (prefill, selection fixed):
dq, dk, dv from msa_sparse_attn_prefill_backward against the oracle's plain
chain rule, on the GPU's own ids, out and lse.

The backward is handed the forward's output `out` in bf16 and forms
D = dO . out from it, as its contract says; the oracle gets the same `out`
(its given-output path, pinned to float64 autograd), so both compute the same
function of the same inputs.

Tolerance: the forward's, |gpu - ref| <= 2e-3 + 1e-2 |ref| per element.  The
kernels take P and dS into the dV, dK and dQ products as a bf16 head plus a
bf16 tail (relative rounding about 2^-17), keep dq per (row, selected slot)
as a bf16 partial, accumulate in float32 and round dq, dk, dv to bf16
(2^-9 relative), which the relative term covers.  The distance to the exact
gradient (D from the unrounded output) is printed beside it: it adds the
effect of out's bf16 rounding on D.
"""
import dataclasses
import sys
import zlib

import numpy as np
import pytest

import oracle
from block_sparse_gqa_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from tests import parity


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_grad(got, ref, name):
    """The forward's elementwise tolerance; returns the largest error over its bound."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    parity.assert_close(got, ref, name)
    return float((np.abs(got - ref) / (parity.ATOL + parity.RTOL * np.abs(ref))).max())


CASES = [
    # name, seqlens_q, seqlens_k, H, h, d, d_idx, B, k
    ("bwd_d128_B64_G4", (700, 129), (700, 129), 16, 4, 128, 64, 64, 4),
    ("bwd_d64_B128_G3", (900,), (900,), 6, 2, 64, 32, 128, 3),
    ("bwd_G6_ragged", (300, 77, 257), (300, 77, 257), 48, 8, 128, 64, 128, 2),
    ("bwd_G1", (400,), (400,), 4, 4, 64, 32, 64, 3),
    ("bwd_G16", (333,), (333,), 16, 1, 128, 64, 64, 2),
    ("bwd_dense", (257,), (257,), 8, 2, 128, 64, 64, 8),
    ("bwd_chunked", (100, 37), (300, 400), 8, 4, 128, 64, 64, 3),
    # 16 groups x 1094 key blocks = 17504 (group, block) keys: more than the
    # LDS histogram of the counting pass holds, so the global-atomic count runs
    ("bwd_many_keys", (64, 64), (40000, 30000), 16, 16, 64, 32, 64, 3),
    # empty sequences inside the batch (no rows, no key blocks)
    ("bwd_empty_seqs", (0, 300, 0, 129), (0, 300, 0, 129), 8, 2, 128, 64, 64, 3),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(case):
    from block_sparse_gqa_amd import device
    name, sq, sk, H, h, d, di, B, k = case
    seed = zlib.crc32(name.encode()) % 1000
    inp = synth.custom(sq, sk, H, h, d, di, B, k, seed=seed, name=name)
    rng = np.random.default_rng(seed)
    dout_bits = synth.f32_to_bf16_bits(rng.standard_normal(inp.q.shape).astype(np.float32))
    dp = device.upload(inp)
    ids, out, lse = device.forward(dp)
    dout = device.to_device_bf16(dout_bits)
    say(f"[{name}] gpu backward")
    dq, dk, dv = device.sparse_attention_backward(dp, ids, out, lse, dout)
    torch.cuda.synchronize()
    gids = ids.cpu().numpy()
    out_bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    rq, rk, rv = oracle.sparse_attention_backward(inp, gids, dout_bits, out=out_bits)
    got = [t.float().cpu().numpy() for t in (dq, dk, dv)]
    e = [check_grad(g_, r, f"{name} {n}") for g_, r, n in zip(got, (rq, rk, rv), ("dq", "dk", "dv"))]
    say(f"[{name}] largest |err| / (2e-3 + 1e-2 |ref|): dq {e[0]:.3g}, dk {e[1]:.3g}, dv {e[2]:.3g}")
    exact = oracle.sparse_attention_backward(inp, gids, dout_bits)
    x = [float(np.abs(g_ - r).max() / np.abs(r).max()) for g_, r in zip(got, exact)]
    say(f"[{name}] against the exact gradient, max |err| / max |ref|: dq {x[0]:.3g}, dk {x[1]:.3g}, dv {x[2]:.3g}")


@pytest.mark.timeout(300)
def test_backward_untouched_tokens_zero():
    """Tokens no row selected get exactly zero dk and dv."""
    from block_sparse_gqa_amd import device
    inp = synth.custom((640,), (640,), 8, 2, 128, 64, 64, 1, seed=3, name="bwd_k1")
    dp = device.upload(inp)
    ids, out, lse = device.forward(dp)
    dout = device.to_device_bf16(synth.f32_to_bf16_bits(np.ones(inp.q.shape, np.float32)))
    _, dk, dv = device.sparse_attention_backward(dp, ids, out, lse, dout)
    torch.cuda.synchronize()
    gids, dkh, dvh = ids.cpu().numpy(), dk.float().cpu().numpy(), dv.float().cpu().numpy()
    for g in range(2):
        used = np.zeros(640, bool)
        for r in range(640):
            j = gids[r, g, 0]
            used[j * 64:min(j * 64 + 64, r + 1)] = True
        assert not dkh[~used, g].any() and not dvh[~used, g].any()


@pytest.mark.timeout(300)
@pytest.mark.parametrize("rows", [777, 5000])
def test_backward_repeat(rows):
    """dq, dk and dv are bitwise reproducible: dq's per-slot partials sum in slot order, and the selection lists that
    dk and dv sum over are sorted after the count pass's atomics hand out the places (5000 rows spread the count
    over several workgroups, whose atomics interleave differently from run to run)."""
    from block_sparse_gqa_amd import device
    inp = synth.custom((rows,), (rows,), 16, 4, 128, 64, 64, 5, seed=5, name=f"bwd_repeat_{rows}")
    dp = device.upload(inp)
    ids, out, lse = device.forward(dp)
    dout = device.to_device_bf16(synth.f32_to_bf16_bits(
        np.random.default_rng(2).standard_normal(inp.q.shape).astype(np.float32)))
    runs = [device.sparse_attention_backward(dp, ids, out, lse, dout) for _ in range(3)]
    torch.cuda.synchronize()
    for other in runs[1:]:
        for x, y, n in zip(runs[0], other, ("dq", "dk", "dv")):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16)), n


@pytest.mark.timeout(600)
def test_backward_full_size_sampled_rows():
    """The 32768-token prefill's backward at full size (the measured configuration, run in two row chunks), checked
    on sampled rows: dq of a row depends only on its own selection, K and V, so the oracle computes it for a
    contiguous range of rows posed as a prefill of those rows against every key before them."""
    from block_sparse_gqa_amd import device
    inp = synth.make_inputs("prefill_32k")
    wl = inp.wl
    rng = np.random.default_rng(11)
    dout_bits = synth.f32_to_bf16_bits(rng.standard_normal(inp.q.shape).astype(np.float32))
    dp = device.upload(inp)
    ids, out, lse = device.forward(dp)
    dout = device.to_device_bf16(dout_bits)
    say("[bwd_full] gpu backward, 32768 tokens")
    dq, dk, dv = device.sparse_attention_backward(dp, ids, out, lse, dout)
    dq2, dk2, dv2 = device.sparse_attention_backward(dp, ids, out, lse, dout)
    torch.cuda.synchronize()
    # bitwise reproducible, row chunks and float32 dk/dv accumulators included
    for x, y, nm in ((dq, dq2, "dq"), (dk, dk2, "dk"), (dv, dv2, "dv")):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16)), nm
    del dq2, dk2, dv2, dk, dv
    gids = ids.cpu().numpy()
    out_bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    dq_gpu = dq.float().cpu().numpy()
    del dp, ids, out, lse, dout, dq
    torch.cuda.empty_cache()
    n = wl.total_q
    for a, b in ((0, 192), (13000, 13192), (n - 192, n)):
        sub_wl = dataclasses.replace(wl, name=f"rows_{a}_{b}", seqlens_q=(b - a,), seqlens_k=(b,))
        sub = synth.Inputs(sub_wl, np.array([0, b - a], np.int32), np.array([0, b], np.int32), inp.q[a:b],
                           inp.k[:b], inp.v[:b], inp.q_idx[a:b], inp.k_idx[:b])
        rq, _, _ = oracle.sparse_attention_backward(sub, gids[a:b], dout_bits[a:b], out=out_bits[a:b])
        e = check_grad(dq_gpu[a:b], rq, f"bwd_full dq rows {a}..{b}")
        say(f"[bwd_full] rows {a}..{b}: largest |err| / (2e-3 + 1e-2 |ref|) of dq {e:.3g}")
