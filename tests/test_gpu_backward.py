"""GPU parity of the sparse-branch backward (prefill, selection fixed):
dq, dk, dv from msa_sparse_attn_prefill_backward against the oracle's plain
chain rule, on the GPU's own ids, out and lse.

Tolerance.  The kernels take P and dS in bf16 for the dV, dK and dQ products
(relative rounding 2^-9) and round dq, dk, dv to bf16; each output element is
a sum of such terms with both signs, so its error is bounded by a small
multiple of 2^-9 times the sum of the magnitudes of its terms, which is at
most the tensor's largest magnitude times a few.  The check is
|gpu - ref| <= 1e-2 |ref| + 1e-2 max|ref| per tensor, with the largest
observed ratio printed for each case.
"""
import sys
import zlib

import numpy as np
import pytest

import oracle
from block_sparse_gqa_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

RTOL = 1e-2
ATOL_REL = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_grad(got, ref, name):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.abs(ref).max()
    bound = RTOL * np.abs(ref) + ATOL_REL * scale
    err = np.abs(got - ref)
    bad = err > bound
    assert not bad.any(), (f"{name}: {int(bad.sum())} elements off; worst at {np.unravel_index(np.argmax(err - bound), err.shape)}"
                           f" err {err.max():.3g} vs max|ref| {scale:.3g}")
    return float(err.max() / max(scale, 1e-30))


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
    rq, rk, rv = oracle.sparse_attention_backward(inp, gids, dout_bits)
    e = [check_grad(t.float().cpu().numpy(), r, f"{name} {n}")
         for t, r, n in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv"))]
    say(f"[{name}] max |err| / max |ref|: dq {e[0]:.3g}, dk {e[1]:.3g}, dv {e[2]:.3g}")


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
def test_backward_repeat():
    """dq is bitwise reproducible (per-slot partials summed in slot order); dk
    and dv follow the run-time order of the selection lists and agree to
    rounding."""
    from block_sparse_gqa_amd import device
    inp = synth.custom((777,), (777,), 16, 4, 128, 64, 64, 5, seed=5, name="bwd_repeat")
    dp = device.upload(inp)
    ids, out, lse = device.forward(dp)
    dout = device.to_device_bf16(synth.f32_to_bf16_bits(
        np.random.default_rng(2).standard_normal(inp.q.shape).astype(np.float32)))
    a = device.sparse_attention_backward(dp, ids, out, lse, dout)
    b = device.sparse_attention_backward(dp, ids, out, lse, dout)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    for x, y, n in ((a[1], b[1], "dk"), (a[2], b[2], "dv")):
        xf, yf = x.float(), y.float()
        assert float((xf - yf).abs().max()) <= 2 ** -7 * float(xf.abs().max()), n
