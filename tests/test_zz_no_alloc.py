"""The allocation-free decode entry point (msa_sparse_attn_decode_noalloc),
through the C ABI: on two calls in a row, the second with a smaller input, its
output and LSE equal those of msa_sparse_attn_decode (which takes a caller
workspace and runs the same kernels) bit for bit, and both meet the oracle's
tolerance; a problem whose partials exceed the fixed scratch is rejected."""
import numpy as np
import pytest

import oracle
from block_sparse_gqa_amd import synth
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def one_call(inp, label):
    from block_sparse_gqa_amd import device, msa
    dp = device.upload(inp)
    ids = device.index_topk(dp)
    out_ws, lse_ws = device.sparse_attention(dp, ids)            # the existing entry point, with a workspace
    out_na, lse_na = device.alloc_out(dp)
    out_na.fill_(7.0)
    lse_na.fill_(7.0)
    msa.msa_sparse_attn_decode_noalloc(dp.problem, dp.q, dp.k, dp.v, ids, inp.wl.scale, out_na, lse_na)
    torch.cuda.synchronize()
    assert torch.equal(out_na, out_ws), f"{label}: O differs from msa_sparse_attn_decode"
    assert torch.equal(lse_na, lse_ws), f"{label}: LSE differs from msa_sparse_attn_decode"
    host_ids = ids.cpu().numpy()
    ref_out, ref_lse = oracle.sparse_attention(inp, host_ids)
    parity.assert_close(out_na.float().cpu().numpy(), ref_out, f"{label}: O against the oracle")
    parity.assert_close(lse_na.cpu().numpy(), ref_lse, f"{label}: LSE against the oracle")
    print(f"[no_alloc] {label}: identical to the workspace entry point", flush=True)


def test_noalloc_decode_matches_workspace_entry_point():
    # first call: 3 sequences up to 5000 tokens, k = 16; second call: smaller (2 shorter sequences, k = 4)
    one_call(synth.custom((1, 1, 1), (5000, 3000, 700), 32, 8, 128, 64, 64, 16, seed=31, name="noalloc_a"), "first")
    one_call(synth.custom((1, 1), (900, 130), 16, 4, 128, 64, 64, 4, seed=32, name="noalloc_b"), "second, smaller")


def test_noalloc_decode_rejects_what_does_not_fit():
    from block_sparse_gqa_amd import msa
    # 512 one-query sequences of 64 heads: one split each, 512 * 64 * (128 + 1) * 4 bytes of partials > 16 MiB
    n = 512
    cu_q = torch.arange(n + 1, dtype=torch.int32, device="cuda")
    cu_k = cu_q * 64
    p = msa.make_problem(cu_q, cu_k, 1, 64, n, n * 64, 64, 8, 128, 64, 64, 4)
    assert msa.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_DECODE, p) > msa.MSA_DECODE_NOALLOC_SCRATCH_BYTES
    dummy = torch.empty(1, dtype=torch.int32, device="cuda")
    with pytest.raises(msa.MsaError) as e:
        msa.msa_sparse_attn_decode_noalloc(p, dummy, dummy, dummy, dummy, 0.088, dummy)
    assert e.value.status == msa.MSA_ERROR_WORKSPACE
