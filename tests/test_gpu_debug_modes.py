"""The library's two debugging aids, on the GPU through the C ABI:

* the wait word of the query-tile prefill: every hand-off wait between the
  waves of a workgroup is bounded, and a wait that reaches its bound is
  counted in the workspace.  MSA_DEBUG_SPIN_LIMIT lowers the bound from the
  host, so the waits give up while every kernel still ends normally; the word
  must then be non-zero, and zero again (with a correct result) once the
  bound is back to its default;
* the debug-validate mode (MSA_DEBUG_VALIDATE): entry points copy cu_seqlens
  and ids to the host and reject a broken contract before launching
  anything.
"""
import os

import numpy as np
import pytest

import oracle
from block_sparse_gqa_amd import synth
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture
def env(monkeypatch):
    return monkeypatch


def test_wait_word_reports_given_up_waits(env):
    from block_sparse_gqa_amd import device, msa
    inp = synth.custom((2048,), (2048,), 8, 2, 128, 64, 64, 4, seed=21, name="wait_word")
    dp = device.upload(inp)
    ids = device.index_topk(dp)
    op = msa.MSA_OP_SPARSE_ATTN_PREFILL_TILES
    ws = device.workspace(dp, op)
    env.setenv("MSA_DEBUG_SPIN_LIMIT", "0")    # a wait gives up at once if its stage is not ready
    device.sparse_attention_tiles(dp, ids, ws=ws)
    torch.cuda.synchronize()
    gave_up = device.wait_word(dp, op, ws)
    print(f"[wait_word] waits given up with a bound of 0 polls: {gave_up}", flush=True)
    assert gave_up > 0
    env.delenv("MSA_DEBUG_SPIN_LIMIT")
    out, lse = device.sparse_attention_tiles(dp, ids, ws=ws)
    torch.cuda.synchronize()
    assert device.wait_word(dp, op, ws) == 0   # cleared by the call, and no wait reached the default bound
    rows = np.arange(0, inp.wl.total_q, 7, dtype=np.int64)
    ref_out, ref_lse = oracle.sparse_attention(inp, ids.cpu().numpy()[rows], rows)
    parity.assert_close(out.float().cpu().numpy()[rows], ref_out, "wait word: O after the bound is restored")
    parity.assert_close(lse.cpu().numpy()[rows], ref_lse, "wait word: LSE after the bound is restored")


def test_debug_validate_rejects_broken_contracts(env):
    from block_sparse_gqa_amd import device, msa
    env.setenv("MSA_DEBUG_VALIDATE", "1")
    inp = synth.custom((300, 129), (300, 129), 8, 2, 128, 64, 64, 3, seed=5, name="validate")
    dp = device.upload(inp)
    ids = device.index_topk(dp)                 # a valid call passes the checks
    out, lse = device.sparse_attention(dp, ids)
    torch.cuda.synchronize()
    host_ids = ids.cpu().numpy()
    ref_out, _ = oracle.sparse_attention(inp, host_ids)
    parity.assert_close(out.float().cpu().numpy(), ref_out, "debug-validate mode: O")
    # an ineligible block (block 4 at position 10) and a duplicate id are rejected before any launch
    for row, slot, val in ((10, 0, 4), (200, 1, int(host_ids[200, 0, 0]))):
        bad = host_ids.copy()
        bad[row, 0, slot] = val
        sentinel = torch.full_like(out, 7.0)
        with pytest.raises(msa.MsaError) as e:
            device.sparse_attention(dp, torch.from_numpy(bad).to(ids.device), out=sentinel, lse=lse)
        assert e.value.status == msa.MSA_ERROR_INVALID_VALUE
        torch.cuda.synchronize()
        assert bool((sentinel == 7.0).all())     # nothing ran
        with pytest.raises(msa.MsaError) as e:
            device.sparse_attention_backward(dp, torch.from_numpy(bad).to(ids.device), out, lse, out)
        assert e.value.status == msa.MSA_ERROR_INVALID_VALUE
    # cu_seqlens that do not end at total_k are rejected by the index call
    keep = torch.tensor([0, 300, 428], dtype=torch.int32, device=ids.device)
    dp.problem.cu_seqlens_k = keep.data_ptr()
    with pytest.raises(msa.MsaError) as e:
        device.index_topk(dp)
    assert e.value.status == msa.MSA_ERROR_INVALID_VALUE
    # without the mode the library does not look (the contract is the caller's)
    env.delenv("MSA_DEBUG_VALIDATE")
    assert os.environ.get("MSA_DEBUG_VALIDATE") is None
